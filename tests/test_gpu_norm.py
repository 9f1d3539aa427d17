"""GPU parity of the per-rank residual update + RMS normalisation (the step
after the partial channel-reduce) through the C ABI against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _normal(shape, seed, scale=1.0, loc=0.0):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((loc + scale * rng.standard_normal(shape)).astype(np.float32))


CASES = [
    # T, M, H, eps
    (8, 64, 4096, 1e-5),   # Llama2-7B hidden size
    (8, 33, 2048, 1e-5),   # TinyLlama-1.1B
    (8, 17, 768, 1e-5),    # 130M
    (3, 7, 776, 1e-6),     # H not a multiple of 2048
    (2, 5, 8192, 1e-5),    # the largest H (four vectors per thread)
    (1, 3, 8, 0.5),        # one vector per row, large eps
]


@pytest.mark.parametrize("T,M,H,eps", CASES)
def test_residual_rmsnorm_parity(ops, T, M, H, eps):
    _announce(f"residual+rmsnorm T={T} M={M} H={H}")
    Z = _normal((T, M, H), 1)
    R = _normal((T, M, H), 2, 2.0)
    g = _normal((H,), 3, 0.1, 1.0)
    Rd, Zd, gd = G.to_dev_bf16(R), G.to_dev_bf16(Z), G.to_dev_bf16(g)
    Rn, N = ops.residual_rmsnorm(Zd, Rd, gd, eps)
    Rn2, N2 = ops.residual_rmsnorm(Zd, Rd, gd, eps)
    torch.cuda.synchronize()
    assert torch.equal(N.view(torch.int16), N2.view(torch.int16)), "not deterministic"
    rRn, rN = oracle.residual_rmsnorm(Z, R, g, eps)
    print(G.check_bf16(G.from_dev_bf16(Rn), rRn, None, "Rn"))
    print(G.check_bf16(G.from_dev_bf16(N), rN, None, "N"))
    # the residual update is one bf16 rounding of the exact sum
    want = synth.f32_to_bf16_bits(rRn.astype(np.float32))
    assert np.array_equal(G.bf16_bits(Rn), want)


def test_residual_rmsnorm_in_place_and_zero_rows(ops):
    """In place (Rout == R) gives the same bits as out of place; a row whose
    update is exactly zero normalises to zero (eps > 0), not NaN."""
    T, M, H = 4, 9, 1024
    _announce(f"residual+rmsnorm in place T={T} M={M} H={H}")
    Z = _normal((T, M, H), 4)
    R = _normal((T, M, H), 5)
    Z[1, 3] = 0
    R[1, 3] = 0
    g = _normal((H,), 6, 0.1, 1.0)
    Rd, Zd, gd = G.to_dev_bf16(R), G.to_dev_bf16(Z), G.to_dev_bf16(g)
    Rn, N = ops.residual_rmsnorm(Zd, Rd, gd, 1e-5)
    Rd2 = G.to_dev_bf16(R)
    Rn2, N2 = ops.residual_rmsnorm(Zd, Rd2, gd, 1e-5, inplace=True)
    torch.cuda.synchronize()
    assert Rn2.data_ptr() == Rd2.data_ptr()
    assert torch.equal(Rn.view(torch.int16), Rd2.view(torch.int16))
    assert torch.equal(N.view(torch.int16), N2.view(torch.int16))
    n = G.from_dev_bf16(N)
    assert np.all(np.isfinite(n)) and np.all(n[1, 3] == 0.0)


def test_residual_rmsnorm_after_partial_reduce_7b_rows(ops):
    """The step as it follows the layer: Z = the partial channel-reduce of the
    7B down-projection's per-rank products (M = 512 tokens); sampled rows of
    (Rn, N) against the oracle applied to the GPU's Z."""
    T, M, Kr, H = 8, 512, 1376, 4096
    _announce("residual+rmsnorm after the 7B down-proj layer")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=21)
    mask = synth.make_mask(H, 0.5, "random", seed=21)
    Z = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    R = _normal((T, M, H), 22)
    g = _normal((H,), 23, 0.1, 1.0)
    Rn, N = ops.residual_rmsnorm(Z, G.to_dev_bf16(R), G.to_dev_bf16(g), 1e-5)
    torch.cuda.synchronize()
    Zb = G.bf16_bits(Z)
    rows = np.random.default_rng(24).choice(T * M, size=64, replace=False)
    ts, ms = rows // M, rows % M
    rRn, rN = oracle.residual_rmsnorm(Zb[ts, ms][None], R[ts, ms][None], g, 1e-5)
    G.check_bf16(G.from_dev_bf16(Rn)[ts, ms][None], rRn, None, "Rn rows")
    G.check_bf16(G.from_dev_bf16(N)[ts, ms][None], rN, None, "N rows")
