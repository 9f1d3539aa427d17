"""GPU parity of the partial channel-reduce with the residual update and RMS
normalisation fused into its epilogue (caat_partial_channel_reduce_residual_rmsnorm).

* Bit for bit against the two-kernel chain it replaces (the bf16 partial
  channel-reduce, then the residual update + norm), which the other GPU tests
  tie to the oracle.
* Against the oracle composed from its two pinned functions (the exact
  partial reduce of Y, then the residual update + norm), under the bf16 bar
  plus the exact effect of the one documented extra rounding: the synced
  channels of Z are bf16 (as the chain stores them), so Rout may differ by
  |bf16(Z) - Z| and N by that times |gamma| / rms(Rout row).
"""
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


def _inputs(T, M, H, kind, p, seed):
    Y = _normal((T, M, H), seed)
    R = _normal((T, M, H), seed + 1, 2.0)
    g = _normal((H,), seed + 2, 0.1, 1.0)
    mask = synth.make_mask(H, p, kind, seed=seed)
    return Y, R, g, mask


CASES = [
    # T, M, H, mask kind, p, eps
    (8, 64, 4096, "random", 0.5, 1e-5),   # Llama2-7B hidden size, Y kept in registers
    (8, 33, 2048, "strided", 0.5, 1e-5),  # TinyLlama-1.1B
    (8, 17, 768, "random", 0.25, 1e-5),   # 130M
    (4, 9, 4096, "prefix", 0.5, 1e-5),
    (2, 5, 8192, "random", 0.5, 1e-5),    # the largest H: ranks in groups, Y read twice
    (3, 7, 776, "random", 0.75, 1e-6),    # odd rank count, H off every vector block
    (13, 6, 1024, "random", 0.5, 1e-5),   # more ranks than one group
    (20, 5, 520, "strided", 0.5, 1e-5),   # runtime rank count: sums in groups of 8 + 8 + 4
    (8, 6, 8192, "random", 0.5, 1e-5),    # eight ranks at the largest H: the runtime-T path
    (1, 3, 8, "random", 1.0, 0.5),        # one rank: the reduce is the identity
    (8, 20, 4096, "random", 0.0, 1e-5),   # nothing synced
    (8, 20, 4096, "random", 1.0, 1e-5),   # everything synced
]


def _chain(ops, Yd, mk, Rd, gd, eps):
    Z = ops.partial_channel_reduce(Yd, mk)
    return ops.residual_rmsnorm(Z, Rd, gd, eps)


@pytest.mark.parametrize("T,M,H,kind,p,eps", CASES)
def test_fused_equals_chain_and_oracle(ops, T, M, H, kind, p, eps):
    _announce(f"reduce+residual+rmsnorm T={T} M={M} H={H} {kind} p={p}")
    Y, R, g, mask = _inputs(T, M, H, kind, p, seed=T * 1000 + H)
    Yd, Rd, gd, mk = G.to_dev_bf16(Y), G.to_dev_bf16(R), G.to_dev_bf16(g), G.to_dev_u8(mask)
    Rn, N = ops.reduce_residual_rmsnorm(Yd, mk, Rd, gd, eps)
    cRn, cN = _chain(ops, Yd, mk, Rd, gd, eps)
    Rn2, N2 = ops.reduce_residual_rmsnorm(Yd, mk, Rd, gd, eps)
    torch.cuda.synchronize()
    assert torch.equal(Rn.view(torch.int16), cRn.view(torch.int16)), "Rout differs from the two-kernel chain"
    assert torch.equal(N.view(torch.int16), cN.view(torch.int16)), "N differs from the two-kernel chain"
    assert torch.equal(N.view(torch.int16), N2.view(torch.int16)), "not deterministic"
    # against the oracle: exact Z, exact residual, exact norm
    Z = oracle.partial_channel_reduce(Y, mask)
    rRn, rN = oracle.residual_rmsnorm(Z, R, g, eps)
    S = (mask != 0)[None, None, :]
    Zb = oracle.bf16_to_f64(G.f32_to_bf16_bits_rne(Z.astype(np.float32)))
    dz = np.where(S, np.abs(Zb - Z), 0.0)
    rms_row = np.sqrt(np.mean(rRn * rRn, axis=-1, keepdims=True) + eps)
    G.check_bf16(G.from_dev_bf16(Rn), rRn, S, "Rout", extra=dz)
    G.check_bf16(G.from_dev_bf16(N), rN, S, "N", extra=dz * np.abs(oracle.bf16_to_f64(g)) / rms_row)


def test_fused_in_place(ops):
    T, M, H = 8, 12, 4096
    _announce(f"reduce+residual+rmsnorm in place T={T} M={M} H={H}")
    Y, R, g, mask = _inputs(T, M, H, "random", 0.5, seed=77)
    Yd, gd, mk = G.to_dev_bf16(Y), G.to_dev_bf16(g), G.to_dev_u8(mask)
    Rn, N = ops.reduce_residual_rmsnorm(Yd, mk, G.to_dev_bf16(R), gd, 1e-5)
    Rd = G.to_dev_bf16(R)
    Rn2, N2 = ops.reduce_residual_rmsnorm(Yd, mk, Rd, gd, 1e-5, inplace=True)
    torch.cuda.synchronize()
    assert Rn2.data_ptr() == Rd.data_ptr()
    assert torch.equal(Rn.view(torch.int16), Rd.view(torch.int16))
    assert torch.equal(N.view(torch.int16), N2.view(torch.int16))


def test_fused_7b_full_size(ops):
    """Llama2-7B shape (T=8, M=16384, H=4096, random half of the channels
    synced): the whole output bit for bit against the two-kernel chain, and
    sampled token rows (every rank) against the oracle."""
    T, M, H = 8, 16384, 4096
    _announce("reduce+residual+rmsnorm at the 7B shape")
    g = torch.Generator(device=G.dev()).manual_seed(5)
    Yd = torch.randn((T, M, H), generator=g, device=G.dev()).to(torch.bfloat16)
    Rd = (2.0 * torch.randn((T, M, H), generator=g, device=G.dev())).to(torch.bfloat16)
    gd = (1.0 + 0.1 * torch.randn((H,), generator=g, device=G.dev())).to(torch.bfloat16)
    mask = synth.make_mask(H, 0.5, "random", seed=5)
    mk = G.to_dev_u8(mask)
    Rn, N = ops.reduce_residual_rmsnorm(Yd, mk, Rd, gd, 1e-5)
    cRn, cN = _chain(ops, Yd, mk, Rd, gd, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(Rn.view(torch.int16), cRn.view(torch.int16))
    assert torch.equal(N.view(torch.int16), cN.view(torch.int16))
    del cRn, cN
    rows = torch.from_numpy(np.sort(np.random.default_rng(6).choice(M, size=16, replace=False))).to(G.dev())
    Y = G.bf16_bits(Yd[:, rows])
    R = G.bf16_bits(Rd[:, rows])
    gb = G.bf16_bits(gd)
    Z = oracle.partial_channel_reduce(Y, mask)
    rRn, rN = oracle.residual_rmsnorm(Z, R, gb, 1e-5)
    S = (mask != 0)[None, None, :]
    Zb = oracle.bf16_to_f64(G.f32_to_bf16_bits_rne(Z.astype(np.float32)))
    dz = np.where(S, np.abs(Zb - Z), 0.0)
    rms_row = np.sqrt(np.mean(rRn * rRn, axis=-1, keepdims=True) + 1e-5)
    G.check_bf16(G.from_dev_bf16(Rn[:, rows]), rRn, S, "Rout rows", extra=dz)
    G.check_bf16(G.from_dev_bf16(N[:, rows]), rN, S, "N rows", extra=dz * np.abs(oracle.bf16_to_f64(gb)) / rms_row)
