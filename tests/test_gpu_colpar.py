"""GPU parity of the column-parallel product on per-rank inputs (the layer
that consumes the partial channel-reduce's output) and of the two-layer chain
-- row-parallel layer with partial channel-reduce, then the column-parallel
product -- through the C ABI against the CPU oracle."""
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


def _int_array(shape, seed, zero_frac):
    rng = np.random.default_rng(seed)
    a = rng.integers(-1, 2, size=shape) * (rng.random(shape) >= zero_frac)
    return synth.f32_to_bf16_bits(a.astype(np.float32))


def _normal(shape, seed, scale):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


RAND_CASES = [
    # T, M, K, N
    (8, 512, 768, 384),   # 130M MLP up-projection shape, fewer tokens
    (3, 300, 200, 136),   # ragged: M, K and N off every tile
    (8, 1, 4096, 1376),   # decode, Llama2-7B up-projection shape
    (8, 32, 4096, 1376),  # decode, two token blocks
    (5, 7, 72, 40),       # decode, ragged
    (8, 64, 4096, 1376),  # decode in two 32-token chunks
    (1, 70, 64, 128),     # T = 1
]


@pytest.mark.parametrize("T,M,K,N", RAND_CASES)
def test_colpar_random_parity(ops, T, M, K, N):
    _announce(f"colpar random T={T} M={M} K={K} N={N}")
    A = _normal((T, M, K), 100 + M, 1.0)
    W = _normal((T, K, N), 200 + K, 0.02)
    dU = _normal((T, M, N), 300 + N, 1.0)
    Ad, Wd, dUd = G.to_dev_bf16(A), G.to_dev_bf16(W), G.to_dev_bf16(dU)
    U = ops.colpar_fwd(Ad, Wd)
    dA, dW = ops.colpar_bwd(dUd, Ad, Wd)
    torch.cuda.synchronize()
    print(G.check_bf16(G.from_dev_bf16(U), oracle.colpar_fwd(A, W), None, "colpar U"))
    rdA, rdW = oracle.colpar_bwd(dU, A, W)
    print(G.check_bf16(G.from_dev_bf16(dA), rdA, None, "colpar dA"))
    print(G.check_bf16(G.from_dev_bf16(dW), rdW, None, "colpar dW"))
    U2 = ops.colpar_fwd(Ad, Wd)
    torch.cuda.synchronize()
    assert torch.equal(U.view(torch.int16), U2.view(torch.int16)), "not deterministic"


INT_CASES = [
    (4, 300, 72, 136),      # tiled path, ragged
    (8, 8, 1376, 520),      # decode
    (8, 100, 1376, 520),    # decode in 32-token chunks
    (2, 16424, 40, 2056),   # 256x256 forward tiles (585 of them)
    (3, 16424, 520, 72),    # 256x256 input-gradient tiles
    (3, 200, 1288, 8456),   # 256x256 weight-gradient tiles
]


@pytest.mark.parametrize("T,M,K,N", INT_CASES)
def test_colpar_integer_inputs_bitexact(ops, T, M, K, N):
    """Small-integer inputs with enough zeros that every sum stays an integer
    below 2^8: any summation order gives the oracle's bits."""
    _announce(f"colpar int T={T} M={M} K={K} N={N}")
    A = _int_array((T, M, K), 1, 0.7)
    W = _int_array((T, K, N), 2, 0.7)
    dU = _int_array((T, M, N), 3, 0.9)
    U_ref = oracle.colpar_fwd(A, W)
    dA_ref, dW_ref = oracle.colpar_bwd(dU, A, W)
    for r in (U_ref, dA_ref, dW_ref):
        assert np.abs(r).max() <= 256
    Ad, Wd, dUd = G.to_dev_bf16(A), G.to_dev_bf16(W), G.to_dev_bf16(dU)
    U = ops.colpar_fwd(Ad, Wd)
    dA, dW = ops.colpar_bwd(dUd, Ad, Wd)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(U), U_ref)
    assert np.array_equal(G.from_dev_bf16(dA), dA_ref)
    assert np.array_equal(G.from_dev_bf16(dW), dW_ref)


@pytest.mark.parametrize("T,M,Kr,H,N,kind,p", [
    (4, 40, 16, 72, 24, "random", 0.5),   # tiled paths
    (8, 8, 32, 264, 40, "random", 0.5),   # decode-shaped forwards
    (3, 50, 24, 136, 16, "prefix", 1.0),  # all synced
    (3, 50, 24, 136, 16, "prefix", 0.0),  # none synced
])
def test_two_layer_chain_bitexact(ops, T, M, Kr, H, N, kind, p):
    """Z = rowpar_pcr_fwd(X, W, S); U = colpar_fwd(Z, W1); backward of
    sum(U * C): (dZ, dW1) = colpar_bwd(C, Z, W1), (dX, dW) = pcr_bwd(dZ, X, W, S).
    Integer inputs keep every intermediate exact in bf16, so the chain must
    equal the oracle's chain bit for bit."""
    _announce(f"two-layer chain T={T} M={M} Kr={Kr} H={H} N={N} {kind} p={p}")
    X = _int_array((T, M, Kr), 11, 0.7)
    W = _int_array((T, Kr, H), 12, 0.7)
    W1 = _int_array((T, H, N), 13, 0.9)
    C = _int_array((T, M, N), 14, 0.5)
    mask = synth.make_mask(H, p, kind, seed=15)
    Z_ref = oracle.rowpar_pcr_fwd(X, W, mask)
    U_ref = oracle.colpar_fwd(Z_ref, W1)
    dZ_ref, dW1_ref = oracle.colpar_bwd(C, Z_ref, W1)
    dX_ref, dW_ref = oracle.pcr_bwd(dZ_ref, X, W, mask)
    for r in (Z_ref, U_ref, dZ_ref, dW1_ref, dX_ref, dW_ref):
        assert np.abs(r).max() <= 256
    Xd, Wd, W1d, Cd, mk = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_bf16(W1), G.to_dev_bf16(C),
                           G.to_dev_u8(mask))
    Z = ops.rowpar_pcr_fwd(Xd, Wd, mk)
    U = ops.colpar_fwd(Z, W1d)
    dZ, dW1 = ops.colpar_bwd(Cd, Z, W1d)
    dX, dW = ops.pcr_bwd(dZ, Xd, Wd, mk)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(Z), Z_ref)
    assert np.array_equal(G.from_dev_bf16(U), U_ref)
    assert np.array_equal(G.from_dev_bf16(dZ), dZ_ref)
    assert np.array_equal(G.from_dev_bf16(dW1), dW1_ref)
    assert np.array_equal(G.from_dev_bf16(dX), dX_ref)
    assert np.array_equal(G.from_dev_bf16(dW), dW_ref)
