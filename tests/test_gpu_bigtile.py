"""GPU parity of the 256x256-tile (eight-wave) GEMM paths on ragged shapes.

The small parity cases run the 128x128 tiles; these shapes are large enough
(at least 512 output tiles) to take the big-tile kernels, with M, Kr and H
off every tile and chunk boundary.  Integer-valued inputs keep every result
exactly representable, so the comparison with the oracle is bitwise."""
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


def _int_grad(T, M, H, seed):
    rng = np.random.default_rng(seed)
    dZ = rng.integers(-1, 2, size=(T, M, H)) * (rng.random((T, M, H)) < 0.3)
    return synth.f32_to_bf16_bits(dZ.astype(np.float32))


def test_fwd_big_tiles_ragged(ops):
    # 65 token tiles x 9 channel tiles = 585 tiles: the 256x256 forward
    T, M, Kr, H = 2, 16424, 40, 2056
    _announce(f"big-tile fwd T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=31, lo=-1, hi=1, x_zero_frac=0.3)
    mask = synth.make_mask(H, 0.5, "random", seed=31)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)


def test_dx_big_tiles_ragged(ops):
    # dX: 65 token tiles x 3 row tiles x 3 ranks = 585 tiles; the contraction
    # over H = 72 channels ends in a partial chunk
    T, M, Kr, H = 3, 16424, 520, 72
    _announce(f"big-tile dX T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=32, lo=-1, hi=1, x_zero_frac=0.5)
    dZ = _int_grad(T, M, H, 32)
    mask = synth.make_mask(H, 0.5, "random", seed=32)
    rdX, _ = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdX).max() <= 256
    dXd, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dw=False)
    torch.cuda.synchronize()
    assert dWd is None
    assert np.array_equal(G.from_dev_bf16(dXd), rdX)


def test_dw_big_tiles_ragged(ops):
    # dW: 34 channel tiles x 6 row tiles x 3 ranks = 612 tiles; the
    # contraction over M = 200 tokens ends in a partial chunk
    T, M, Kr, H = 3, 200, 1288, 8456
    _announce(f"big-tile dW T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=33, lo=-1, hi=1, x_zero_frac=0.7)
    dZ = _int_grad(T, M, H, 33)
    mask = synth.make_mask(H, 0.5, "random", seed=33)
    _, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdW).max() <= 256
    dXd, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dx=False)
    torch.cuda.synchronize()
    assert dXd is None
    assert np.array_equal(G.from_dev_bf16(dWd), rdW)


@pytest.mark.parametrize("dtype,T,M,H", [("f32", 3, 1024, 4096), ("bf16", 3, 2048, 4096), ("f32", 2, 4096, 4096)])
def test_reduce_interleaved_block_order(ops, dtype, T, M, H):
    """Rank slices a multiple of 16 MiB apart take the interleaved workgroup
    order (two row regions); the result is the same bits as the float32
    emulation of ascending-rank summation."""
    _announce(f"reduce {dtype} interleaved order T={T} M={M} H={H}")
    mask = synth.make_mask(H, 0.5, "random", seed=M)
    S = mask != 0
    if dtype == "f32":
        Y = synth.make_reduce_input(T, M, H, seed=M)
        out = ops.partial_channel_reduce(torch.from_numpy(Y).to(G.dev()), G.to_dev_u8(mask))
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), G.f32_sequential_reduce(Y, mask).view(np.uint32))
    else:
        Yb = synth.make_reduce_input(T, M, H, seed=M, dtype="bf16")
        out = ops.partial_channel_reduce(G.to_dev_bf16(Yb), G.to_dev_u8(mask))
        want = Yb.copy()
        seq = G.f32_sequential_reduce(oracle.bf16_to_f64(Yb).astype(np.float32), mask)
        want[:, :, S] = G.f32_to_bf16_bits_rne(seq[:, :, S])
        assert np.array_equal(G.bf16_bits(out), want)
