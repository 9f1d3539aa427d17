"""GPU parity on both sides of every kernel-selection threshold.

The library picks a kernel by problem size: the weight-streaming decode
kernel up to 32 tokens, the split forward while the fused tiles would be too
few for their walk over the ranks, then fused tiles of 128x64, 128x128 or
256x256 by how many tiles the output has (256x256 from 160 of them in the
forward, from 256 in the backward's products).  Each case here sits one
token or eight channels below or above such a switch, so an off-by-one in
the selection or in a kernel's edge handling shows up as a wrong element.
Integer-valued inputs keep every product and sum exact in bf16 and fp32, so
the comparison with the oracle is bitwise."""
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


def _int_grad(T, M, H, seed, nz=0.3):
    rng = np.random.default_rng(seed)
    dZ = rng.integers(-1, 2, size=(T, M, H)) * (rng.random((T, M, H)) < nz)
    return synth.f32_to_bf16_bits(dZ.astype(np.float32))


def _tiles(rows, cols, tr, tc, batch=1):
    return -(-rows // tr) * -(-cols // tc) * batch


# Forward, T = 2 ranks, Kr = 40, H = 1024 channels (8 tiles of 128, 4 of 256):
#   M <= 32 decode;  33 <= M <= 1024 the split forward (at most 128 fused
#   tiles of 128x64 for a walk of two chunks);
#   M = 1025 the first 128x64-tile call;
#   M = 8064 -> 504 tiles of 128x128 (still 128x64), M = 8065 -> 512 (128x128);
#   M = 9984 -> 156 tiles of 256x256 (still 128x128), M = 9985 -> 160 (256x256).
FWD_M = [32, 33, 192, 1024, 1025, 8064, 8065, 9984, 9985]


# With a random S every 256-channel group of the mask is mixed, so past the
# split range the register-queue kernel takes every tile (a one-chunk
# contraction); with S = the first 512 channels every group is uniform and
# the tiled kernels take them all.  Both sides of each switch run both ways.
@pytest.mark.parametrize("kind", ["random", "prefix"])
@pytest.mark.parametrize("M", FWD_M)
def test_fwd_across_kernel_switch(ops, M, kind):
    T, Kr, H = 2, 40, 1024
    assert _tiles(H, 1024, 128, 64) == 128 and _tiles(H, 1025, 128, 64) == 136
    assert _tiles(8064, H, 128, 128) == 504 and _tiles(8065, H, 128, 128) == 512
    assert _tiles(9984, H, 256, 256) == 156 and _tiles(9985, H, 256, 256) == 160
    _announce(f"dispatch fwd T={T} M={M} Kr={Kr} H={H} {kind}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=M, lo=-1, hi=1, x_zero_frac=0.4)
    mask = synth.make_mask(H, 0.5, kind, seed=M + 1)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)


# dX = G W^T, T = 4, Kr = 520 (3 row tiles of 256): M = 5376 -> 21 token tiles,
# 252 big tiles (128x128 kernel); M = 5377 -> 22, 264 big tiles (256x256).
@pytest.mark.parametrize("M", [5376, 5377])
def test_dx_across_kernel_switch(ops, M):
    T, Kr, H = 4, 520, 72
    assert _tiles(M, Kr, 256, 256, T) == (252 if M == 5376 else 264)
    _announce(f"dispatch dX T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=M, lo=-1, hi=1, x_zero_frac=0.5)
    dZ = _int_grad(T, M, H, M)
    mask = synth.make_mask(H, 0.5, "random", seed=M + 2)
    rdX, _ = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdX).max() <= 256
    dXd, _ = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dw=False)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dXd), rdX)


# dX with 256 big tiles (T = 8, M = 8192: 32 token tiles): Kr = 248 fills
# under a 256-row tile, so the 128x128 kernel runs; Kr = 256 the 256x256 one.
@pytest.mark.parametrize("Kr", [248, 256])
def test_dx_short_contraction_switch(ops, Kr):
    T, M, H = 8, 8192, 64
    assert _tiles(M, Kr, 256, 256, T) == 256
    _announce(f"dispatch dX short Kr T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=Kr, lo=-1, hi=1, x_zero_frac=0.5)
    dZ = _int_grad(T, M, H, Kr)
    mask = synth.make_mask(H, 0.5, "random", seed=Kr + 4)
    rdX, _ = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdX).max() <= 256
    dXd, _ = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dw=False)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dXd), rdX)


# dW = X^T G, T = 4, Kr = 264 (2 row tiles of 256): H = 7936 -> 31 channel
# tiles, 248 big tiles (128x128 kernel); H = 7944 -> 32, 256 (256x256).
@pytest.mark.parametrize("H", [7936, 7944])
def test_dw_across_kernel_switch(ops, H):
    T, M, Kr = 4, 40, 264
    assert _tiles(Kr, H, 256, 256, T) == (248 if H == 7936 else 256)
    _announce(f"dispatch dW T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=H, lo=-1, hi=1, x_zero_frac=0.5)
    dZ = _int_grad(T, M, H, H)
    mask = synth.make_mask(H, 0.5, "random", seed=H + 3)
    _, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdW).max() <= 256
    _, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dx=False)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dWd), rdW)


# dW with too few tiles to fill the chip runs as a split of the token range:
# fp32 pieces summed in piece order.  T = 2, Kr = 96, H = 264: six 128x128
# tiles, M = 4000 tokens (62.5 chunks of 64) -> seven pieces of nine chunks,
# the last one ragged.
def test_dw_split_token_range_bitexact(ops):
    T, M, Kr, H = 2, 4000, 96, 264
    _announce(f"dW split T={T} M={M} Kr={Kr} H={H}")
    base = -(-(T * M * H * 2) // 256) * 256
    assert ops.bwd_workspace_bytes(T, M, Kr, H) - base - 256 == 7 * T * Kr * H * 4  # G, tile classes, pieces
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=77, lo=-1, hi=1, x_zero_frac=0.8)
    dZ = _int_grad(T, M, H, 77, nz=0.2)
    mask = synth.make_mask(H, 0.5, "random", seed=77)
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdW).max() <= 256 and np.abs(rdX).max() <= 256
    args = (G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    dXd, dWd = ops.pcr_bwd(*args)
    dXe, dWe = ops.pcr_bwd(*args)  # a second call: same bits
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dWd), rdW)
    assert np.array_equal(G.from_dev_bf16(dXd), rdX)
    assert torch.equal(dWd.view(torch.int16), dWe.view(torch.int16))


# The 130M model's out-projection (Kr = 96, H = 768, M = 8192 tokens): 48 tiles
# of dW, six pieces.  Gaussian inputs against the oracle on sampled rows of dW.
def test_dw_split_130m_out_proj(ops):
    T, M, Kr, H = 8, 8192, 96, 768
    _announce(f"dW split 130M out-proj T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=5)
    dZ = synth.make_grad(T, M, H, seed=5)
    mask = synth.make_mask(H, 0.5, "random", seed=5)
    _, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dx=False)
    torch.cuda.synchronize()
    got = G.from_dev_bf16(dWd)
    _, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    G.check_bf16(got, rdW, (mask != 0)[None, None, :], "dW split 130M out-proj")


# The same with 256x256 tiles: T = 4, Kr = 264, H = 2056 have 72 of them;
# three pieces (216 workgroups) fill a round best.  M = 1600 tokens is 25
# chunks: pieces of 9, 9 and 7.
def test_dw_split_big_tiles_bitexact(ops):
    T, M, Kr, H = 4, 1600, 264, 2056
    _announce(f"dW split, 256x256 tiles T={T} M={M} Kr={Kr} H={H}")
    base = -(-(T * M * H * 2) // 256) * 256
    assert ops.bwd_workspace_bytes(T, M, Kr, H) - base - 256 == 3 * T * Kr * H * 4
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=78, lo=-1, hi=1, x_zero_frac=0.8)
    dZ = _int_grad(T, M, H, 78, nz=0.2)
    mask = synth.make_mask(H, 0.5, "random", seed=78)
    _, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdW).max() <= 256
    _, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dx=False)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dWd), rdW)
