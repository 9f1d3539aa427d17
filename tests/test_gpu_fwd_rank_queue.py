"""The forward kernel that holds the earlier ranks' tiles in registers (128x64
tiles, T <= 4, or T <= 8 with at most two 64-wide chunks of contraction per
rank) and the standard kernel beside it: integer inputs, bit for bit against
the oracle, with ragged token counts, channel counts and contractions and
every kind of sync set; and Gaussian inputs at the 130M down-projection's
shape with four ranks, under the bf16 bars."""
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


# (T, Kr): held in registers for T <= 4 and for (5..8, Kr <= 128); the
# standard kernel for (5, 136) and (8, 136).  M = 3600 and H = 776 leave a
# partial token tile and a partial channel tile (776 = 6 x 128 + 8); 399
# fused tiles of 128 x 64 are more than the split forward takes for any of
# these walks, and fewer than 512 of 128 x 128, so the 128 x 64 path runs.
RANKS_KR = [(2, 40), (3, 136), (4, 384), (4, 1376), (5, 128), (8, 96), (8, 8), (5, 136), (8, 136)]
MASKS = [("random", 0.5), ("prefix", 0.5), ("strided", 0.5), ("random", 0.0), ("random", 1.0), ("random", 0.1)]


@pytest.mark.parametrize("T,Kr", RANKS_KR)
@pytest.mark.parametrize("kind,p", MASKS)
def test_fwd_rank_queue_bitwise(ops, T, Kr, kind, p):
    M, H = 3600, 776
    _announce(f"fwd rank queue T={T} M={M} Kr={Kr} H={H} {kind} p={p}")
    zf = 0.4 if T * Kr <= 1200 else 0.97
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=T * 100 + Kr, lo=-1, hi=1, x_zero_frac=zf)
    mask = synth.make_mask(H, p, kind, seed=T + Kr)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())  # every element must be written
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)


def test_fwd_rank_queue_gaussian_130m_t4(ops):
    T, M, Kr, H = 4, 8192, 384, 768
    _announce(f"fwd rank queue gaussian T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=11)
    mask = synth.make_mask(H, 0.5, "random", seed=11)
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    got = G.from_dev_bf16(out)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    G.check_bf16(got, ref, (mask != 0)[None, None, :], "fwd rank queue 130M T=4")
    s = np.flatnonzero(mask)
    assert all(np.array_equal(got[0][:, s], got[t][:, s]) for t in range(1, T))


def test_fwd_rank_queue_run_to_run(ops):
    T, M, Kr, H = 8, 8192, 96, 768
    _announce(f"fwd rank queue repeat T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=12)
    mask = synth.make_mask(H, 0.5, "random", seed=12)
    args = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    a = ops.rowpar_pcr_fwd(*args)
    b = ops.rowpar_pcr_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# Eight-rank queue tiles held to three workgroups per CU, the form taken when
# 513 to 768 tiles of 128 x 64 fit one round at three per CU but not at two:
# 585 tiles with every tile in the queue (Kr = 96), 658 with the two-launch
# split of the mask's channel groups (Kr = 384, six chunks) and 768 at the
# window's edge.
THREE_PER_CU = [(8, 4100, 96, 1032), (6, 6000, 384, 776), (8, 8192, 256, 768)]


@pytest.mark.parametrize("T,M,Kr,H", THREE_PER_CU)
@pytest.mark.parametrize("kind,p", [("random", 0.5), ("prefix", 0.5), ("strided", 0.5), ("random", 0.1)])
def test_fwd_rank_queue_three_per_cu_bitwise(ops, T, M, Kr, H, kind, p):
    tiles = -(-H // 128) * -(-M // 64)
    assert 512 < tiles <= 768
    _announce(f"fwd rank queue 3/CU T={T} M={M} Kr={Kr} H={H} {kind} p={p}")
    zf = 0.4 if T * Kr <= 1200 else 0.97
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=T * 100 + Kr + 1, lo=-1, hi=1, x_zero_frac=zf)
    mask = synth.make_mask(H, p, kind, seed=T + Kr + 1)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)
