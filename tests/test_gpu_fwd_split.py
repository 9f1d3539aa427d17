"""The forward for token counts between decode and full tiles: one workgroup
per (rank, channel block, token block) -- tiles of 128 x 64, 128 x 128 or
256 x 256, and with few tiles and long contractions one per slice of the
contraction -- writing that rank's fp32 product tile, then a streaming pass
that forms the partial channel-reduce.  Integer inputs bit for bit against the
oracle (blocks with and without synced channels, ragged token, channel and
contraction counts, up to 13 ranks, all three tile sizes, the column-parallel
layer with no mask), Gaussian inputs at the Llama2-7B down-projection with 512
tokens (256 x 256 tiles), one workspace shared by calls of every path, and
run-to-run bits."""
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


def _mask(H, kind, p, seed):
    if kind == "blocks":  # channels 0..255 synced (two 128-channel blocks), the rest local
        m = np.zeros(H, dtype=np.uint8)
        m[:256] = 1
        return m
    return synth.make_mask(H, p, kind, seed=seed)


# (T, M, Kr, H): M from 33 (one partial token block) to 1900; H = 776 leaves
# a partial channel block (6 x 128 + 8, 3 x 256 + 8).  The first seven run
# 128 x 64 tiles, (4, 130, 1376, 512) and (3, 40, 1048, 264) with each rank's
# contraction in two slices (22 chunks, the last a half one: 11 + 11; 17
# chunks: 9 + 8); (8, 1000, 136, 1032) 576 tiles of 128 x 128 (1032 = 8 x 128
# + 8); the last two 256 x 256 tiles: 192 of them with a partial token block
# (1800 = 7 x 256 + 8), and 256 with partial channel and token blocks.
SHAPES = [(2, 33, 40, 776), (3, 100, 136, 776), (8, 257, 96, 1024), (8, 1000, 64, 776), (13, 64, 72, 520),
          (4, 130, 1376, 512), (3, 40, 1048, 264), (8, 1000, 136, 1032), (8, 1800, 136, 768),
          (8, 1900, 200, 776)]
MASKS = [("random", 0.5), ("prefix", 0.5), ("strided", 0.5), ("random", 0.0), ("random", 1.0), ("blocks", 0.0)]


@pytest.mark.parametrize("T,M,Kr,H", SHAPES)
@pytest.mark.parametrize("kind,p", MASKS)
def test_fwd_split_bitwise(ops, T, M, Kr, H, kind, p):
    _announce(f"fwd split T={T} M={M} Kr={Kr} H={H} {kind} p={p}")
    zf = 0.4 if T * Kr <= 1200 else 0.97
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=T * 1000 + M, lo=-1, hi=1, x_zero_frac=zf)
    mask = _mask(H, kind, p, seed=M + H)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())  # every element must be written
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)


@pytest.mark.parametrize("T,M,Kr,H", [(8, 257, 96, 1024), (3, 1000, 136, 776)])
def test_colpar_split_bitwise(ops, T, M, Kr, H):
    _announce(f"colpar split T={T} M={M} Kr={Kr} H={H}")
    A, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=T + M, lo=-1, hi=1, x_zero_frac=0.4)
    ref = oracle.colpar_fwd(A, W)
    assert np.abs(ref).max() <= 256
    U = ops.colpar_fwd(G.to_dev_bf16(A), G.to_dev_bf16(W))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(U), ref)


def test_fwd_split_gaussian_7b_m512(ops):
    T, M, Kr, H = 8, 512, 1376, 4096
    _announce(f"fwd split gaussian T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=21)
    mask = synth.make_mask(H, 0.5, "random", seed=21)
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    got = G.from_dev_bf16(out)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    G.check_bf16(got, ref, (mask != 0)[None, None, :], "fwd split 7B M=512")
    s = np.flatnonzero(mask)
    assert all(np.array_equal(got[0][:, s], got[t][:, s]) for t in range(1, T))


def test_fwd_split_shared_workspace(ops):
    """One workspace, zeroed once, serves split, decode and chunked calls of
    growing H in turn; the arrival counters are zero after every call."""
    T, Kr = 8, 96
    calls = [(100, 1032), (32, 1032), (1000, 776), (8, 4096), (257, 4096), (150, 9000), (33, 264)]
    need = max(ops.fwd_workspace_bytes(T, M, Kr, H) for M, H in calls)
    ws = torch.zeros(need, dtype=torch.uint8, device=G.dev())
    ws[2048:].fill_(0x7F)  # partials: arbitrary bytes
    for i, (M, H) in enumerate(calls):
        _announce(f"fwd shared workspace call {i} M={M} H={H}")
        X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=40 + i, lo=-1, hi=1, x_zero_frac=0.5)
        mask = synth.make_mask(H, 0.5, "random", seed=40 + i)
        out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(G.from_dev_bf16(out), oracle.rowpar_pcr_fwd(X, W, mask))
        assert int(ws[:2048].count_nonzero()) == 0, "arrival counters not returned to zero"


def test_fwd_split_run_to_run(ops):
    T, M, Kr, H = 8, 384, 1376, 4096
    _announce(f"fwd split repeat T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=22)
    mask = synth.make_mask(H, 0.5, "random", seed=22)
    args = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    a = ops.rowpar_pcr_fwd(*args)
    b = ops.rowpar_pcr_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fwd_chunked_decode_single_rank(ops):
    """With one rank, 33..192 tokens still run the decode kernel 32 at a time."""
    T, M, Kr, H = 1, 150, 512, 1032
    _announce(f"fwd chunked decode T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=31, lo=-1, hi=1, x_zero_frac=0.8)
    mask = synth.make_mask(H, 0.5, "random", seed=31)
    assert ops.fwd_workspace_bytes(T, M, Kr, H) == ops.fwd_workspace_bytes(T, 32, Kr, H)
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), oracle.rowpar_pcr_fwd(X, W, mask))


def test_noalloc_split_fallback(ops):
    """The allocation-free forward declines the split path when its fp32
    products exceed the library's 16 MiB scratch and runs the chunked decode
    kernel instead: integer inputs bit for bit against the oracle, Gaussian
    ones within the bar, synced channels identical across ranks."""
    T, M, Kr, H = 8, 160, 512, 4096
    assert ops.fwd_workspace_bytes(T, M, Kr, H) > (16 << 20)
    _announce(f"noalloc split fallback T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=32, lo=-1, hi=1, x_zero_frac=0.8)
    mask = synth.make_mask(H, 0.5, "random", seed=32)
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())
    ops.rowpar_pcr_fwd_noalloc(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), oracle.rowpar_pcr_fwd(X, W, mask))
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=33)
    ops.rowpar_pcr_fwd_noalloc(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    got = G.from_dev_bf16(out)
    G.check_bf16(got, oracle.rowpar_pcr_fwd(X, W, mask), (mask != 0)[None, None, :], "noalloc split fallback")
    s = np.flatnonzero(mask)
    assert all(np.array_equal(got[0][:, s], got[t][:, s]) for t in range(1, T))


def test_noalloc_fewer_slices(ops):
    """The Llama2-7B down-projection at 64 tokens cuts each rank's contraction
    in two slices (2 x 8.4 MB of fp32 products, over the 16 MiB scratch); the
    allocation-free forward then runs whole contractions (8.4 MB).  Integer
    inputs bit for bit against the oracle on both entry points; Gaussian ones
    within the bar on both, and the two agree to the bf16 rounding of
    different fp32 summation orders."""
    T, M, Kr, H = 8, 64, 1376, 4096
    assert ops.fwd_workspace_bytes(T, M, Kr, H) == 2048 + 2 * T * M * H * 4 > (16 << 20)
    _announce(f"noalloc fewer slices T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=34, lo=-1, hi=1, x_zero_frac=0.97)
    mask = synth.make_mask(H, 0.5, "random", seed=34)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    args = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    out_n = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())
    ops.rowpar_pcr_fwd_noalloc(*args, out_n)
    out_w = ops.rowpar_pcr_fwd(*args)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out_n), ref)
    assert np.array_equal(G.from_dev_bf16(out_w), ref)
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=35)
    args = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    ops.rowpar_pcr_fwd_noalloc(*args, out_n)
    out_w = ops.rowpar_pcr_fwd(*args)
    torch.cuda.synchronize()
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    cls = (mask != 0)[None, None, :]
    got_n, got_w = G.from_dev_bf16(out_n), G.from_dev_bf16(out_w)
    G.check_bf16(got_n, ref, cls, "noalloc, whole contractions")
    G.check_bf16(got_w, ref, cls, "two contraction slices")
    s = np.flatnonzero(mask)
    for got in (got_n, got_w):
        assert all(np.array_equal(got[0][:, s], got[t][:, s]) for t in range(1, T))


# Whole contractions with H a multiple of 64: 64-channel groups with no synced
# channel go from the product kernel straight to out in bf16 and the reduce
# pass skips them.  (T, M, Kr, H): 128 x 64 tiles (one group per wave),
# 128 x 128 tiles (512 workgroups) and 256 x 256 tiles (two groups per wave,
# ragged tokens).  Masks: a prefix whose end falls inside a group, alternating
# 64-channel groups, a sparse random set (some groups wholly local, some
# not), nothing synced (every group goes straight to out) and everything.
LOCAL_SHAPES = [(8, 300, 136, 1024), (8, 1000, 136, 1024), (8, 1800, 136, 768)]


def _local_mask(H, kind, seed):
    if kind == "prefix47":
        return synth.make_mask(H, 0.47, "prefix", seed=seed)
    if kind == "alt64":
        m = np.zeros(H, dtype=np.uint8)
        for g in range(0, H, 128):
            m[g:g + 64] = 1
        return m
    if kind == "sparse":
        return synth.make_mask(H, 0.02, "random", seed=seed)
    return synth.make_mask(H, 0.0 if kind == "none" else 1.0, "prefix", seed=seed)


@pytest.mark.parametrize("T,M,Kr,H", LOCAL_SHAPES)
@pytest.mark.parametrize("kind", ["prefix47", "alt64", "sparse", "none", "all"])
def test_split_local_groups_bitwise(ops, T, M, Kr, H, kind):
    assert H % 64 == 0 and ops.fwd_workspace_bytes(T, M, Kr, H) == 2048 + T * M * H * 4  # whole contractions
    _announce(f"split local groups T={T} M={M} Kr={Kr} H={H} {kind}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=M + H, lo=-1, hi=1, x_zero_frac=0.4)
    mask = _local_mask(H, kind, seed=M)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())  # every element must be written
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)
