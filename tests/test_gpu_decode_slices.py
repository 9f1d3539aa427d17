"""Decode-sized calls with few ranks or channel blocks: each rank's contraction
is cut into ks slices of whole 32-row stages, one workgroup each, and the last
of a channel block's T * ks workgroups adds each rank's slices in slice order,
then the synced channels over the ranks in ascending order.  Integer inputs
bit for bit against the oracle (8, 4 and 2 slices; one to four ranks; ragged
contraction stages, channel blocks and token counts; blocks with and without
synced channels, which now all go through the exchange; one rank in 32-token
chunks), Gaussian inputs within the bar at the Llama2-7B down-projection's
width, one workspace shared with unsliced calls, the allocation-free entry
point, and the column-parallel layer (no mask: whole contractions)."""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G
from tests.sweep_cases import decode_slices, forward_path

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


def _need(T, M, Kr, H):
    ks = decode_slices(T, Kr, H)
    return 2048 + -(-ks * T * min(M, 32) * H * 4 // 256) * 256


# (T, M, Kr, H) -> slices: (1, 3, 4104, 520) 8 (129 stages, the last of 8
# rows; a partial channel block), (1, 17, 4096, 256) 8 (two 16-token MFMA
# blocks), (2, 9, 2056, 776) 4, (2, 15, 5504, 264) 4 (the last token count
# before the split forward), (3, 7, 2000, 264) 2 (six partials per block),
# (4, 1, 1024, 1032) 2 (16 stages each), (1, 70, 1032, 264) 2 in chunks of
# 32 + 32 + 6 tokens.
SHAPES = [(1, 3, 4104, 520), (1, 17, 4096, 256), (2, 9, 2056, 776), (2, 15, 5504, 264), (3, 7, 2000, 264),
          (4, 1, 1024, 1032), (1, 70, 1032, 264)]
KINDS = [("random", 0.5), ("prefix", 0.5), ("strided", 0.5), ("random", 0.0), ("random", 1.0), ("blocks", 0.0)]


@pytest.mark.parametrize("T,M,Kr,H", SHAPES)
@pytest.mark.parametrize("kind,p", KINDS)
def test_decode_slices_bitwise(ops, T, M, Kr, H, kind, p):
    assert decode_slices(T, Kr, H) > 1 and forward_path(T, M, Kr, H).endswith("_sliced")
    assert ops.fwd_workspace_bytes(T, M, Kr, H) == _need(T, M, Kr, H)
    _announce(f"decode slices T={T} M={M} Kr={Kr} H={H} {kind} p={p}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=T * 100 + M, lo=-1, hi=1, x_zero_frac=0.97)
    mask = _mask(H, kind, p, seed=M + H)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())  # every element must be written
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)


@pytest.mark.parametrize("T,M,Kr", [(1, 1, 11008), (2, 8, 5504), (4, 15, 2752)])
def test_decode_slices_gaussian(ops, T, M, Kr):
    """The Llama2-7B down-projection's width (H = 4096) with one, two and four
    ranks (8, 4 and 2 slices): within the bar, synced channels identical on
    every rank, and the same bits on a second call."""
    H = 4096
    assert decode_slices(T, Kr, H) == 8 // T
    _announce(f"decode slices gaussian T={T} M={M} Kr={Kr}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=40 + T)
    mask = synth.make_mask(H, 0.5, "random", seed=40 + T)
    args = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    out = ops.rowpar_pcr_fwd(*args)
    again = ops.rowpar_pcr_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    got = G.from_dev_bf16(out)
    G.check_bf16(got, oracle.rowpar_pcr_fwd(X, W, mask), (mask != 0)[None, None, :], f"decode slices T={T}")
    s = np.flatnonzero(mask)
    assert all(np.array_equal(got[0][:, s], got[t][:, s]) for t in range(1, T))


def test_decode_slices_shared_workspace(ops):
    """One workspace serves sliced and whole-contraction decode calls in turn:
    the arrival counters (which now count T * ks arrivals) are zero again after
    every call, and the partials region may hold anything on entry."""
    calls = [(2, 9, 2056, 776), (8, 8, 512, 1032), (1, 3, 4104, 520), (1, 70, 1032, 264), (4, 1, 1024, 1032),
             (8, 1, 512, 1032)]
    ws = torch.zeros(max(ops.fwd_workspace_bytes(*c) for c in calls), dtype=torch.uint8, device=G.dev())
    ws[2048:].fill_(0x7F)
    for i, (T, M, Kr, H) in enumerate(calls):
        _announce(f"decode slices shared workspace call {i} T={T} M={M} Kr={Kr} H={H}")
        X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=50 + i, lo=-1, hi=1, x_zero_frac=0.97)
        mask = synth.make_mask(H, 0.5, "random", seed=50 + i)
        out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(G.from_dev_bf16(out), oracle.rowpar_pcr_fwd(X, W, mask))
        assert int(ws[:2048].count_nonzero()) == 0, "arrival counters not returned to zero"


def test_decode_slices_noalloc(ops):
    """The allocation-free entry point takes the same slices (their partials fit
    its scratch): the same bits as the workspace entry point, twice in a row
    with a smaller second call."""
    for T, M, Kr, H in ((2, 15, 5504, 4096), (2, 3, 2056, 776)):
        _announce(f"decode slices noalloc T={T} M={M} Kr={Kr} H={H}")
        X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=60 + M)
        mask = synth.make_mask(H, 0.5, "random", seed=60 + M)
        args = (G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
        out_n = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())
        ops.rowpar_pcr_fwd_noalloc(*args, out_n)
        out_w = ops.rowpar_pcr_fwd(*args)
        torch.cuda.synchronize()
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))


def test_colpar_decode_whole_contractions(ops):
    """With no mask there is no workspace: the decode kernel keeps whole
    contractions and writes every block directly."""
    T, M, K, N = 2, 8, 5504, 264
    _announce(f"colpar decode T={T} M={M} K={K} N={N}")
    A, W = synth.make_integer_fwd_inputs(T, M, K, N, seed=70, lo=-1, hi=1, x_zero_frac=0.97)
    ref = oracle.colpar_fwd(A, W)
    assert np.abs(ref).max() <= 256
    got = ops.colpar_fwd(G.to_dev_bf16(A), G.to_dev_bf16(W))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(got), ref)
