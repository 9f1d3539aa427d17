"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs (small and ragged sizes with the full oracle; the bench's full
sizes on sampled outputs and size-independent properties)."""
import json
import os

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


def run_fwd(ops, Xb, Wb, mask):
    X, W, mk = G.to_dev_bf16(Xb), G.to_dev_bf16(Wb), G.to_dev_u8(mask)
    out = ops.rowpar_pcr_fwd(X, W, mk)
    torch.cuda.synchronize()
    return out


def synced_identical(out_bits: np.ndarray, mask: np.ndarray) -> bool:
    S = mask != 0
    return all(np.array_equal(out_bits[t][:, S], out_bits[0][:, S]) for t in range(1, out_bits.shape[0]))


# ---------------------------------------------------------------------------
# standalone reduce
# ---------------------------------------------------------------------------

RED_CASES = [
    (1, 5, 64, "random", 0.5),
    (2, 7, 776, "prefix", 0.5),
    (3, 33, 136, "strided", 0.25),
    (4, 64, 768, "random", 0.75),
    (8, 257, 4096, "random", 0.5),
    (8, 1, 4096, "random", 0.5),
    (8, 32, 4096, "random", 1.0),
    (8, 16, 768, "random", 0.0),
    (8, 7, 776, "strided", 0.5),    # T = 8 out of place: a partial last block of 512 vectors
    (8, 3, 264, "prefix", 0.5),     # one partial block
    (13, 9, 200, "random", 0.5),
    (20, 17, 520, "strided", 0.5),  # runtime rank count: groups of 8 + 8 + 4
    (16, 33, 264, "random", 0.5),
]


@pytest.mark.parametrize("T,M,H,kind,p", RED_CASES)
@pytest.mark.parametrize("inplace", [False, True])
def test_reduce_f32(ops, T, M, H, kind, p, inplace):
    _announce(f"reduce f32 T={T} M={M} H={H} {kind} p={p} inplace={inplace}")
    Y = synth.make_reduce_input(T, M, H, seed=T + M)
    mask = synth.make_mask(H, p, kind, seed=1)
    Yd = torch.from_numpy(Y).to(G.dev())
    out = ops.partial_channel_reduce(Yd, G.to_dev_u8(mask), inplace=inplace)
    got = out.cpu().numpy()
    # bitwise against the float32 emulation of ascending-rank summation
    want = G.f32_sequential_reduce(Y, mask)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    G.check_f32(got, oracle.partial_channel_reduce(Y, mask), "reduce f32")
    S = mask != 0
    if inplace:  # local channels untouched
        assert np.array_equal(got[:, :, ~S].view(np.uint32), Y[:, :, ~S].view(np.uint32))
    # a second run gives the same bits
    out2 = ops.partial_channel_reduce(torch.from_numpy(Y).to(G.dev()), G.to_dev_u8(mask))
    assert np.array_equal(out2.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_reduce_f32_inplace_leaves_local_sentinels(ops):
    T, M, H = 8, 64, 4096
    _announce("reduce f32 sentinel")
    Y = synth.make_reduce_input(T, M, H, seed=5)
    mask = synth.make_mask(H, 0.5, "random", seed=5)
    S = mask != 0
    Y[:, :, ~S] = np.float32(-1234.5)  # sentinel in every local channel
    Yd = torch.from_numpy(Y).to(G.dev())
    ops.partial_channel_reduce(Yd, G.to_dev_u8(mask), inplace=True)
    got = Yd.cpu().numpy()
    assert np.all(got[:, :, ~S] == np.float32(-1234.5))


@pytest.mark.parametrize("T,M,H,kind,p", RED_CASES[:6] + RED_CASES[8:10] + RED_CASES[-3:])
@pytest.mark.parametrize("inplace", [False, True])
def test_reduce_bf16(ops, T, M, H, kind, p, inplace):
    _announce(f"reduce bf16 T={T} M={M} H={H} {kind} p={p} inplace={inplace}")
    Yb = synth.make_reduce_input(T, M, H, seed=T * 7 + M, dtype="bf16")
    mask = synth.make_mask(H, p, kind, seed=2)
    Yd = G.to_dev_bf16(Yb)
    out = ops.partial_channel_reduce(Yd, G.to_dev_u8(mask), inplace=inplace)
    got_bits = G.bf16_bits(out)
    Yf = oracle.bf16_to_f64(Yb).astype(np.float32)
    want_bits = Yb.copy()
    S = mask != 0
    seq = G.f32_sequential_reduce(Yf, mask)
    want_bits[:, :, S] = G.f32_to_bf16_bits_rne(seq[:, :, S])
    assert np.array_equal(got_bits, want_bits)
    G.check_bf16(oracle.bf16_to_f64(got_bits), oracle.partial_channel_reduce(Yb, mask), S[None, None, :], "reduce bf16")


def test_reduce_empty(ops):
    Y = torch.empty((8, 0, 64), dtype=torch.float32, device=G.dev())
    mask = G.to_dev_u8(np.ones(64, np.uint8))
    assert ops.partial_channel_reduce(Y, mask).shape == (8, 0, 64)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def test_golden_fixture(ops):
    _announce("golden tiny integer case")
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_integer_case.json")
    d = json.load(open(path))
    X = np.array(d["X_bf16_bits"], dtype=np.uint16)
    W = np.array(d["W_bf16_bits"], dtype=np.uint16)
    dZ = np.array(d["dZ_bf16_bits"], dtype=np.uint16)
    mask = np.array(d["mask"], dtype=np.uint8)
    out = run_fwd(ops, X, W, mask)
    assert np.array_equal(G.from_dev_bf16(out), np.array(d["Z"]))
    dX, dW = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dX), np.array(d["dX"]))
    assert np.array_equal(G.from_dev_bf16(dW), np.array(d["dW"]))


INT_CASES = [
    (2, 256, 1536, 768, "prefix", 0.5),  # the tiny 130M-shaped layer
    (3, 300, 200, 776, "random", 0.5),   # ragged: M, Kr and H off every tile
    (8, 129, 96, 264, "strided", 0.5),
    (8, 32, 1376, 512, "random", 0.5),   # decode path, M = 32
    (8, 1, 1376, 4096, "random", 0.5),   # decode path, M = 1
    (5, 7, 72, 136, "random", 0.25),     # decode path, ragged
    (1, 70, 64, 128, "random", 0.5),     # T = 1
    (20, 5, 64, 136, "random", 0.5),     # M <= 32, T = 20
    (3, 17, 96, 72, "random", 0.5),      # decode, H not a multiple of 16
    (16, 23, 40, 264, "strided", 0.5),   # decode, T = 16, the last size before the split
    (16, 24, 40, 264, "strided", 0.5),   # split from 24 tokens with more than 8 ranks
    (1, 3, 64, 136, "random", 0.5),      # decode, T = 1 (every workgroup arrives last)
    (13, 17, 40, 264, "strided", 0.5),   # decode, T = 13, two token blocks
    (8, 1, 1376, 4096, "prefix", 0.5),   # decode: all-synced and all-local channel blocks
    (8, 32, 256, 1024, "prefix", 0.25),  # decode, M = 32, block-uniform mask
    (4, 5, 64, 200, "prefix", 0.0),      # decode, nothing synced (no exchange), ragged block
    (4, 9, 64, 200, "prefix", 1.0),      # decode, everything synced, ragged block
    (13, 20, 40, 392, "prefix", 0.5),    # decode, T = 13, one mixed block between uniform ones
    (8, 33, 1376, 512, "random", 0.5),   # split from 33 tokens at T = 8 (two contraction slices)
    (8, 100, 96, 264, "prefix", 0.5),    # split, 128 x 64 tiles
    (13, 70, 40, 136, "random", 0.5),    # split, T = 13
    (4, 192, 64, 200, "strided", 0.5),   # split, ragged channel block
    (1, 192, 64, 200, "strided", 0.5),   # one rank: decode in 32-token chunks, the largest chunked M
]


@pytest.mark.parametrize("T,M,Kr,H,kind,p", INT_CASES)
def test_fwd_integer_inputs_bitexact(ops, T, M, Kr, H, kind, p):
    """Small-integer inputs: every product and partial sum is exact, so the GPU
    must reproduce the oracle bit for bit whatever its summation order."""
    _announce(f"fwd int T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=3, lo=-1, hi=1, x_zero_frac=0.8)
    mask = synth.make_mask(H, p, kind, seed=3)
    want = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(want).max() <= 256  # exact in bf16
    out = run_fwd(ops, X, W, mask)
    assert np.array_equal(G.from_dev_bf16(out), want)


@pytest.mark.parametrize("T,M,Kr,H", [(8, 300, 64, 776), (8, 8, 1376, 4096), (4, 64, 8, 64)])
def test_fwd_rank_tag_routing(ops, T, M, Kr, H):
    """One-hot rows, W_t = 2**t * s_c: local outputs name their rank, synced
    outputs equal s_c * (2**T - 1); bit-exact."""
    _announce(f"fwd rank tags T={T} M={M} Kr={Kr} H={H}")
    X, W, s = synth.make_rank_tag_inputs(T, M, Kr, H, seed=1)
    mask = synth.make_mask(H, 0.5, "random", seed=9)
    got = G.from_dev_bf16(run_fwd(ops, X, W, mask))
    for t in range(T):
        want = np.where(mask != 0, s * (2 ** T - 1), s * 2.0 ** t)
        assert np.array_equal(got[t], np.broadcast_to(want, (M, H))), t
    assert np.array_equal(got, oracle.rowpar_pcr_fwd(X, W, mask))


RAND_CASES = [
    (2, 256, 1536, 768, "prefix", 0.5),
    (2, 256, 1536, 768, "prefix", 0.0),
    (2, 256, 1536, 768, "prefix", 1.0),
    (3, 300, 200, 776, "random", 0.5),
    (8, 512, 384, 768, "random", 0.25),   # 130M down-proj shape, fewer tokens
    (8, 512, 96, 768, "random", 0.75),    # 130M out-proj shape, fewer tokens
    (8, 200, 704, 2048, "strided", 0.5),  # 1.1B down-proj shape, fewer tokens
    (8, 1, 1376, 4096, "random", 0.5),    # decode
    (8, 8, 1376, 4096, "random", 0.5),
    (8, 32, 1376, 4096, "random", 0.5),
    (8, 32, 512, 4096, "random", 0.5),
    (8, 64, 1376, 4096, "random", 0.5),   # two decode chunks
    (8, 192, 512, 4096, "random", 0.5),   # six decode chunks
]


@pytest.mark.parametrize("T,M,Kr,H,kind,p", RAND_CASES)
def test_fwd_random_parity(ops, T, M, Kr, H, kind, p):
    _announce(f"fwd random T={T} M={M} Kr={Kr} H={H} {kind} p={p}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=M + Kr)
    mask = synth.make_mask(H, p, kind, seed=4)
    out = run_fwd(ops, X, W, mask)
    bits = G.bf16_bits(out)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    rep = G.check_bf16(oracle.bf16_to_f64(bits), ref, (mask != 0)[None, None, :], "fwd")
    print(rep)
    assert synced_identical(bits, mask)
    out2 = run_fwd(ops, X, W, mask)
    assert np.array_equal(G.bf16_bits(out2), bits), "not deterministic"


def test_fwd_empty(ops):
    X = torch.empty((8, 0, 64), dtype=torch.bfloat16, device=G.dev())
    W = torch.zeros((8, 64, 64), dtype=torch.bfloat16, device=G.dev())
    mask = G.to_dev_u8(np.ones(64, np.uint8))
    assert ops.rowpar_pcr_fwd(X, W, mask).shape == (8, 0, 64)


def test_decode_repeated_calls(ops):
    """Back-to-back decode-shaped calls with different masks, token counts and
    inputs each match the oracle exactly (no state carried between calls)."""
    T, Kr, H = 8, 256, 1024
    for i, M in enumerate((32, 8, 1, 32)):
        _announce(f"decode repeated call {i} M={M}")
        X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=i, lo=-1, hi=1, x_zero_frac=0.5)
        mask = synth.make_mask(H, 0.5, "random", seed=i)
        got = G.from_dev_bf16(run_fwd(ops, X, W, mask))
        assert np.array_equal(got, oracle.rowpar_pcr_fwd(X, W, mask))


def test_decode_shared_workspace(ops):
    """One workspace serves back-to-back decode calls of different sizes: the
    per-block arrival counters at its head are zero again after every call,
    and the partials region may hold anything on entry."""
    T, Kr = 8, 512
    ws = torch.zeros(ops.fwd_workspace_bytes(T, 32, Kr, 9000), dtype=torch.uint8, device=G.dev())
    cnt_bytes = 2048  # the arrival counters: a fixed region, whatever H
    ws[cnt_bytes:].fill_(0x7F)  # partials: arbitrary bytes
    # H grows from call to call as well: the counter region does not move
    for i, (M, H) in enumerate(((32, 1032), (8, 1032), (1, 2056), (32, 4096), (17, 9000), (5, 264))):
        _announce(f"decode shared workspace call {i} M={M} H={H}")
        X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=20 + i, lo=-1, hi=1, x_zero_frac=0.5)
        mask = synth.make_mask(H, 0.5, "random", seed=20 + i)
        out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(G.from_dev_bf16(out), oracle.rowpar_pcr_fwd(X, W, mask))
        assert int(ws[:cnt_bytes].count_nonzero()) == 0, "arrival counters not returned to zero"


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

BWD_CASES = [
    (2, 256, 1536, 768, "prefix", 0.5),
    (3, 300, 200, 776, "random", 0.5),
    (8, 130, 96, 264, "random", 0.25),
    (8, 512, 384, 768, "random", 0.5),
    (1, 65, 64, 64, "random", 0.5),
    (8, 8, 1376, 512, "random", 0.5),
]


@pytest.mark.parametrize("T,M,Kr,H,kind,p", BWD_CASES)
def test_bwd_random_parity(ops, T, M, Kr, H, kind, p):
    _announce(f"bwd random T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=11)
    dZ = synth.make_grad(T, M, H, seed=11)
    mask = synth.make_mask(H, p, kind, seed=11)
    dXd, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    ax, aw = G.bwd_g_allowance(dZ, X, W, mask)
    G.check_bf16(G.from_dev_bf16(dXd), rdX, None, "dX", extra=ax)
    G.check_bf16(G.from_dev_bf16(dWd), rdW, (mask != 0)[None, None, :], "dW", extra=aw)
    dX2, dW2 = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    assert np.array_equal(G.bf16_bits(dX2), G.bf16_bits(dXd))
    assert np.array_equal(G.bf16_bits(dW2), G.bf16_bits(dWd))


@pytest.mark.parametrize("T,M,Kr,H", [(2, 256, 1536, 768), (3, 70, 40, 136), (8, 64, 64, 128)])
def test_bwd_integer_inputs_bitexact(ops, T, M, Kr, H):
    _announce(f"bwd int T={T} M={M} Kr={Kr} H={H}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=5, lo=-1, hi=1, x_zero_frac=0.8)
    rng = np.random.default_rng(5)
    dZ = rng.integers(-1, 2, size=(T, M, H)) * (rng.random((T, M, H)) < 0.2)
    dZ = synth.f32_to_bf16_bits(dZ.astype(np.float32))
    mask = synth.make_mask(H, 0.5, "random", seed=5)
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert max(np.abs(rdX).max(), np.abs(rdW).max()) <= 256
    dXd, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dXd), rdX)
    assert np.array_equal(G.from_dev_bf16(dWd), rdW)


def test_bwd_only_dw_and_empty(ops):
    T, M, Kr, H = 2, 64, 64, 64
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=1, lo=-1, hi=1)
    dZ = X[:, :, :H].copy()
    mask = synth.make_mask(H, 0.5, "random", seed=1)
    dXd, dWd = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), need_dx=False)
    torch.cuda.synchronize()
    assert dXd is None
    assert np.array_equal(G.from_dev_bf16(dWd), oracle.pcr_bwd(dZ, X, W, mask)[1])
    # no tokens: dW is zero
    e = torch.empty((T, 0, H), dtype=torch.bfloat16, device=G.dev())
    ex = torch.empty((T, 0, Kr), dtype=torch.bfloat16, device=G.dev())
    dW0 = torch.full((T, Kr, H), 7.0, dtype=torch.bfloat16, device=G.dev())
    ops.pcr_bwd(e, ex, G.to_dev_bf16(W), G.to_dev_u8(mask), dW=dW0)
    torch.cuda.synchronize()
    assert float(dW0.float().abs().max()) == 0.0
