"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: whole output rows at sampled positions (at least 64K
elements of every output) against the oracle, plus properties that hold at
any size (synced channels bitwise identical across ranks, run-to-run
determinism, exact float32 summation order of the standalone reduce).  The
complete element-by-element comparison of the Llama2-7B forward is in
test_gpu_fullsize_7b.py."""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

MIN_ELEMS = 65536  # compared elements per output at least


def _sample_rows(rng, n_outer, n_rows, width):
    """(outer, row) pairs whose whole rows of `width` elements make at least
    MIN_ELEMS, always including the first and the last row of the last and
    the first rank (tile edges)."""
    n = max(4, -(-MIN_ELEMS // width))
    o = rng.integers(0, n_outer, size=n)
    r = rng.integers(0, n_rows, size=n)
    o[:2], r[:2] = (0, n_outer - 1), (n_rows - 1, 0)
    return o, r


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _gather(t, *idx):
    """Elements of a device tensor at numpy index arrays, as bf16 bits."""
    ii = tuple(torch.from_numpy(np.asarray(i, dtype=np.int64)).to(t.device) for i in idx)
    return G.bf16_bits(t[ii])


@pytest.mark.parametrize(
    "name,T,M,Kr,H,kind,p",
    [
        ("Llama2-7B down-proj", 8, 16384, 1376, 4096, "random", 0.5),
        ("Llama2-7B down-proj, S = first half", 8, 16384, 1376, 4096, "prefix", 0.5),
        ("Llama2-7B out-proj", 8, 16384, 512, 4096, "random", 0.5),
        ("TinyLlama-1.1B down-proj", 8, 32768, 704, 2048, "strided", 0.5),
        ("TinyLlama-1.1B down-proj, S = first half", 8, 32768, 704, 2048, "prefix", 0.5),
        ("TinyLlama-1.1B out-proj", 8, 32768, 256, 2048, "strided", 0.5),
        ("130M down-proj", 8, 8192, 384, 768, "random", 0.5),
        ("130M out-proj", 8, 8192, 96, 768, "random", 0.5),
        ("130M down-proj, p = 0", 8, 8192, 384, 768, "random", 0.0),
        ("130M down-proj, p = 0.25", 8, 8192, 384, 768, "random", 0.25),
        ("130M out-proj, p = 0.75", 8, 8192, 96, 768, "random", 0.75),
        ("130M out-proj, p = 1", 8, 8192, 96, 768, "random", 1.0),
        ("Llama2-7B down-proj over 2 ranks", 2, 16384, 5504, 4096, "random", 0.5),
        ("Llama2-7B down-proj over 4 ranks", 4, 16384, 2752, 4096, "random", 0.5),
        ("Llama2-7B down-proj over 16 ranks", 16, 16384, 688, 4096, "random", 0.5),
    ],
)
def test_fwd_full_size_sampled(ops, name, T, M, Kr, H, kind, p):
    _announce(f"full-size fwd {name}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=1)
    mask = synth.make_mask(H, p, kind, seed=1)
    Xd, Wd, mk = G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask)
    out = ops.rowpar_pcr_fwd(Xd, Wd, mk)
    out2 = ops.rowpar_pcr_fwd(Xd, Wd, mk)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    S = torch.from_numpy(mask != 0).to(G.dev())
    o16 = out.view(torch.int16)
    for t in range(1, T):
        assert torch.equal(o16[t][:, S], o16[0][:, S]), f"synced channels differ between rank 0 and {t}"
    rng = np.random.default_rng(7)
    ts, ms = _sample_rows(rng, T, M, H)
    ref = oracle.fwd_rows(X, W, mask, ts, ms)
    got = oracle.bf16_to_f64(_gather(out, ts, ms))
    assert got.size >= MIN_ELEMS
    G.check_bf16(got, ref, (mask != 0)[None, :], f"fwd {name}")


@pytest.mark.parametrize(
    "name,T,M,Kr,H,kind,p",
    [
        ("Llama2-7B down-proj", 8, 16384, 1376, 4096, "random", 0.5),
        ("Llama2-7B down-proj, S = first half", 8, 16384, 1376, 4096, "prefix", 0.5),
        ("Llama2-7B out-proj", 8, 16384, 512, 4096, "random", 0.5),
        ("TinyLlama-1.1B down-proj", 8, 32768, 704, 2048, "strided", 0.5),
        ("TinyLlama-1.1B out-proj", 8, 32768, 256, 2048, "prefix", 0.5),
        ("130M down-proj, p = 0.25", 8, 8192, 384, 768, "random", 0.25),
        ("130M out-proj, p = 0.75", 8, 8192, 96, 768, "random", 0.75),
        ("Llama2-7B down-proj over 2 ranks", 2, 16384, 5504, 4096, "random", 0.5),
        ("Llama2-7B down-proj over 16 ranks", 16, 16384, 688, 4096, "random", 0.5),
    ],
)
def test_bwd_full_size_sampled(ops, name, T, M, Kr, H, kind, p):
    _announce(f"full-size bwd {name}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=2)
    dZ = synth.make_grad(T, M, H, seed=2)
    mask = synth.make_mask(H, p, kind, seed=2)
    args = (G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    dX, dW = ops.pcr_bwd(*args)
    dX2, dW2 = ops.pcr_bwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX2.view(torch.int16))
    assert torch.equal(dW.view(torch.int16), dW2.view(torch.int16))
    rng = np.random.default_rng(8)
    ts, ms = _sample_rows(rng, T, M, Kr)
    ref = oracle.bwd_dx_rows(dZ, W, mask, ts, ms)
    got = oracle.bf16_to_f64(_gather(dX, ts, ms))
    assert got.size >= MIN_ELEMS
    G.check_bf16(got, ref, None, f"dX {name}", extra=G.dx_rows_g_allowance(dZ, W, mask, ts, ms))
    ts, ks = _sample_rows(rng, T, Kr, H)
    ref = oracle.bwd_dw_rows(dZ, X, mask, ts, ks)
    got = oracle.bf16_to_f64(_gather(dW, ts, ks))
    assert got.size >= MIN_ELEMS
    G.check_bf16(got, ref, (mask != 0)[None, :], f"dW {name}", extra=G.dw_rows_g_allowance(dZ, X, mask, ts, ks))


@pytest.mark.parametrize("Kr", [1376, 512])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_decode_7b_full_size(ops, M, Kr):
    """Decode-shaped forward on the 7B down-proj (Kr = 1376) and out-proj
    (Kr = 512): complete comparison (the oracle finishes these sizes quickly)."""
    T, H = 8, 4096
    _announce(f"full-size decode M={M} Kr={Kr}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=3)
    mask = synth.make_mask(H, 0.5, "random", seed=3)
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    bits = G.bf16_bits(out)
    S = mask != 0
    assert all(np.array_equal(bits[t][:, S], bits[0][:, S]) for t in range(T))
    G.check_bf16(oracle.bf16_to_f64(bits), oracle.rowpar_pcr_fwd(X, W, mask), S[None, None, :], "decode")


def test_reduce_f32_full_size(ops):
    """fp32 reduce on Y[8, 16384, 4096] with a random 50% mask: sampled rows
    bitwise against the float32 emulation of ascending-rank summation, and
    against the fp64 oracle within 1e-4 rms."""
    T, M, H = 8, 16384, 4096
    _announce("full-size reduce f32")
    Y = synth.make_reduce_input(T, M, H, seed=4)
    mask = synth.make_mask(H, 0.5, "random", seed=4)
    Yd = torch.from_numpy(Y).to(G.dev())
    out = ops.partial_channel_reduce(Yd, G.to_dev_u8(mask))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(M, size=64, replace=False))
    got = out[:, torch.from_numpy(rows).to(G.dev()), :].cpu().numpy()
    Ys = Y[:, rows, :]
    want = G.f32_sequential_reduce(Ys, mask)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    G.check_f32(got, oracle.partial_channel_reduce(Ys, mask), "reduce full size")
    # in place on the same data: local channels untouched everywhere
    ops.partial_channel_reduce(Yd, G.to_dev_u8(mask), inplace=True)
    torch.cuda.synchronize()
    L = torch.from_numpy(mask == 0).to(G.dev())
    Yref = torch.from_numpy(Y).to(G.dev())
    assert torch.equal(Yd[:, :, L].view(torch.int32), Yref[:, :, L].view(torch.int32))
    assert torch.equal(Yd.view(torch.int32), out.view(torch.int32))
