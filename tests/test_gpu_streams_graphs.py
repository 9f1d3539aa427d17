"""The library enqueues every call on the caller's stream and allocates
nothing, so its calls run on any stream and can be captured into a HIP graph
(the decode kernel's arrival counters return to zero after every call).
Checked here: a side stream gives the default stream's bits; a captured
sequence (decode-shaped forward, whole and in contraction slices, split
forward and its reduce pass, fused tiled forward, backward) replayed several
times, with eager calls and synchronisation in between, reproduces the eager
results bit for bit every time."""
import numpy as np
import pytest
import torch

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


def test_side_stream_matches_default_stream(ops):
    _announce("side stream")
    T, M, Kr, H = 4, 300, 200, 776
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=51)
    dZ = synth.make_grad(T, M, H, seed=51)
    mask = synth.make_mask(H, 0.5, "random", seed=51)
    Xd, Wd, dZd, mk = G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_bf16(dZ), G.to_dev_u8(mask)
    out0 = ops.rowpar_pcr_fwd(Xd, Wd, mk)
    dX0, dW0 = ops.pcr_bwd(dZd, Xd, Wd, mk)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out1 = ops.rowpar_pcr_fwd(Xd, Wd, mk)
        dX1, dW1 = ops.pcr_bwd(dZd, Xd, Wd, mk)
    side.synchronize()
    for a, b in ((out0, out1), (dX0, dX1), (dW0, dW1)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_graph_replays_match_eager(ops):
    _announce("graph capture and replay")
    dev = G.dev()
    T, Kr, H = 8, 1376, 512
    Md, Mt = 8, 300
    mask = G.to_dev_u8(synth.make_mask(H, 0.5, "random", seed=52))
    Xd_, W_ = synth.make_fwd_inputs(T, Md, Kr, H, seed=52)
    Xt_, _ = synth.make_fwd_inputs(T, Mt, Kr, H, seed=53)
    dZ_ = synth.make_grad(T, Mt, H, seed=53)
    Xdec, W, Xt, dZ = G.to_dev_bf16(Xd_), G.to_dev_bf16(W_), G.to_dev_bf16(Xt_), G.to_dev_bf16(dZ_)
    # a fused-tile forward too: 2100 tokens with a two-chunk contraction
    Mf, Krf = 2100, 96
    Xf_, Wf_ = synth.make_fwd_inputs(T, Mf, Krf, H, seed=54)
    Xf, Wf = G.to_dev_bf16(Xf_), G.to_dev_bf16(Wf_)
    assert ops.fwd_workspace_bytes(T, Mf, Krf, H) == 0 and ops.fwd_workspace_bytes(T, Mt, Kr, H) > 2048
    # a decode call with two ranks: each contraction in four slices
    Ts, Krs = 2, 2056
    Xs_, Ws_ = synth.make_fwd_inputs(Ts, Md, Krs, H, seed=55)
    Xs, Ws = G.to_dev_bf16(Xs_), G.to_dev_bf16(Ws_)
    assert ops.fwd_workspace_bytes(Ts, Md, Krs, H) == 2048 + 4 * Ts * Md * H * 4
    # every buffer exists before capture: nothing is allocated inside the graph
    o_dec = torch.empty((T, Md, H), dtype=torch.bfloat16, device=dev)
    o_t = torch.empty((T, Mt, H), dtype=torch.bfloat16, device=dev)
    o_f = torch.empty((T, Mf, H), dtype=torch.bfloat16, device=dev)
    o_s = torch.empty((Ts, Md, H), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((T, Mt, Kr), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((T, Kr, H), dtype=torch.bfloat16, device=dev)
    ws_dec = torch.zeros(ops.fwd_workspace_bytes(T, Md, Kr, H), dtype=torch.uint8, device=dev)
    ws_t = torch.zeros(ops.fwd_workspace_bytes(T, Mt, Kr, H), dtype=torch.uint8, device=dev)
    ws_s = torch.zeros(ops.fwd_workspace_bytes(Ts, Md, Krs, H), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(ops.bwd_workspace_bytes(T, Mt, Kr, H), dtype=torch.uint8, device=dev)

    def seq():
        ops.rowpar_pcr_fwd(Xdec, W, mask, out=o_dec, workspace=ws_dec)
        ops.rowpar_pcr_fwd(Xt, W, mask, out=o_t, workspace=ws_t)  # split forward + reduce pass
        ops.rowpar_pcr_fwd(Xf, Wf, mask, out=o_f)  # fused tiles, no workspace
        ops.rowpar_pcr_fwd(Xs, Ws, mask, out=o_s, workspace=ws_s)  # decode in contraction slices
        ops.pcr_bwd(dZ, Xt, W, mask, dX=dX, dW=dW, workspace=ws_bwd)

    seq()
    torch.cuda.synchronize()
    outs = (o_dec, o_t, o_f, o_s, dX, dW)
    want = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        seq()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    torch.cuda.synchronize()

    scratch = torch.empty_like(o_t)
    for rep in range(4):
        for t in outs:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("decode out", "split out", "fused out", "sliced decode out", "dX", "dW"), outs, want):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (rep, name)
        # eager work between replays, on other buffers
        ops.rowpar_pcr_fwd(Xt, W, mask, out=scratch)
        torch.cuda.synchronize()
    # the decode workspace's arrival counters are back at zero after the replays
    H_blocks = (H + 127) // 128
    assert int(ws_dec[: 4 * H_blocks].view(torch.int32).abs().sum().item()) == 0
    assert int(ws_s[:2048].count_nonzero()) == 0


def test_graph_replays_split_dw_backward(ops):
    """A backward whose dW is split over the token range (fp32 pieces in the
    workspace, then their ordered sum) captured in a graph: 128x128 tiles in
    seven pieces and 256x256 tiles in three.  Every replay matches eager."""
    _announce("graph capture of split-dW backwards")
    dev = G.dev()
    cases = [(2, 4000, 96, 264, 61), (4, 1600, 264, 2056, 62)]
    bufs = []
    for T, M, Kr, H, seed in cases:
        X_, W_ = synth.make_fwd_inputs(T, M, Kr, H, seed=seed)
        dZ_ = synth.make_grad(T, M, H, seed=seed)
        mk = G.to_dev_u8(synth.make_mask(H, 0.5, "random", seed=seed))
        ws = torch.empty(ops.bwd_workspace_bytes(T, M, Kr, H), dtype=torch.uint8, device=dev)
        assert ws.numel() > -(-(T * M * H * 2) // 256) * 256  # the split's pieces are in the workspace
        bufs.append((G.to_dev_bf16(dZ_), G.to_dev_bf16(X_), G.to_dev_bf16(W_), mk, ws,
                     torch.empty((T, M, Kr), dtype=torch.bfloat16, device=dev),
                     torch.empty((T, Kr, H), dtype=torch.bfloat16, device=dev)))

    def seq():
        for dZ, X, W, mk, ws, dX, dW in bufs:
            ops.pcr_bwd(dZ, X, W, mk, dX=dX, dW=dW, workspace=ws)

    seq()
    torch.cuda.synchronize()
    want = [(b[5].clone(), b[6].clone()) for b in bufs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        seq()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    torch.cuda.synchronize()
    for rep in range(3):
        for b in bufs:
            b[5].fill_(0)
            b[6].fill_(0)
            b[4].fill_(0x7F)  # stale workspace contents must not matter
        g.replay()
        torch.cuda.synchronize()
        for i, (b, (wx, ww)) in enumerate(zip(bufs, want)):
            assert torch.equal(b[5].view(torch.int16), wx.view(torch.int16)), (rep, i, "dX")
            assert torch.equal(b[6].view(torch.int16), ww.view(torch.int16)), (rep, i, "dW")
        seq()  # eager work between replays
        torch.cuda.synchronize()
