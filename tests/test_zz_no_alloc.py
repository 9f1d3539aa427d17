"""The forward entry point that allocates nothing (caat_rowpar_pcr_fwd_noalloc),
called through the C ABI, against the entry point that takes a workspace
(caat_rowpar_pcr_fwd): bit for bit on the same inputs, several calls in a row
on one GPU's shared scratch, the second smaller than the first, and against
the oracle's bar."""
import ctypes

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


def _call_noalloc(L, X, W, mk, out):
    T, M, Kr = X.shape
    H = W.shape[2]
    st = L.caat_rowpar_pcr_fwd_noalloc(ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(W.data_ptr()),
                                       ctypes.c_void_p(mk.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                       T, M, Kr, H, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


# (T, M, Kr, H, mask kind): the first two are the required pair (the second
# smaller); then a chunked decode call, a tiled call (no scratch used), a
# wide H and an odd rank count
CASES = [
    (8, 32, 1376, 4096, "random"),
    (4, 8, 512, 2048, "random"),
    (8, 100, 512, 4096, "prefix"),
    (8, 256, 384, 768, "random"),
    (2, 5, 64, 9000, "strided"),
    (3, 1, 1376, 4096, "random"),
]


def test_noalloc_matches_workspace_entry_point(ops):
    L = ops.lib()
    for i, (T, M, Kr, H, kind) in enumerate(CASES):
        print(f"[case] noalloc call {i}: T={T} M={M} Kr={Kr} H={H} {kind}", flush=True)
        X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=80 + i)
        mask = synth.make_mask(H, 0.5, kind, seed=80 + i)
        Xd, Wd, mk = G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask)
        ref = ops.rowpar_pcr_fwd(Xd, Wd, mk)
        out = torch.full((T, M, H), float("nan"), dtype=torch.bfloat16, device=G.dev())
        assert _call_noalloc(L, Xd, Wd, mk, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {i} differs from caat_rowpar_pcr_fwd"
        G.check_bf16(G.from_dev_bf16(out), oracle.rowpar_pcr_fwd(X, W, mask), (mask != 0)[None, None, :],
                     f"noalloc call {i}")


def test_noalloc_refuses_oversized_scratch(ops):
    L = ops.lib()
    T, M, Kr, H = 8, 32, 64, 16384  # 8 * 32 * 16384 * 4 bytes of partials: above 16 MiB
    X = torch.zeros((T, M, Kr), dtype=torch.bfloat16, device=G.dev())
    W = torch.zeros((T, Kr, H), dtype=torch.bfloat16, device=G.dev())
    mk = torch.ones(H, dtype=torch.uint8, device=G.dev())
    out = torch.zeros((T, M, H), dtype=torch.bfloat16, device=G.dev())
    assert _call_noalloc(L, X, W, mk, out) == 6  # CAAT_ERR_WORKSPACE, nothing enqueued
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).count_nonzero()) == 0
    # the workspace entry point still serves it
    ops.rowpar_pcr_fwd(X, W, mk, out=out)
    torch.cuda.synchronize()
