"""A seeded sweep of random shapes over every forward path (decode, chunked
decode, split with 128x64 tiles -- whole contractions or two slices of them --
128x128 and 256x256 tiles, fused 128x64 / 128x128 / 256x256 tiles, the
register-queue tiles) and the backward: integer inputs, bit for bit against the
oracle, several ranks, ragged sizes, every kind of sync set."""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G
from tests.sweep_cases import cases, forward_path

pytestmark = pytest.mark.gpu

CASES = cases()


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _inputs(T, M, Kr, H, kind, p, seed):
    # few nonzero products per output: every partial sum is an integer below 2^8
    zf = 1.0 - min(0.9, 6.0 / np.sqrt(max(1, T * Kr)))
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=seed, lo=-1, hi=1, x_zero_frac=zf)
    mask = synth.make_mask(H, p, kind, seed=seed + 1)
    return X, W, mask


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-M{c[1]}-Kr{c[2]}-H{c[3]}-{c[4]}{c[5]}" for c in CASES])
def test_sweep_forward_bitwise(ops, case):
    T, M, Kr, H, kind, p, seed = case
    print(f"[case] sweep fwd {case} path={forward_path(T, M, Kr, H)}", flush=True)
    X, W, mask = _inputs(*case)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)


BWD_CASES = CASES[::4] + [c for c in CASES if c[0] == 64 and c not in CASES[::4]]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"T{c[0]}-M{c[1]}-Kr{c[2]}-H{c[3]}-{c[4]}{c[5]}" for c in BWD_CASES])
def test_sweep_backward_bitwise(ops, case):
    T, M, Kr, H, kind, p, seed = case
    print(f"[case] sweep bwd {case}", flush=True)
    X, W, mask = _inputs(*case)
    rng = np.random.default_rng(seed + 2)
    nz = min(0.5, 6.0 / np.sqrt(max(1, T * max(M, H))))
    dZ = synth.f32_to_bf16_bits((rng.integers(-1, 2, size=(T, M, H)) * (rng.random((T, M, H)) < nz)).astype(np.float32))
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert max(np.abs(rdX).max(), np.abs(rdW).max()) <= 256
    dX, dW = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dX), rdX)
    assert np.array_equal(G.from_dev_bf16(dW), rdW)
