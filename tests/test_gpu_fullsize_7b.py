"""The Llama2-7B down-projection at full size, compared completely.

* The forward at the benchmark's shape (T=8, M=16384, Kr=1376, H=4096,
  p=0.5), random and contiguous S: every one of the 537M outputs against the
  fp64 oracle, taken in blocks of 2048 tokens, under both the whole-tensor
  and the per-class bar; synced channels bitwise identical across ranks.
* The eight-wave 256x256 kernels at the headline's contraction (T=8,
  Kr=1376: 21 full 64-wide chunks and a half chunk per rank, rank boundaries
  in the middle of the stream) with integer-valued inputs, so that every
  result is exact and forward, dX and dW must equal the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BLOCK = 2048


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("kind", ["random", "prefix"])
def test_fwd_7b_every_element(ops, kind):
    T, M, Kr, H = 8, 16384, 1376, 4096
    _announce(f"7B forward, every element, {kind} S")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=5)
    mask = synth.make_mask(H, 0.5, kind, seed=5)
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    bits = G.bf16_bits(out)
    del out
    S = mask != 0
    for t in range(1, T):
        assert np.array_equal(bits[t][:, S], bits[0][:, S]), f"synced channels differ between rank 0 and {t}"
    bar = G.Bf16Bar(f"7B fwd {kind}")
    for m0 in range(0, M, BLOCK):
        ref = oracle.rowpar_pcr_fwd(X[:, m0:m0 + BLOCK], W, mask)
        bar.add(oracle.bf16_to_f64(bits[:, m0:m0 + BLOCK]), ref, S[None, None, :])
    rep = bar.finish()
    print(f"[result] {rep}", flush=True)


def _int_inputs(T, M, Kr, H, seed):
    # X, W in {-1, 0, 1} (X 80% zeros), dZ in {-1, 0, 1} (95% zeros): every
    # output, partial and synced sum is an integer well inside bf16's exact
    # range, so any summation order gives the same bits
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=seed, lo=-1, hi=1, x_zero_frac=0.8)
    rng = np.random.default_rng(seed + 70_000)
    dZ = rng.integers(-1, 2, size=(T, M, H)).astype(np.float32) * (rng.random((T, M, H)) < 0.05)
    return X, W, synth.f32_to_bf16_bits(dZ.astype(np.float32))


def test_big_tiles_7b_contraction_bitwise(ops):
    T, M, Kr, H = 8, 4096, 1376, 4096
    _announce(f"eight-wave kernels, T={T} M={M} Kr={Kr} H={H}, integer inputs")
    X, W, dZ = _int_inputs(T, M, Kr, H, seed=61)
    mask = synth.make_mask(H, 0.5, "random", seed=61)
    Xd, Wd, dZd, mk = G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_bf16(dZ), G.to_dev_u8(mask)
    out = ops.rowpar_pcr_fwd(Xd, Wd, mk)
    dX, dW = ops.pcr_bwd(dZd, Xd, Wd, mk)
    torch.cuda.synchronize()
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    assert np.array_equal(G.from_dev_bf16(out), ref), "forward differs from the oracle"
    del ref
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert np.abs(rdX).max() <= 256 and np.abs(rdW).max() <= 256
    assert np.array_equal(G.from_dev_bf16(dX), rdX), "dX differs from the oracle"
    assert np.array_equal(G.from_dev_bf16(dW), rdW), "dW differs from the oracle"
