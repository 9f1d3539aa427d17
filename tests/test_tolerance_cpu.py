"""The comparison bars of the GPU parity tests, checked on the CPU: the
stated whole-tensor bar max|err| <= 2e-2 * rms(ref) (+ half a bf16 ulp) is
asserted even where the per-class bars would pass, by check_bf16 and by its
block-by-block form."""
import numpy as np
import pytest

import oracle
from tests import gpu_util as G


def _case():
    rng = np.random.default_rng(0)
    n = 4096
    synced = np.arange(n) % 2 == 0
    ref = np.where(synced, 3.0, 1.0) * rng.standard_normal(n)
    got = oracle.bf16_to_f64(G.f32_to_bf16_bits_rne(ref.astype(np.float32)))
    return ref, got, synced


def test_correctly_rounded_output_passes():
    ref, got, synced = _case()
    G.check_bf16(got, ref, synced, "rounded")
    bar = G.Bf16Bar("rounded")
    for s in range(0, ref.size, 1000):
        bar.add(got[s:s + 1000], ref[s:s + 1000], synced[s:s + 1000])
    bar.finish()


def _plant(ref, got, synced):
    # a synced element near zero (half an ulp there is tiny) off by 0.05:
    # above 2e-2 * whole rms (~0.045), below 2e-2 * synced rms (~0.06)
    i = int(np.flatnonzero(synced)[0])
    ref = ref.copy()
    got = got.copy()
    ref[i] = 1e-3
    got[i] = 1e-3 + 0.05
    return ref, got


def test_whole_tensor_violation_is_rejected():
    ref, got, synced = _case()
    ref, got = _plant(ref, got, synced)
    r_all = G.rms(ref)
    r_s = G.rms(ref[synced])
    assert G.BF16_TOL * r_all < 0.05 < G.BF16_TOL * r_s
    with pytest.raises(AssertionError, match="whole tensor"):
        G.check_bf16(got, ref, synced, "planted")
    bar = G.Bf16Bar("planted")
    for s in range(0, ref.size, 1000):
        bar.add(got[s:s + 1000], ref[s:s + 1000], synced[s:s + 1000])
    with pytest.raises(AssertionError, match="whole"):
        bar.finish()


def test_class_violation_is_rejected():
    ref, got, synced = _case()
    i = int(np.flatnonzero(~synced)[0])
    ref[i] = 1e-3
    got[i] = 1e-3 + 0.03  # local rms ~1: above 2e-2 * 1, below 2e-2 * whole rms
    with pytest.raises(AssertionError, match="class"):
        G.check_bf16(got, ref, synced, "planted local")


def _emulated_bwd(dZ, X, W, mask):
    """The backward as documented: G's synced channels rounded once to bf16
    (fp32 ascending-rank sum), exact products, outputs rounded to bf16."""
    from partial_channel_reduce_amd import synth  # noqa: F401

    Gt = oracle.partial_channel_reduce(dZ, mask) + G.g_rounding_shift(dZ, mask)[None]
    Xf, Wf = oracle.bf16_to_f64(X), oracle.bf16_to_f64(W)
    T = Xf.shape[0]
    rnd = lambda a: oracle.bf16_to_f64(G.f32_to_bf16_bits_rne(a.astype(np.float32)))  # noqa: E731
    return (rnd(np.stack([Gt[t] @ Wf[t].T for t in range(T)])), rnd(np.stack([Xf[t].T @ Gt[t] for t in range(T)])))


def test_g_rounding_allowance():
    """A backward with a short contraction (8 tokens) carries the effect of
    G's bf16 rounding; with the allowance the documented arithmetic passes
    the whole-tensor bar, an error beyond it still fails, and with no synced
    channel the allowance is zero."""
    from partial_channel_reduce_amd import synth

    T, M, Kr, H = 8, 8, 1376, 512
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=11)
    dZ = synth.make_grad(T, M, H, seed=11)
    mask = synth.make_mask(H, 0.5, "random", seed=11)
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    eX, eW = _emulated_bwd(dZ, X, W, mask)
    with pytest.raises(AssertionError, match="whole tensor"):
        G.check_bf16(eW, rdW, (mask != 0)[None, None, :], "no allowance")
    ax, aw = G.bwd_g_allowance(dZ, X, W, mask)
    G.check_bf16(eX, rdX, None, "dX", extra=ax)
    G.check_bf16(eW, rdW, (mask != 0)[None, None, :], "dW", extra=aw)
    i = np.unravel_index(np.argmax(np.abs(rdW)), rdW.shape)
    bad = eW.copy()
    bad[i] = rdW[i] - np.sign(rdW[i]) * (0.04 * G.rms(rdW) + G.half_ulp_bf16(rdW[i]) + aw[i])
    with pytest.raises(AssertionError):
        G.check_bf16(bad, rdW, (mask != 0)[None, None, :], "planted", extra=aw)
    ax0, aw0 = G.bwd_g_allowance(dZ, X, W, np.zeros(H, dtype=np.uint8))
    assert not ax0.any() and not aw0.any()
    # the row forms used at full size agree with the whole-tensor form
    ts, ms, ks = np.array([1, 0, 7]), np.array([5, 0, 7]), np.array([3, 1375, 700])
    assert np.allclose(G.dx_rows_g_allowance(dZ, W, mask, ts, ms), ax[ts, ms])
    assert np.allclose(G.dw_rows_g_allowance(dZ, X, mask, ts, ks, block=3), aw[ts, ks])


def test_sweep_covers_every_forward_path():
    """The GPU sweep's seeded shapes reach every forward kernel."""
    from tests.sweep_cases import cases, forward_path

    paths = {forward_path(*c[:4]) for c in cases()}
    assert paths >= {"decode", "chunked", "decode_sliced", "chunked_sliced", "split64", "split64x2", "split128", "split256", "fused128x64", "fused128", "fused256", "queue",
                     "fused256+queue", "fused128+queue", "fused128x64+queue"}, paths
