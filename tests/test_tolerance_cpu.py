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
