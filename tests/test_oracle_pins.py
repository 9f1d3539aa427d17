"""CPU: the oracle against its pins, and planted mistakes against the same pins."""
import numpy as np
import pytest

import oracle
from partial_channel_reduce_amd import synth
from tests import pins


def _fwd(X, W, mask):
    return oracle.rowpar_pcr_fwd(X, W, mask)


def test_fwd_matches_device_simulation_all_masks():
    pins.check_against_device_simulation(_fwd)


def test_all_synced_is_vanilla_layer():
    pins.check_all_synced_is_vanilla(_fwd)


def test_none_synced_is_ensemble():
    pins.check_none_synced_is_ensemble(_fwd)


def test_mixed_mask_invariants():
    pins.check_mixed_invariants(_fwd)


def test_single_rank_is_identity():
    pins.check_single_rank_identity(oracle.partial_channel_reduce)


def test_rank_tags_closed_form():
    pins.check_rank_tags(_fwd)


def test_reduce_matches_device_simulation_all_masks():
    pins.check_reduce_against_device_simulation(oracle.partial_channel_reduce)


def test_reduce_is_self_adjoint():
    pins.check_adjoint(oracle.partial_channel_reduce)


def test_backward_finite_differences():
    pins.check_finite_differences(_fwd, oracle.pcr_bwd)


def test_elementwise_forms_match_simulation():
    """fwd_at / bwd_dx_at / bwd_dw_at, pinned to the device simulation and to
    finite differences on integer inputs (exact)."""
    rng = np.random.default_rng(11)
    T, M, Kr, H = 3, 4, 3, 7
    X = rng.integers(-3, 4, size=(T, M, Kr)).astype(np.float64)
    W = rng.integers(-3, 4, size=(T, Kr, H)).astype(np.float64)
    dZ = rng.integers(-3, 4, size=(T, M, H)).astype(np.float64)
    mask = np.array([1, 0, 1, 1, 0, 0, 1], dtype=np.uint8)
    Z = pins.simulate_devices(X.tolist(), W.tolist(), mask.tolist())
    idx = list(np.ndindex(T, M, H))
    ts, ms, cs = map(np.array, zip(*idx))
    assert np.array_equal(oracle.fwd_at(X, W, mask, ts, ms, cs), Z[ts, ms, cs])

    def loss(Xa, Wa):
        return float(np.sum(pins.simulate_devices(Xa.tolist(), Wa.tolist(), mask.tolist()) * dZ))

    for t, m, k in np.ndindex(T, M, Kr):
        Xp, Xm = X.copy(), X.copy()
        Xp[t, m, k] += 1
        Xm[t, m, k] -= 1
        fd = (loss(Xp, W) - loss(Xm, W)) / 2
        assert oracle.bwd_dx_at(dZ, W, mask, [t], [m], [k])[0] == fd
    for t, k, c in np.ndindex(T, Kr, H):
        Wp, Wm = W.copy(), W.copy()
        Wp[t, k, c] += 1
        Wm[t, k, c] -= 1
        fd = (loss(X, Wp) - loss(X, Wm)) / 2
        assert oracle.bwd_dw_at(dZ, X, mask, [t], [k], [c])[0] == fd


def test_row_forms_match_finite_differences():
    """fwd_rows equals the device simulation's rows; bwd_dx_rows / bwd_dw_rows:
    every entry of the returned rows equals the central difference of the
    device simulation's loss (exact on integers)."""
    rng = np.random.default_rng(12)
    T, M, Kr, H = 3, 5, 4, 6
    X = rng.integers(-3, 4, size=(T, M, Kr)).astype(np.float64)
    W = rng.integers(-3, 4, size=(T, Kr, H)).astype(np.float64)
    dZ = rng.integers(-3, 4, size=(T, M, H)).astype(np.float64)
    mask = np.array([0, 1, 1, 0, 1, 0], dtype=np.uint8)

    def loss(Xa, Wa):
        return float(np.sum(pins.simulate_devices(Xa.tolist(), Wa.tolist(), mask.tolist()) * dZ))

    ts, ms = np.array([2, 0, 1, 2]), np.array([4, 0, 3, 1])
    Z = pins.simulate_devices(X.tolist(), W.tolist(), mask.tolist())
    assert np.array_equal(oracle.fwd_rows(X, W, mask, ts, ms), Z[ts, ms, :])
    rows = oracle.bwd_dx_rows(dZ, W, mask, ts, ms)
    for i, (t, m) in enumerate(zip(ts, ms)):
        for k in range(Kr):
            Xp, Xm = X.copy(), X.copy()
            Xp[t, m, k] += 1
            Xm[t, m, k] -= 1
            assert rows[i, k] == (loss(Xp, W) - loss(Xm, W)) / 2
    ts, ks = np.array([1, 0, 2, 1]), np.array([3, 0, 2, 1])
    rows = oracle.bwd_dw_rows(dZ, X, mask, ts, ks)
    for i, (t, k) in enumerate(zip(ts, ks)):
        for c in range(H):
            Wp, Wm = W.copy(), W.copy()
            Wp[t, k, c] += 1
            Wm[t, k, c] -= 1
            assert rows[i, c] == (loss(X, Wp) - loss(X, Wm)) / 2


def test_bf16_upcast_is_exact():
    # bf16 patterns with known values: 1.0, -2.0, 0.5, smallest normal 2**-126, 3.140625
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0080, 0x4049], dtype=np.uint16)
    want = np.array([1.0, -2.0, 0.5, 2.0 ** -126, 3.140625])
    assert np.array_equal(oracle.bf16_to_f64(bits), want)


@pytest.mark.parametrize("kind", synth.MASK_KINDS)
@pytest.mark.parametrize("H,p", [(768, 0.0), (768, 0.25), (768, 0.5), (768, 0.75), (768, 1.0), (2048, 0.5), (4096, 0.5)])
def test_payload_scales_with_p(kind, H, p):
    """Abstract / Introduction: syncing a fraction p of the channels cuts the
    payload to p of a full all-reduce (p = 0.5 -> the 50% cut)."""
    M, T = 1024, 8
    mask = synth.make_mask(H, p, kind, seed=3)
    n = int(mask.sum())
    assert n == round(p * H)
    assert oracle.synced_elements(mask, M) == int(p * H) * M
    full = oracle.ring_allreduce_bytes_per_rank(T, M, H, 2)
    part = oracle.ring_allreduce_bytes_per_rank(T, M, n, 2)
    assert part == pytest.approx(p * full, rel=0, abs=1e-6)


def test_ring_bytes_match_device_simulation():
    """The ring payload helper equals the elements the message-passing
    device model actually sends (reduce-scatter + all-gather)."""
    pins.check_ring_bytes(oracle.ring_allreduce_bytes_per_rank)


def _ring_no_factor_two(T, M, n, esz):
    return oracle.ring_allreduce_bytes_per_rank(T, M, n, esz) / 2


def _ring_t_not_t_minus_1(T, M, n, esz):
    return 2.0 * T / T * M * n * esz if T > 1 else 0.0


def _ring_over_t_minus_1(T, M, n, esz):
    return 2.0 * (T - 1) / max(T - 1, 1) * M * n * esz if T > 1 else 0.0


def _ring_all_channels(T, M, n, esz):
    return 2.0 * (T - 1) / T * M * max(n, 1) * esz * 2 if T > 1 else 0.0


@pytest.mark.parametrize("mutant", [_ring_no_factor_two, _ring_t_not_t_minus_1, _ring_over_t_minus_1, _ring_all_channels])
def test_ring_bytes_pin_rejects_mutants(mutant):
    with pytest.raises(AssertionError):
        pins.check_ring_bytes(mutant)


def test_strided_half_mask_is_even_channels():
    mask = synth.make_mask(2048, 0.5, "strided")
    assert np.array_equal(np.flatnonzero(mask), np.arange(0, 2048, 2))


# ---------------------------------------------------------------------------
# Planted mistakes.  Each mutant is a plausible slip in the oracle; at least
# one pin must reject it.
# ---------------------------------------------------------------------------

def _mut_mean(X, W, mask):
    Z = oracle.rowpar_pcr_fwd(X, W, mask)
    S = mask != 0
    Z[:, :, S] /= X.shape[0]
    return Z


def _mut_inverted_mask(X, W, mask):
    return oracle.rowpar_pcr_fwd(X, W, (np.asarray(mask) == 0).astype(np.uint8))


def _mut_drop_last_rank(X, W, mask):
    Y = oracle.rowpar_partials(X, W)
    T = Y.shape[0]
    S = np.asarray(mask) != 0
    Z = Y.copy()
    tot = Y[: max(T - 1, 1)].sum(axis=0)
    Z[:, :, S] = tot[None][:, :, S]
    return Z


def _mut_local_from_rank0(X, W, mask):
    Y = oracle.rowpar_partials(X, W)
    Z = oracle.partial_channel_reduce(Y, mask)
    L = np.asarray(mask) == 0
    Z[:, :, L] = Y[0][None][:, :, L]
    return Z


def _mut_wrong_rank_weight(X, W, mask):
    # rank t multiplies by rank (t+1)'s weights
    W2 = np.roll(np.asarray(W, dtype=np.float64), 1, axis=0)
    return oracle.rowpar_pcr_fwd(X, W2, mask)


def _mut_scaled_local(X, W, mask):
    Z = oracle.rowpar_pcr_fwd(X, W, mask)
    L = np.asarray(mask) == 0
    Z[:, :, L] *= X.shape[0]
    return Z


@pytest.mark.parametrize(
    "mutant",
    [_mut_mean, _mut_inverted_mask, _mut_drop_last_rank, _mut_local_from_rank0, _mut_wrong_rank_weight, _mut_scaled_local],
)
def test_forward_pins_reject_mutants(mutant):
    checks = [
        pins.check_against_device_simulation,
        pins.check_all_synced_is_vanilla,
        pins.check_none_synced_is_ensemble,
        pins.check_mixed_invariants,
        pins.check_rank_tags,
    ]
    failed = 0
    for chk in checks:
        try:
            chk(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin rejects {mutant.__name__}"


def _bwd_no_reduce(dZ, X, W, mask):
    return oracle.pcr_bwd(dZ, X, W, np.zeros_like(np.asarray(mask)))


def _bwd_dw_uses_raw_grad(dZ, X, W, mask):
    dX, _ = oracle.pcr_bwd(dZ, X, W, mask)
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    return dX, np.stack([X[t].T @ dZ[t] for t in range(X.shape[0])])


def _bwd_sign(dZ, X, W, mask):
    dX, dW = oracle.pcr_bwd(dZ, X, W, mask)
    return -dX, dW


def _bwd_mean(dZ, X, W, mask):
    T = np.asarray(dZ).shape[0]
    G = oracle.partial_channel_reduce(dZ, mask)
    S = np.asarray(mask) != 0
    G[:, :, S] /= T
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return (np.stack([G[t] @ W[t].T for t in range(T)]), np.stack([X[t].T @ G[t] for t in range(T)]))


@pytest.mark.parametrize("mutant", [_bwd_no_reduce, _bwd_dw_uses_raw_grad, _bwd_sign, _bwd_mean])
def test_backward_pin_rejects_mutants(mutant):
    with pytest.raises(AssertionError):
        pins.check_finite_differences(_fwd, mutant)


def _red_mean(Y, mask):
    Z = oracle.partial_channel_reduce(Y, mask)
    S = np.asarray(mask) != 0
    Z[:, :, S] /= np.asarray(Y).shape[0]
    return Z


def _red_scale_local(Y, mask):
    Z = oracle.partial_channel_reduce(Y, mask)
    L = np.asarray(mask) == 0
    Z[:, :, L] *= 2
    return Z


@pytest.mark.parametrize("mutant", [_red_mean, _red_scale_local])
def test_reduce_pins_reject_mutants(mutant):
    failed = 0
    for chk in (pins.check_single_rank_identity, pins.check_adjoint, pins.check_reduce_against_device_simulation):
        try:
            chk(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1


# ---- the two-layer chain with the column-parallel product ----------------

def test_two_layer_chain_finite_differences():
    pins.check_two_layer_finite_differences(_fwd, oracle.pcr_bwd, oracle.colpar_fwd, oracle.colpar_bwd)


def test_two_layer_all_synced_is_vanilla():
    pins.check_two_layer_all_synced_is_vanilla(_fwd, oracle.pcr_bwd, oracle.colpar_fwd, oracle.colpar_bwd)


def test_two_layer_none_synced_is_ensemble():
    pins.check_two_layer_none_synced_is_ensemble(_fwd, oracle.pcr_bwd, oracle.colpar_fwd, oracle.colpar_bwd)


def _colbwd_allreduce(dU, A, W):
    # the ordinary tensor-parallel backward: the input gradient summed over
    # the ranks, as if every rank's input were the same tensor
    dA, dW = oracle.colpar_bwd(dU, A, W)
    return np.broadcast_to(dA.sum(axis=0), dA.shape).copy(), dW


def _colbwd_next_rank_weight(dU, A, W):
    dA, dW = oracle.colpar_bwd(dU, A, np.roll(np.asarray(W, dtype=np.float64), 1, axis=0))
    return dA, oracle.colpar_bwd(dU, A, W)[1]


def _colbwd_dw_from_wrong_rank(dU, A, W):
    dA, _ = oracle.colpar_bwd(dU, A, W)
    return dA, oracle.colpar_bwd(dU, np.roll(np.asarray(A, dtype=np.float64), 1, axis=0), W)[1]


@pytest.mark.parametrize("mutant", [_colbwd_allreduce, _colbwd_next_rank_weight, _colbwd_dw_from_wrong_rank])
def test_two_layer_pins_reject_mutants(mutant):
    failed = 0
    for chk in (pins.check_two_layer_finite_differences, pins.check_two_layer_all_synced_is_vanilla,
                pins.check_two_layer_none_synced_is_ensemble):
        try:
            chk(_fwd, oracle.pcr_bwd, oracle.colpar_fwd, mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin rejects {mutant.__name__}"
    # the finite-difference pin alone catches every one of them
    with pytest.raises(AssertionError):
        pins.check_two_layer_finite_differences(_fwd, oracle.pcr_bwd, oracle.colpar_fwd, mutant)


# ---- residual update + RMS normalisation ---------------------------------

def test_rmsnorm_closed_forms():
    pins.check_rmsnorm_closed_forms(oracle.residual_rmsnorm)


def test_rmsnorm_invariants():
    pins.check_rmsnorm_invariants(oracle.residual_rmsnorm)


def _rms_sum_not_mean(Z, R, g, eps):
    Rn = np.asarray(Z, np.float64) + np.asarray(R, np.float64)
    return Rn, Rn / np.sqrt(np.sum(Rn * Rn, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def _rms_eps_outside(Z, R, g, eps):
    Rn = np.asarray(Z, np.float64) + np.asarray(R, np.float64)
    return Rn, Rn / (np.sqrt(np.mean(Rn * Rn, axis=-1, keepdims=True)) + eps) * np.asarray(g, np.float64)


def _rms_no_gamma(Z, R, g, eps):
    Rn = np.asarray(Z, np.float64) + np.asarray(R, np.float64)
    return Rn, Rn / np.sqrt(np.mean(Rn * Rn, axis=-1, keepdims=True) + eps)


def _rms_norm_before_residual(Z, R, g, eps):
    Z = np.asarray(Z, np.float64)
    Rn = Z + np.asarray(R, np.float64)
    return Rn, Z / np.sqrt(np.mean(Z * Z, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


@pytest.mark.parametrize("mutant", [_rms_sum_not_mean, _rms_eps_outside, _rms_no_gamma, _rms_norm_before_residual])
def test_rmsnorm_pins_reject_mutants(mutant):
    failed = 0
    for chk in (pins.check_rmsnorm_closed_forms, pins.check_rmsnorm_invariants):
        try:
            chk(mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin rejects {mutant.__name__}"


def test_golden_fixture_reproduces_from_oracle():
    """The stored fixture is exactly what the oracle writes today."""
    import json
    import os

    from tests.golden import make_golden

    here = os.path.join(os.path.dirname(__file__), "golden", "tiny_integer_case.json")
    with open(here) as f:
        stored = json.load(f)
    fresh = json.loads(json.dumps(make_golden.tiny_integer_case()))
    assert stored == fresh
