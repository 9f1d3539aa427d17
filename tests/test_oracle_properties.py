"""Property-based checks of the CPU oracle over random shapes, rank counts and
sync masks (the fixed-shape pins in test_oracle_pins cover the named cases).
Facts checked, from the definition of the partial channel-reduce (CAAT-Net
paper, Introduction): synced channels hold the un-sharded layer's output on
every rank; local channels add up over the ranks to it; the reduce is
self-adjoint; the backward is the gradient (integer inputs, exact); the
two-layer chain's input gradient reduces to the textbook one when every
channel is synced."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from tests import pins

shapes = st.tuples(st.integers(1, 6), st.integers(1, 5), st.integers(1, 5), st.integers(1, 9))


def _case(seed, T, M, Kr, H, ints=False):
    rng = np.random.default_rng(seed)
    if ints:
        X = rng.integers(-3, 4, size=(T, M, Kr)).astype(np.float64)
        W = rng.integers(-3, 4, size=(T, Kr, H)).astype(np.float64)
    else:
        X = rng.standard_normal((T, M, Kr))
        W = rng.standard_normal((T, Kr, H))
    mask = (rng.random(H) < rng.random()).astype(np.uint8)
    return rng, X, W, mask


@settings(max_examples=60, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1))
def test_synced_equal_full_layer_and_locals_add_up(shp, seed):
    T, M, Kr, H = shp
    _, X, W, mask = _case(seed, T, M, Kr, H)
    Z = oracle.rowpar_pcr_fwd(X, W, mask)
    full = pins.full_layer(X, W)
    S = mask != 0
    for t in range(T):
        np.testing.assert_allclose(Z[t][:, S], full[:, S], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Z[:, :, ~S].sum(axis=0), full[:, ~S], rtol=1e-12, atol=1e-12)


@settings(max_examples=60, deadline=None)
@given(shapes, st.integers(0, 2**31 - 1))
def test_reduce_self_adjoint(shp, seed):
    T, M, _, H = shp
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal((T, M, H))
    D = rng.standard_normal((T, M, H))
    mask = (rng.random(H) < 0.5).astype(np.uint8)
    lhs = np.sum(oracle.partial_channel_reduce(Y, mask) * D)
    rhs = np.sum(Y * oracle.partial_channel_reduce(D, mask))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


@settings(max_examples=25, deadline=None)
@given(st.tuples(st.integers(1, 4), st.integers(1, 3), st.integers(1, 3), st.integers(1, 5)), st.integers(0, 2**31 - 1))
def test_backward_is_exact_gradient_on_integers(shp, seed):
    T, M, Kr, H = shp
    rng, X, W, mask = _case(seed, T, M, Kr, H, ints=True)
    dZ = rng.integers(-3, 4, size=(T, M, H)).astype(np.float64)
    dX, dW = oracle.pcr_bwd(dZ, X, W, mask)

    def loss(Xa, Wa):
        return float(np.sum(oracle.rowpar_pcr_fwd(Xa, Wa, mask) * dZ))

    for idx in np.ndindex(*X.shape):
        Xp, Xm = X.copy(), X.copy()
        Xp[idx] += 1.0
        Xm[idx] -= 1.0
        assert (loss(Xp, W) - loss(Xm, W)) / 2.0 == dX[idx]
    for idx in np.ndindex(*W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += 1.0
        Wm[idx] -= 1.0
        assert (loss(X, Wp) - loss(X, Wm)) / 2.0 == dW[idx]


@settings(max_examples=40, deadline=None)
@given(st.tuples(st.integers(1, 6), st.integers(1, 4), st.integers(1, 4), st.integers(1, 6), st.integers(1, 4)),
       st.integers(0, 2**31 - 1))
def test_two_layer_all_synced_matches_textbook(shp, seed):
    T, M, Kr, H, N = shp
    rng = np.random.default_rng(seed)
    X, W = rng.standard_normal((T, M, Kr)), rng.standard_normal((T, Kr, H))
    W1, C = rng.standard_normal((T, H, N)), rng.standard_normal((T, M, N))
    mask = np.ones(H, dtype=np.uint8)
    dZ, _ = oracle.colpar_bwd(C, oracle.rowpar_pcr_fwd(X, W, mask), W1)
    dX, _ = oracle.pcr_bwd(dZ, X, W, mask)
    cat = lambda A, ax: np.concatenate([A[t] for t in range(T)], axis=ax)  # noqa: E731
    want = cat(C, 1) @ cat(W1, 1).T @ cat(W, 0).T
    np.testing.assert_allclose(cat(dX, 1), want, rtol=1e-10, atol=1e-10)
