"""Independent checks that pin the CPU oracle (and any implementation of the
same maps) to facts the pages and the mathematics fix.

Each checker takes the implementation under test as a callable and returns
None on success or raises AssertionError.  The pin tests run them against the
oracle; the mutation tests run them against deliberately broken copies of the
oracle and expect a failure, which shows each pin can catch a plausible slip.

Source of the facts: "Tensor-Parallelism with Partially Synchronized
Activations", Introduction (only a subset of hidden channels is reduced;
activations then differ across devices; no channel reduced = an ensemble; all
channels reduced = the vanilla model; forward and backward must agree) and
Abstract (the payload falls with the fraction of synced channels).
"""
from __future__ import annotations

import itertools

import numpy as np


# ---------------------------------------------------------------------------
# A message-passing model of T devices.  Each device computes its own partial
# product with scalar loops, packs the channels of S into a send buffer, and
# the devices run a ring all-reduce (reduce-scatter then all-gather) on that
# buffer only; each device then unpacks the reduced channels.  This is the
# collective the partial channel-reduce stands for, written as a different
# algorithm from the oracle's direct definition.  With small-integer inputs
# every sum is exact, so the two must agree bit for bit.
# ---------------------------------------------------------------------------

def simulate_devices(X, W, mask, sent=None):
    """Run the model; if `sent` is a list, it receives the number of elements
    each device put on the ring (both phases)."""
    T = len(X)
    M = len(X[0])
    Kr = len(X[0][0])
    H = len(W[0][0])
    partial = [
        [[sum(X[t][m][k] * W[t][k][c] for k in range(Kr)) for c in range(H)] for m in range(M)]
        for t in range(T)
    ]
    S = [c for c in range(H) if mask[c]]
    send = [[partial[t][m][c] for m in range(M) for c in S] for t in range(T)]
    n = len(S) * M
    bounds = [n * i // T for i in range(T + 1)]
    nsent = [0] * T

    def seg(i):
        i %= T
        return range(bounds[i], bounds[i + 1])

    # reduce-scatter: at step s device t passes segment (t - s) to device t+1
    for s in range(T - 1):
        msgs = [(t, [send[t][j] for j in seg(t - s)]) for t in range(T)]
        for t, payload in msgs:
            nsent[t] += len(payload)
            dst = (t + 1) % T
            for j, v in zip(seg(t - s), payload):
                send[dst][j] += v
    # device t now holds the full sum of segment (t + 1); all-gather it around the ring
    for s in range(T - 1):
        msgs = [(t, [send[t][j] for j in seg(t + 1 - s)]) for t in range(T)]
        for t, payload in msgs:
            nsent[t] += len(payload)
            dst = (t + 1) % T
            for j, v in zip(seg(t + 1 - s), payload):
                send[dst][j] = v
    if sent is not None:
        sent[:] = nsent
    out = [[[partial[t][m][c] for c in range(H)] for m in range(M)] for t in range(T)]
    for t in range(T):
        j = 0
        for m in range(M):
            for c in S:
                out[t][m][c] = send[t][j]
                j += 1
    return np.asarray(out, dtype=np.float64)


def check_against_device_simulation(fwd, shapes=((1, 2, 3, 4), (2, 2, 3, 5), (3, 3, 2, 4), (4, 2, 4, 6)), seed=0):
    """All 2**H masks for each (T, M, Kr, H): fwd must equal the ring simulation exactly."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H in shapes:
        X = rng.integers(-3, 4, size=(T, M, Kr)).astype(np.float64)
        W = rng.integers(-3, 4, size=(T, Kr, H)).astype(np.float64)
        for bits in itertools.product((0, 1), repeat=H):
            mask = np.asarray(bits, dtype=np.uint8)
            want = simulate_devices(X.tolist(), W.tolist(), mask.tolist())
            got = fwd(X, W, mask)
            assert got.shape == want.shape, (got.shape, want.shape)
            assert np.array_equal(got, want), f"T={T} M={M} Kr={Kr} H={H} mask={bits}"


def _random_case(rng, T, M, Kr, H):
    X = rng.standard_normal((T, M, Kr))
    W = 0.02 * rng.standard_normal((T, Kr, H))
    return X, W


def full_layer(X, W):
    """The un-sharded layer: X_full[m, t*Kr+k] = X[t,m,k], W_full[t*Kr+k, c] = W[t,k,c]."""
    T, M, Kr = X.shape
    X_full = np.concatenate([X[t] for t in range(T)], axis=1)
    W_full = np.concatenate([W[t] for t in range(T)], axis=0)
    return X_full @ W_full


def check_all_synced_is_vanilla(fwd, seed=1):
    """Every channel synced: each rank holds the un-sharded layer's output."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H in ((1, 5, 4, 6), (2, 7, 5, 8), (4, 6, 3, 10), (8, 4, 2, 16)):
        X, W = _random_case(rng, T, M, Kr, H)
        want = full_layer(X, W)
        Z = fwd(X, W, np.ones(H, dtype=np.uint8))
        for t in range(T):
            np.testing.assert_allclose(Z[t], want, rtol=1e-12, atol=1e-13)


def check_none_synced_is_ensemble(fwd, seed=2):
    """No channel synced: each rank holds its own layer's output (an ensemble)."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H in ((1, 5, 4, 6), (2, 7, 5, 8), (4, 6, 3, 10)):
        X, W = _random_case(rng, T, M, Kr, H)
        want = np.matmul(X, W)  # batched per-rank product (library routine)
        Z = fwd(X, W, np.zeros(H, dtype=np.uint8))
        np.testing.assert_allclose(Z, want, rtol=1e-12, atol=1e-13)


def check_mixed_invariants(fwd, seed=3):
    """Any S: synced channels equal the un-sharded layer on every rank; the
    local channels' per-rank values add up to the un-sharded layer."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H in ((2, 5, 4, 8), (3, 4, 6, 9), (8, 3, 2, 16)):
        X, W = _random_case(rng, T, M, Kr, H)
        full = full_layer(X, W)
        for _ in range(3):
            mask = (rng.random(H) < 0.5).astype(np.uint8)
            S = mask != 0
            Z = fwd(X, W, mask)
            for t in range(T):
                np.testing.assert_allclose(Z[t][:, S], full[:, S], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Z[:, :, ~S].sum(axis=0), full[:, ~S], rtol=1e-12, atol=1e-13)
            # synced channels are one value broadcast to all ranks
            for t in range(1, T):
                assert np.array_equal(Z[t][:, S], Z[0][:, S])


def check_single_rank_identity(reduce_fn, seed=4):
    """T = 1: the reduce is the identity for any mask."""
    rng = np.random.default_rng(seed)
    Y = rng.standard_normal((1, 6, 10))
    for _ in range(4):
        mask = (rng.random(10) < 0.5).astype(np.uint8)
        assert np.array_equal(reduce_fn(Y, mask), Y)


def check_rank_tags(fwd, T=8, M=12, Kr=5, H=16):
    """One-hot rows and W_t = 2**t * s_c make each local output name its rank
    (2**t * s_c) and each synced output equal s_c * (2**T - 1)."""
    rng = np.random.default_rng(5)
    s = rng.choice([1.0, 2.0], size=H)
    X = np.zeros((T, M, Kr))
    X[:, np.arange(M), np.arange(M) % Kr] = 1.0
    W = np.stack([(2.0 ** t) * np.tile(s, (Kr, 1)) for t in range(T)])
    mask = (rng.random(H) < 0.5).astype(np.uint8)
    Z = fwd(X, W, mask)
    for t in range(T):
        for c in range(H):
            want = s[c] * (2 ** T - 1) if mask[c] else s[c] * 2 ** t
            assert np.all(Z[t, :, c] == want), (t, c)


def check_reduce_against_device_simulation(reduce_fn, seed=8):
    """The reduce alone on integer per-rank tensors, all 2**H masks: equal to the
    ring simulation fed with identity rows (so each device's partial is Y[t])."""
    rng = np.random.default_rng(seed)
    for T, M, H in ((1, 2, 4), (2, 3, 5), (3, 2, 4), (4, 2, 5)):
        Y = rng.integers(-4, 5, size=(T, M, H)).astype(np.float64)
        eye = np.stack([np.eye(M) for _ in range(T)])
        for bits in itertools.product((0, 1), repeat=H):
            mask = np.asarray(bits, dtype=np.uint8)
            want = simulate_devices(eye.tolist(), Y.tolist(), mask.tolist())
            assert np.array_equal(reduce_fn(Y, mask), want), (T, M, H, bits)


def check_adjoint(reduce_fn, seed=6):
    """The reduce is self-adjoint: <R(Y), D> = <Y, R(D)> for every Y, D, S."""
    rng = np.random.default_rng(seed)
    for T, M, H in ((2, 4, 6), (4, 3, 9), (8, 2, 16)):
        for _ in range(3):
            Y = rng.standard_normal((T, M, H))
            D = rng.standard_normal((T, M, H))
            mask = (rng.random(H) < 0.5).astype(np.uint8)
            lhs = float(np.sum(reduce_fn(Y, mask) * D))
            rhs = float(np.sum(Y * reduce_fn(D, mask)))
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def check_finite_differences(fwd, bwd, seed=7):
    """Backward = gradient of L(X, W) = sum(fwd(X, W) * dZ).

    L is bilinear in (X, W), so the central difference with step 1 is exact on
    integer inputs; every entry of dX and dW is checked."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H in ((2, 3, 2, 4), (3, 2, 3, 5), (4, 2, 2, 6)):
        X = rng.integers(-3, 4, size=(T, M, Kr)).astype(np.float64)
        W = rng.integers(-3, 4, size=(T, Kr, H)).astype(np.float64)
        dZ = rng.integers(-3, 4, size=(T, M, H)).astype(np.float64)
        mask = (rng.random(H) < 0.5).astype(np.uint8)
        mask[0], mask[-1] = 1, 0  # at least one channel of each kind

        def loss(Xa, Wa):
            return float(np.sum(fwd(Xa, Wa, mask) * dZ))

        dX, dW = bwd(dZ, X, W, mask)
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += 1.0
            Xm[idx] -= 1.0
            fd = (loss(Xp, W) - loss(Xm, W)) / 2.0
            assert fd == dX[idx], ("dX", idx, fd, dX[idx])
        for idx in np.ndindex(*W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += 1.0
            Wm[idx] -= 1.0
            fd = (loss(X, Wp) - loss(X, Wm)) / 2.0
            assert fd == dW[idx], ("dW", idx, fd, dW[idx])


# ---------------------------------------------------------------------------
# The two-layer chain: the row-parallel layer with partial channel-reduce,
# then a column-parallel product that takes each rank's own (now different)
# activation.  Introduction: forward and backward must agree; the ordinary
# tensor-parallel backward, which sums the column-parallel layer's input
# gradient over the ranks because that input is replicated, does not.
# ---------------------------------------------------------------------------

def _concat_ranks(A, axis):
    return np.concatenate([A[t] for t in range(A.shape[0])], axis=axis)


def check_two_layer_finite_differences(fwd, bwd, colfwd, colbwd, seed=9):
    """Chained backward (colbwd, then bwd on its input gradient) = gradient
    of L(X, W, W1) = sum(colfwd(fwd(X, W), W1) * C).  L is linear in each of
    X, W and W1, so the central difference with step 1 is exact on integer
    inputs; every entry of dX, dW and dW1 is checked."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H, N in ((2, 2, 2, 4, 3), (3, 2, 2, 5, 2), (4, 2, 1, 4, 2)):
        X = rng.integers(-2, 3, size=(T, M, Kr)).astype(np.float64)
        W = rng.integers(-2, 3, size=(T, Kr, H)).astype(np.float64)
        W1 = rng.integers(-2, 3, size=(T, H, N)).astype(np.float64)
        C = rng.integers(-2, 3, size=(T, M, N)).astype(np.float64)
        mask = (rng.random(H) < 0.5).astype(np.uint8)
        mask[0], mask[-1] = 1, 0  # at least one channel of each kind

        def loss(Xa, Wa, W1a):
            return float(np.sum(colfwd(fwd(Xa, Wa, mask), W1a) * C))

        dZ, dW1 = colbwd(C, fwd(X, W, mask), W1)
        dX, dW = bwd(dZ, X, W, mask)
        for name, arr, grad in (("dX", X, dX), ("dW", W, dW), ("dW1", W1, dW1)):
            for idx in np.ndindex(*arr.shape):
                p, m = arr.copy(), arr.copy()
                p[idx] += 1.0
                m[idx] -= 1.0
                args_p = [X, W, W1]
                args_m = [X, W, W1]
                k = ("dX", "dW", "dW1").index(name)
                args_p[k], args_m[k] = p, m
                fd = (loss(*args_p) - loss(*args_m)) / 2.0
                assert fd == grad[idx], (name, (T, M, Kr, H, N), idx, fd, grad[idx])


def check_two_layer_all_synced_is_vanilla(fwd, bwd, colfwd, colbwd, seed=10):
    """All channels synced: the chain is the un-sharded two-layer product
    U_full = X_full W_full W1_full, whose gradients are the textbook ones:
    d X_full = C_full W1_full^T W_full^T, d W_full = X_full^T (C_full W1_full^T),
    d W1_full = (X_full W_full)^T C_full (each rank holds its slices)."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H, N in ((2, 5, 3, 6, 4), (4, 3, 2, 8, 3), (8, 2, 2, 5, 2)):
        X = rng.standard_normal((T, M, Kr))
        W = rng.standard_normal((T, Kr, H))
        W1 = rng.standard_normal((T, H, N))
        C = rng.standard_normal((T, M, N))
        mask = np.ones(H, dtype=np.uint8)
        dZ, dW1 = colbwd(C, fwd(X, W, mask), W1)
        dX, dW = bwd(dZ, X, W, mask)
        Xf, Wf = _concat_ranks(X, 1), _concat_ranks(W, 0)
        W1f, Cf = _concat_ranks(W1, 1), _concat_ranks(C, 1)
        Gf = Cf @ W1f.T
        np.testing.assert_allclose(_concat_ranks(dX, 1), Gf @ Wf.T, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(_concat_ranks(dW, 0), Xf.T @ Gf, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(_concat_ranks(dW1, 1), (Xf @ Wf).T @ Cf, rtol=1e-11, atol=1e-11)


def check_two_layer_none_synced_is_ensemble(fwd, bwd, colfwd, colbwd, seed=11):
    """No channel synced: T independent two-layer products, dX[t] = C[t] W1[t]^T W[t]^T."""
    rng = np.random.default_rng(seed)
    for T, M, Kr, H, N in ((2, 5, 3, 6, 4), (4, 3, 2, 8, 3)):
        X = rng.standard_normal((T, M, Kr))
        W = rng.standard_normal((T, Kr, H))
        W1 = rng.standard_normal((T, H, N))
        C = rng.standard_normal((T, M, N))
        mask = np.zeros(H, dtype=np.uint8)
        np.testing.assert_allclose(colfwd(fwd(X, W, mask), W1), np.matmul(np.matmul(X, W), W1), rtol=1e-11, atol=1e-11)
        dZ, _ = colbwd(C, fwd(X, W, mask), W1)
        dX, _ = bwd(dZ, X, W, mask)
        want = np.matmul(np.matmul(C, np.transpose(W1, (0, 2, 1))), np.transpose(W, (0, 2, 1)))
        np.testing.assert_allclose(dX, want, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# Residual update + RMS normalisation (the step after the partial reduce).
# ---------------------------------------------------------------------------

def check_rmsnorm_closed_forms(fn):
    """Values the definition fixes by hand: x = (3, 4), eps = 1, gamma = 1
    gives mean square 12.5 and x / sqrt(13.5); a one-hot row c*e_k with
    eps = 0 gives sign(c) * sqrt(H) * gamma_k at k and zeros elsewhere; a
    zero row with eps > 0 stays zero."""
    Z = np.array([[[3.0, 4.0]]])
    _, N = fn(Z, np.zeros_like(Z), np.ones(2), 1.0)
    np.testing.assert_allclose(N[0, 0], [3.0 / np.sqrt(13.5), 4.0 / np.sqrt(13.5)], rtol=1e-14)
    H = 16
    gamma = np.linspace(0.5, 2.0, H)
    for c, k in ((2.5, 3), (-7.0, 0), (0.125, 15)):
        Z = np.zeros((1, 1, H))
        Z[0, 0, k] = c
        _, N = fn(Z, np.zeros_like(Z), gamma, 0.0)
        want = np.zeros(H)
        want[k] = np.sign(c) * np.sqrt(H) * gamma[k]
        np.testing.assert_allclose(N[0, 0], want, rtol=1e-13, atol=1e-15)
    _, N = fn(np.zeros((2, 3, 8)), np.zeros((2, 3, 8)), np.ones(8), 1e-5)
    assert np.all(N == 0.0)


def check_rmsnorm_invariants(fn, seed=12):
    """The residual update is the plain sum; with eps = 0 the norm is
    invariant to positive scaling of a row, odd in the row, and with
    gamma = 1 every output row has mean square 1 and points along R + Z."""
    rng = np.random.default_rng(seed)
    T, M, H = 3, 5, 24
    Z = rng.standard_normal((T, M, H))
    R = rng.standard_normal((T, M, H))
    g = rng.uniform(0.5, 1.5, H)
    Rn, N = fn(Z, R, g, 0.0)
    np.testing.assert_allclose(Rn, Z + R, rtol=0, atol=0)
    _, N2 = fn(3.5 * Z, 3.5 * R, g, 0.0)
    np.testing.assert_allclose(N2, N, rtol=1e-13, atol=1e-14)
    _, N3 = fn(-Z, -R, g, 0.0)
    np.testing.assert_allclose(N3, -N, rtol=1e-13, atol=1e-14)
    _, N1 = fn(Z, R, np.ones(H), 0.0)
    np.testing.assert_allclose(np.mean(N1 * N1, axis=-1), 1.0, rtol=1e-13)
    # what is normalised is the updated residual R + Z: with gamma = 1 each
    # output row is that sum divided by its root mean square
    S = Z + R
    np.testing.assert_allclose(N1 * np.sqrt(np.mean(S * S, axis=-1, keepdims=True)), S, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Payload of the restricted all-reduce (Abstract and Introduction: the
# payload falls with the fraction of synced channels).  The device model
# above counts the elements every device puts on the ring; a helper that
# prices that traffic must match the count: on average over the devices
# exactly, and per device whenever the packed buffer splits evenly.
# ---------------------------------------------------------------------------

def check_ring_bytes(ring_bytes, cases=((1, 2, 4), (2, 3, 5), (3, 2, 6), (4, 3, 8), (5, 2, 5), (8, 4, 16)), seed=0):
    rng = np.random.default_rng(seed)
    for T, M, H in cases:
        X = rng.integers(-2, 3, size=(T, M, 2)).astype(np.float64)
        W = rng.integers(-2, 3, size=(T, 2, H)).astype(np.float64)
        for trial in range(4):
            mask = (rng.random(H) < (trial + 1) / 4).astype(np.uint8)
            n_ch = int(mask.sum())
            sent = []
            simulate_devices(X.tolist(), W.tolist(), mask.tolist(), sent=sent)
            assert len(sent) == T
            for esz in (2, 4):
                got = float(ring_bytes(T, M, n_ch, esz))
                mean = float(np.mean(sent)) * esz
                assert abs(got - mean) <= 1e-9 * max(1.0, mean), (T, M, H, n_ch, esz, got, mean)
                if (M * n_ch) % T == 0:
                    assert all(s * esz == got for s in sent), (T, M, n_ch, sent, got)
