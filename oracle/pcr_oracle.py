"""CPU oracle for the partial channel-reduce hot path (TEST INFRASTRUCTURE ONLY).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path never calls it, and it shares no code
with the HIP library.

Source: "Tensor-Parallelism with Partially Synchronized Activations"
(Lamprecht, Karnieli, Hanani, Giladi, Soudry; NeurIPS 2025, arXiv 2506.19645),
Introduction.  In tensor parallelism each of the T devices holds a partial
activation after its row-parallel linear layer, and an all-reduce normally
sums those partials so that every device holds the same tensor.  The
partial channel-reduce sums only a subset S of the hidden-dimension channels;
every other channel keeps the device's own partial, so the devices'
activations differ afterwards.  With S empty the model behaves as an ensemble
of independent devices; with S all channels it is the ordinary (vanilla)
transformer.  The Introduction also requires the backward pass to agree with
this forward (the forward/backward mismatch it warns about).

Notation: T ranks, M tokens, Kr = K/T input features per rank, H hidden
channels.  X[T,M,Kr], W[T,Kr,H], mask[H] (nonzero = channel in S).

Everything is computed in float64 from the exact values of the bf16 inputs,
with no blocking, fusion or reordering beyond what the definition states.
Readings of points the pages leave open (the reduce is a SUM; local channels
are not rescaled; the layer has no bias; forward and backward use the same
S; the incoming gradient differs per rank) are listed with the design notes.

The layer that consumes the reduce's output, a column-parallel product, now
takes a different input on every rank; colpar_fwd / colpar_bwd define it and
its exact backward, whose input gradient stays on its rank.

Every function here is pinned by the CPU tests to something other than
itself: a message-passing simulation of the restricted all-reduce on integer
inputs, the un-sharded layer (all channels synced), the per-rank layer (no
channel synced), the adjoint identity and finite differences (of the layer
alone and of the two-layer chain with the column-parallel product).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64",
    "sync_channels",
    "partial_channel_reduce",
    "rowpar_partials",
    "rowpar_pcr_fwd",
    "pcr_bwd",
    "colpar_fwd",
    "colpar_bwd",
    "residual_rmsnorm",
    "fwd_at",
    "bwd_dx_at",
    "bwd_dw_at",
    "fwd_rows",
    "bwd_dx_rows",
    "bwd_dw_rows",
    "synced_elements",
    "ring_allreduce_bytes_per_rank",
]


def bf16_to_f64(a) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64; float arrays pass through."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sync_channels(mask) -> np.ndarray:
    """Indices of the channels in the sync set S (mask entry nonzero)."""
    return np.flatnonzero(np.asarray(mask) != 0)


def partial_channel_reduce(Y, mask) -> np.ndarray:
    """The partial channel-reduce of per-rank activations Y[T,M,H].

    Introduction: only the channels in S are reduced (summed over the T
    ranks); each rank keeps its own value in the other channels.
        Z[t][:, c] = sum_{t'} Y[t'][:, c]   for c in S
        Z[t][:, c] = Y[t][:, c]             for c not in S
    """
    Y = bf16_to_f64(Y)
    T = Y.shape[0]
    S = sync_channels(mask)
    Z = Y.copy()
    total = np.zeros(Y.shape[1:], dtype=np.float64)
    for t in range(T):
        total += Y[t]
    for t in range(T):
        Z[t][:, S] = total[:, S]
    return Z


def rowpar_partials(X, W) -> np.ndarray:
    """Each rank's row-parallel partial product Y[t] = X[t] @ W[t]  -> [T,M,H]."""
    X = bf16_to_f64(X)
    W = bf16_to_f64(W)
    T = X.shape[0]
    return np.stack([X[t] @ W[t] for t in range(T)])


def rowpar_pcr_fwd(X, W, mask) -> np.ndarray:
    """Row-parallel linear layer followed by the partial channel-reduce -> Z[T,M,H]."""
    return partial_channel_reduce(rowpar_partials(X, W), mask)


def pcr_bwd(dZ, X, W, mask):
    """Exact backward of rowpar_pcr_fwd for incoming per-rank gradients dZ[T,M,H].

    The reduce is linear and self-adjoint: a synced channel's gradient is the
    sum over ranks of the incoming gradients, a local channel's gradient
    passes through.  Then, per rank, G = that gradient and
        dX[t] = G[t] @ W[t].T      [M,Kr]
        dW[t] = X[t].T @ G[t]      [Kr,H]
    """
    G = partial_channel_reduce(dZ, mask)
    X = bf16_to_f64(X)
    W = bf16_to_f64(W)
    T = X.shape[0]
    dX = np.stack([G[t] @ W[t].T for t in range(T)])
    dW = np.stack([X[t].T @ G[t] for t in range(T)])
    return dX, dW


def colpar_fwd(A, W) -> np.ndarray:
    """Column-parallel product on per-rank inputs: U[t] = A[t] @ W[t] -> [T,M,N].

    After the partial channel-reduce each rank holds its own activation, so
    the next layer's column-parallel product multiplies rank t's activation
    A[t] [M,K] by rank t's column slice W[t] [K,N]."""
    A = bf16_to_f64(A)
    W = bf16_to_f64(W)
    return np.stack([A[t] @ W[t] for t in range(A.shape[0])])


def colpar_bwd(dU, A, W):
    """Exact backward of colpar_fwd for per-rank incoming gradients dU[T,M,N]:
        dA[t] = dU[t] @ W[t].T     [M,K]
        dW[t] = A[t].T @ dU[t]     [K,N]
    A[t] is rank t's own input, so its gradient stays with rank t (no sum over
    ranks here); in the two-layer chain the only cross-rank sum is pcr_bwd's,
    over the synced channels."""
    dU = bf16_to_f64(dU)
    A = bf16_to_f64(A)
    W = bf16_to_f64(W)
    T = A.shape[0]
    dA = np.stack([dU[t] @ W[t].T for t in range(T)])
    dW = np.stack([A[t].T @ dU[t] for t in range(T)])
    return dA, dW


def residual_rmsnorm(Z, R, gamma, eps: float):
    """Per-rank residual update and RMS normalisation of the result.

    The partial channel-reduce leaves each rank with its own activation Z[t]
    (Introduction), which is added to that rank's own residual stream R[t];
    the Llama-family blocks the pages train then RMS-normalise it:
        Rn[t, m, :] = R[t, m, :] + Z[t, m, :]
        N[t, m, :]  = Rn[t, m, :] / sqrt(mean_c Rn[t, m, c]**2 + eps) * gamma
    -> (Rn, N), both [T,M,H]; gamma [H] is the same on every rank."""
    Rn = bf16_to_f64(R) + bf16_to_f64(Z)
    g = bf16_to_f64(gamma)
    ms = np.mean(Rn * Rn, axis=-1, keepdims=True)
    return Rn, Rn / np.sqrt(ms + eps) * g


# ---------------------------------------------------------------------------
# Element-wise evaluation, for sampled checks at sizes where the full oracle
# would not finish.  Each takes index arrays and evaluates the same definition
# one output element at a time (the inputs may be bf16 bit arrays; only the
# rows/columns an element needs are upcast).
# ---------------------------------------------------------------------------

def _rows(A, t, m):
    return bf16_to_f64(np.asarray(A)[t, m, :])


def _cols(A, t, c):
    return bf16_to_f64(np.asarray(A)[t, :, c])


def fwd_at(X, W, mask, ts, ms, cs) -> np.ndarray:
    """Z[t,m,c] for each (t,m,c) in zip(ts, ms, cs)."""
    mask = np.asarray(mask)
    T = np.asarray(X).shape[0]
    out = np.empty(len(ts), dtype=np.float64)
    for i, (t, m, c) in enumerate(zip(ts, ms, cs)):
        if mask[c] != 0:
            out[i] = sum(float(_rows(X, u, m) @ _cols(W, u, c)) for u in range(T))
        else:
            out[i] = float(_rows(X, t, m) @ _cols(W, t, c))
    return out


def _g_row(dZ, mask, t, m) -> np.ndarray:
    """Row m of rank t's reduced gradient G[t] (all H channels)."""
    dZ = np.asarray(dZ)
    T = dZ.shape[0]
    S = np.asarray(mask) != 0
    own = bf16_to_f64(dZ[t, m, :])
    total = np.zeros_like(own)
    for u in range(T):
        total += bf16_to_f64(dZ[u, m, :])
    return np.where(S, total, own)


def _g_col(dZ, mask, t, c) -> np.ndarray:
    """Column c of rank t's reduced gradient G[t] (all M tokens)."""
    dZ = np.asarray(dZ)
    T = dZ.shape[0]
    if np.asarray(mask)[c] != 0:
        total = np.zeros(dZ.shape[1], dtype=np.float64)
        for u in range(T):
            total += bf16_to_f64(dZ[u, :, c])
        return total
    return bf16_to_f64(dZ[t, :, c])


def bwd_dx_at(dZ, W, mask, ts, ms, ks) -> np.ndarray:
    """dX[t,m,k] = sum_c G[t,m,c] * W[t,k,c] for each sampled (t,m,k)."""
    out = np.empty(len(ts), dtype=np.float64)
    for i, (t, m, k) in enumerate(zip(ts, ms, ks)):
        out[i] = float(_g_row(dZ, mask, t, m) @ bf16_to_f64(np.asarray(W)[t, k, :]))
    return out


def bwd_dw_at(dZ, X, mask, ts, ks, cs) -> np.ndarray:
    """dW[t,k,c] = sum_m X[t,m,k] * G[t,m,c] for each sampled (t,k,c)."""
    out = np.empty(len(ts), dtype=np.float64)
    for i, (t, k, c) in enumerate(zip(ts, ks, cs)):
        out[i] = float(bf16_to_f64(np.asarray(X)[t, :, k]) @ _g_col(dZ, mask, t, c))
    return out


def fwd_rows(X, W, mask, ts, ms) -> np.ndarray:
    """Whole output rows Z[t,m,:] for each sampled (t,m) -> [n, H]: the sum
    over ranks of X[u][m,:] @ W[u] on the synced channels, rank t's own
    X[t][m,:] @ W[t] elsewhere."""
    X = np.asarray(X)
    W = np.asarray(W)
    T = X.shape[0]
    S = np.asarray(mask) != 0
    ms = np.asarray(ms)
    um = np.unique(ms)
    Y = np.stack([bf16_to_f64(X[u][um, :]) @ bf16_to_f64(W[u]) for u in range(T)])  # [T, len(um), H]
    total = np.zeros(Y.shape[1:], dtype=np.float64)
    for u in range(T):
        total += Y[u]
    pos = np.searchsorted(um, ms)
    out = np.empty((len(ts), W.shape[2]), dtype=np.float64)
    for i, (t, j) in enumerate(zip(ts, pos)):
        out[i] = np.where(S, total[j], Y[int(t), j])
    return out


def bwd_dx_rows(dZ, W, mask, ts, ms) -> np.ndarray:
    """Whole rows of the input gradient: dX[t,m,:] = G[t][m,:] @ W[t].T for
    each sampled (t,m) -> [n, Kr].  G[t][m,:] is rank t's reduced gradient
    row (the synced channels summed over the ranks, its own values
    elsewhere)."""
    out = np.empty((len(ts), np.asarray(W).shape[1]), dtype=np.float64)
    for t in sorted(set(int(v) for v in ts)):
        Wt = bf16_to_f64(np.asarray(W)[t])
        for i in np.flatnonzero(np.asarray(ts) == t):
            out[i] = _g_row(dZ, mask, t, int(ms[i])) @ Wt.T
    return out


def bwd_dw_rows(dZ, X, mask, ts, ks) -> np.ndarray:
    """Whole rows of the weight gradient: dW[t,k,:] = X[t][:,k] @ G[t] for
    each sampled (t,k) -> [n, H], with G[t] rank t's reduced gradient."""
    dZ = np.asarray(dZ)
    X = np.asarray(X)
    T, _, H = dZ.shape
    S = np.asarray(mask) != 0
    total = np.zeros(dZ.shape[1:], dtype=np.float64)
    for u in range(T):
        total += bf16_to_f64(dZ[u])
    out = np.empty((len(ts), H), dtype=np.float64)
    for t in sorted(set(int(v) for v in ts)):
        Gt = np.where(S, total, bf16_to_f64(dZ[t]))
        rows = np.flatnonzero(np.asarray(ts) == t)
        Xk = bf16_to_f64(X[t][:, np.asarray(ks)[rows]])  # [M, n_t]
        out[rows] = Xk.T @ Gt
    return out


# ---------------------------------------------------------------------------
# Communication payload (Abstract and Introduction: reducing only a fraction p
# of the channels cuts the tensor-parallel payload by that fraction; p = 0.5
# gives the 50% cut the pages report).
# ---------------------------------------------------------------------------

def synced_elements(mask, M: int) -> int:
    """Number of activation elements that take part in the reduce: M * |S|."""
    return int(M) * int(len(sync_channels(mask)))


def ring_allreduce_bytes_per_rank(T: int, M: int, n_channels: int, elem_bytes: int) -> float:
    """Bytes each rank sends in a ring all-reduce of an [M, n_channels] tensor:
    a reduce-scatter and an all-gather, each T-1 steps of 1/T of the tensor."""
    if T <= 1:
        return 0.0
    return 2.0 * (T - 1) / T * M * n_channels * elem_bytes
