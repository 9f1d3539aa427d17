"""Seeded synthetic inputs for the row-parallel layer and its partial channel-reduce.

This module is the only code shared by the HIP path's callers (tests, bench)
and the CPU oracle's callers.  It draws numbers and builds channel masks; it
holds none of the method's arithmetic (no product, no sum, no reduce).

Workload recipe (the pages train Llama2-7B, TinyLlama-1.1B and a 130M model
with tensor parallelism 8 and a sync fraction p = 0.5; they print no data, so
Gaussian stand-ins of the same shapes are used):

* activations   X[T, M, Kr]  ~ N(0, 1)     rounded to bf16 (round-to-nearest-even)
* weights       W[T, Kr, H]  ~ N(0, 0.02)  rounded to bf16
* out-gradient  dZ[T, M, H]  ~ N(0, 1)     rounded to bf16, independent per rank
* reduce input  Y[T, M, H]   ~ N(0, 1)     float32 (or bf16)
* channel mask  mask[H]      uint8, 1 = channel in the sync set S, exactly
  round(p*H) ones, laid out as a prefix, evenly strided, or a seeded random
  subset.

bf16 tensors are carried as their raw uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

MASK_KINDS = ("prefix", "strided", "random")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the uint16 bits.

    Inputs are finite draws; NaN/Inf are not produced by this module.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    # Draw in float32 in bounded slabs so large shapes do not need a float64 copy.
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    n = flat.size
    step = 1 << 24
    for s in range(0, n, step):
        e = min(n, s + step)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        flat[s:e] = f32_to_bf16_bits(v)
    return out


def sync_count(H: int, p: float) -> int:
    """|S| = round(p*H), half rounded up (every workload here has p*H integral)."""
    if not 0.0 <= p <= 1.0:
        raise ValueError("p must lie in [0, 1]")
    return int(np.floor(p * H + 0.5))


def make_mask(H: int, p: float, kind: str = "random", seed: int = 0) -> np.ndarray:
    """uint8[H] channel mask with exactly round(p*H) synced channels.

    prefix : channels 0 .. |S|-1
    strided: channels floor(i*H/|S|), i = 0 .. |S|-1 (p = 0.5 gives the even channels)
    random : the first |S| entries of a seeded permutation of 0 .. H-1
    """
    n = sync_count(H, p)
    mask = np.zeros(H, dtype=np.uint8)
    if n == 0:
        return mask
    if kind == "prefix":
        mask[:n] = 1
    elif kind == "strided":
        idx = (np.arange(n, dtype=np.int64) * H) // n
        mask[idx] = 1
    elif kind == "random":
        rng = np.random.default_rng(seed + 10_000)
        mask[rng.permutation(H)[:n]] = 1
    else:
        raise ValueError(f"unknown mask kind {kind!r}; expected one of {MASK_KINDS}")
    return mask


def make_fwd_inputs(T: int, M: int, Kr: int, H: int, seed: int = 0):
    """(X bits [T,M,Kr], W bits [T,Kr,H]) as uint16 bf16 patterns."""
    rng = np.random.default_rng(seed)
    X = _normal_bf16(rng, (T, M, Kr), 1.0)
    W = _normal_bf16(rng, (T, Kr, H), 0.02)
    return X, W


def make_grad(T: int, M: int, H: int, seed: int = 0) -> np.ndarray:
    """dZ bits [T,M,H]: independent N(0,1) per rank, bf16."""
    rng = np.random.default_rng(seed + 20_000)
    return _normal_bf16(rng, (T, M, H), 1.0)


def make_reduce_input(T: int, M: int, H: int, seed: int = 0, dtype: str = "f32") -> np.ndarray:
    """Y[T,M,H] ~ N(0,1): float32 array, or uint16 bf16 bits when dtype == 'bf16'."""
    rng = np.random.default_rng(seed + 30_000)
    if dtype == "bf16":
        return _normal_bf16(rng, (T, M, H), 1.0)
    if dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return rng.standard_normal((T, M, H), dtype=np.float32)


def make_integer_fwd_inputs(T: int, M: int, Kr: int, H: int, seed: int = 0, lo: int = -2, hi: int = 2,
                            x_zero_frac: float = 0.0):
    """Small-integer X, W (exact in bf16).  With few enough nonzero products
    every partial sum stays an integer below 2**8, so any summation order gives
    the same bits; x_zero_frac zeroes that fraction of X to keep long
    contractions in range."""
    rng = np.random.default_rng(seed + 40_000)
    X = rng.integers(lo, hi + 1, size=(T, M, Kr)).astype(np.float32)
    if x_zero_frac > 0:
        X *= (rng.random((T, M, Kr)) >= x_zero_frac).astype(np.float32)
    W = rng.integers(lo, hi + 1, size=(T, Kr, H)).astype(np.float32)
    return f32_to_bf16_bits(X), f32_to_bf16_bits(W)


def make_rank_tag_inputs(T: int, M: int, Kr: int, H: int, scale_choices=(1, 2), seed: int = 0):
    """Rank-tag routing inputs.

    Row m of X_t is one-hot at k = m % Kr, and W_t[k, c] = 2**t * s_c with
    s_c in scale_choices drawn per channel.  Then Y_t[m, c] = 2**t * s_c exactly,
    so a local output names the rank it came from and a synced output equals
    s_c * (2**T - 1).  Needs T <= 8 for the synced value to stay exact in bf16.
    """
    rng = np.random.default_rng(seed + 50_000)
    s = rng.choice(np.asarray(scale_choices, dtype=np.float32), size=H)
    X = np.zeros((T, M, Kr), dtype=np.float32)
    X[:, np.arange(M), np.arange(M) % Kr] = 1.0
    W = np.empty((T, Kr, H), dtype=np.float32)
    for t in range(T):
        W[t] = (2.0 ** t) * s[None, :]
    return f32_to_bf16_bits(X), f32_to_bf16_bits(W), s
