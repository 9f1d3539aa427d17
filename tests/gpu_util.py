"""Helpers for the GPU parity tests: host<->device bf16 transfer and the
comparison bars.

Tolerances (the bar the parity tests apply):
* bf16 outputs: every element within 2e-2 * rms(ref) + half a bf16 ulp of
  |ref|, asserted twice: with rms over the whole compared tensor (the stated
  bar), and with rms over the element's channel class (synced channels and
  local channels separately: synced values are about sqrt(T) larger, so the
  local class gets its own, tighter bound).  Half an ulp is the rounding any
  bf16 result carries; without it a correctly rounded output at the largest
  magnitudes would already exceed 2e-2 * rms.  The strict ratio
  max|err| / rms(ref), without the half-ulp term, is reported beside it.
* backward outputs (dX, dW) may also differ by the exact effect of one
  documented rounding: the reduced gradient G that feeds the bf16 products
  holds its synced channels as bf16 (the fp32 sum over ranks in ascending
  order, rounded once), while the oracle uses the exact sum.  The allowance
  is |X^T (G_bf16 - G)| for dW and |(G_bf16 - G) W^T| for dX, computed here
  from the inputs (zero when no channel is synced); it matters only for
  short contractions, where those few rounding errors do not average out.
* fp32 reduce: max|err| <= 1e-4 * rms(ref), and bitwise equality with a
  float32 emulation of the documented summation order.
* integer-valued inputs, routing, cross-rank identity of synced channels and
  run-to-run determinism: bitwise.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

BF16_TOL = 2e-2
F32_TOL = 1e-4


def dev():
    return torch.device("cuda", 0)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(bf16_bits(t))


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers at |ref| (bf16 keeps 8 significant bits)."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    _, e = np.frexp(a)  # a = m * 2**e, m in [0.5, 1)
    h = np.ldexp(1.0, e - 9)
    return np.where(a > 0, h, 0.0)


def rms(a: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def check_bf16(got: np.ndarray, ref: np.ndarray, classes: np.ndarray | None = None, what: str = "",
               extra: np.ndarray | None = None):
    """Assert the bf16 bar; `classes` is a boolean array broadcastable to ref
    splitting elements into two channel classes (None = one class); `extra`
    (broadcastable to ref) is the backward's G-rounding allowance."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if extra is not None:
        err = np.maximum(err - np.broadcast_to(np.asarray(extra, dtype=np.float64), err.shape), 0.0)
    report = {"strict_max_over_rms": float(err.max() / max(rms(ref), 1e-300)) if err.size else 0.0}
    if err.size:
        r_all = rms(ref)
        excess = err - (BF16_TOL * r_all + half_ulp_bf16(ref))
        worst = int(np.argmax(excess))
        assert excess.flat[worst] <= 0.0, (
            f"{what}: whole tensor: |err| {err.flat[worst]:.4g} > 2e-2 * rms {r_all:.4g} + half ulp "
            f"(ref {ref.flat[worst]:.5g}, got {got.flat[worst]:.5g})"
        )
    if classes is None:
        groups = [np.ones(ref.shape, dtype=bool)]
    else:
        cl = np.broadcast_to(classes, ref.shape)
        groups = [cl, ~cl]
    for gi, g in enumerate(groups):
        if not g.any():
            continue
        r = rms(ref[g])
        bound = BF16_TOL * r + half_ulp_bf16(ref[g])
        excess = err[g] - bound
        worst = int(np.argmax(excess))
        assert excess[worst] <= 0.0, (
            f"{what}: class {gi}: |err| {err[g][worst]:.4g} > bound {bound[worst]:.4g} "
            f"(ref {ref[g][worst]:.5g}, got {got[g][worst]:.5g}, rms {r:.4g})"
        )
        report[f"class{gi}_max_err_over_rms"] = float(err[g].max() / max(r, 1e-300))
    return report


def check_f32(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    r = rms(ref)
    assert err <= F32_TOL * r, f"{what}: max|err| {err:.3g} > {F32_TOL} * rms {r:.3g}"
    return err / max(r, 1e-300)


def f32_sequential_reduce(Y: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """float32 emulation of the kernel's documented order for the synced
    channels: acc = Y[0]; acc += Y[1]; ... (each add rounded to fp32)."""
    S = np.asarray(mask) != 0
    acc = Y[0].astype(np.float32).copy()
    for t in range(1, Y.shape[0]):
        acc = (acc + Y[t].astype(np.float32)).astype(np.float32)
    out = Y.astype(np.float32).copy()
    out[:, :, S] = acc[None][:, :, S]
    return out


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


class Bf16Bar:
    """check_bf16 for a tensor compared block by block: the whole-tensor and
    per-class rms are only known once every block is in, so each block
    contributes the largest excess over half an ulp and its sums of squares,
    and finish() asserts both bars."""

    def __init__(self, what: str = ""):
        self.what = what
        self.sumsq = [0.0, 0.0, 0.0]  # whole, class 0, class 1
        self.count = [0, 0, 0]
        self.excess = [-np.inf, -np.inf, -np.inf]
        self.max_err = 0.0

    def add(self, got, ref, classes=None, extra=None):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        assert np.all(np.isfinite(got)), f"{self.what}: non-finite output"
        d = np.abs(got - ref) - half_ulp_bf16(ref)
        if extra is not None:
            d = d - np.broadcast_to(np.asarray(extra, dtype=np.float64), d.shape)
        self.max_err = max(self.max_err, float(np.max(np.abs(got - ref)))) if ref.size else self.max_err
        groups = [np.ones(ref.shape, dtype=bool)]
        if classes is not None:
            cl = np.broadcast_to(classes, ref.shape)
            groups += [cl, ~cl]
        for gi, g in enumerate(groups):
            if g.any():
                self.sumsq[gi] += float(np.sum(ref[g] * ref[g]))
                self.count[gi] += int(g.sum())
                self.excess[gi] = max(self.excess[gi], float(d[g].max()))

    def finish(self):
        report = {}
        for gi, name in enumerate(("whole", "class0", "class1")):
            if self.count[gi] == 0:
                continue
            r = float(np.sqrt(self.sumsq[gi] / self.count[gi]))
            assert self.excess[gi] <= BF16_TOL * r, (
                f"{self.what}: {name}: |err| - half ulp reaches {self.excess[gi]:.4g} > 2e-2 * rms {r:.4g}"
            )
            report[name + "_rms"] = r
        report["strict_max_over_rms"] = self.max_err / max(report.get("whole_rms", 1e-300), 1e-300)
        return report


# ---- the backward's G-rounding allowance ------------------------------------

def g_rounding_shift(dZ: np.ndarray, mask: np.ndarray, rows=None) -> np.ndarray:
    """G_bf16 - G on the synced channels (zero elsewhere) for token rows
    `rows` (all when None): G_bf16 is the fp32 sum of the ranks' bf16
    gradients in ascending rank order, rounded once to bf16; G is the exact
    sum.  The same for every rank.  -> [len(rows), H] float64."""
    dZ = np.asarray(dZ)
    sel = slice(None) if rows is None else np.asarray(rows)
    S = np.asarray(mask) != 0
    acc = oracle.bf16_to_f64(dZ[0][sel]).astype(np.float32)
    exact = oracle.bf16_to_f64(dZ[0][sel])
    for t in range(1, dZ.shape[0]):
        zt = oracle.bf16_to_f64(dZ[t][sel])
        acc = (acc + zt.astype(np.float32)).astype(np.float32)
        exact = exact + zt
    gb = oracle.bf16_to_f64(f32_to_bf16_bits_rne(acc))
    return np.where(S[None, :], gb - exact, 0.0)


def bwd_g_allowance(dZ, X, W, mask):
    """Whole-tensor allowances (dX [T,M,Kr], dW [T,Kr,H]) for small cases."""
    D = g_rounding_shift(dZ, mask)
    Xf = oracle.bf16_to_f64(X)
    Wf = oracle.bf16_to_f64(W)
    T = Xf.shape[0]
    return (np.stack([np.abs(D @ Wf[t].T) for t in range(T)]), np.stack([np.abs(Xf[t].T @ D) for t in range(T)]))


def dx_rows_g_allowance(dZ, W, mask, ts, ms):
    """Allowance for whole dX rows at sampled (t, m) -> [n, Kr]."""
    D = g_rounding_shift(dZ, mask, ms)
    out = np.empty((len(ts), np.asarray(W).shape[1]))
    for t in sorted(set(int(v) for v in ts)):
        idx = np.flatnonzero(np.asarray(ts) == t)
        out[idx] = np.abs(D[idx] @ oracle.bf16_to_f64(np.asarray(W)[t]).T)
    return out


def dw_rows_g_allowance(dZ, X, mask, ts, ks, block: int = 2048):
    """Allowance for whole dW rows at sampled (t, k) -> [n, H] (the signed
    sum over every token, taken block by block, then its magnitude)."""
    dZ = np.asarray(dZ)
    X = np.asarray(X)
    M, H = dZ.shape[1], dZ.shape[2]
    acc = np.zeros((len(ts), H))
    for m0 in range(0, M, block):
        rows = np.arange(m0, min(M, m0 + block))
        D = g_rounding_shift(dZ, mask, rows)
        for t in sorted(set(int(v) for v in ts)):
            idx = np.flatnonzero(np.asarray(ts) == t)
            Xk = oracle.bf16_to_f64(X[t][rows][:, np.asarray(ks)[idx]])
            acc[idx] += Xk.T @ D
    return np.abs(acc)
