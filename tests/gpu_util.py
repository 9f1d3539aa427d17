"""Helpers for the GPU parity tests: host<->device bf16 transfer and the
comparison bars.

Tolerances (the bar the parity tests apply):
* bf16 outputs: every element within 2e-2 * rms(ref) + half a bf16 ulp of
  |ref|, with rms taken over the element's channel class (synced channels and
  local channels separately, since synced values are about sqrt(T) larger).
  Half an ulp is the rounding any bf16 result carries; without it a correctly
  rounded output at the largest magnitudes of a class would already exceed
  2e-2 * rms.  The strict whole-tensor ratio max|err| / rms(ref) is reported
  beside it.
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


def check_bf16(got: np.ndarray, ref: np.ndarray, classes: np.ndarray | None = None, what: str = ""):
    """Assert the bf16 bar; `classes` is a boolean array broadcastable to ref
    splitting elements into two channel classes (None = one class)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    report = {"strict_max_over_rms": float(err.max() / max(rms(ref), 1e-300)) if err.size else 0.0}
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
