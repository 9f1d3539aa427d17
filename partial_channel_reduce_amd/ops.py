"""Python binding of libcaat_pcr.so (C ABI in include/caat_pcr.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  If the
library is not built, every call raises; there is no fallback path.

Tensors: bf16 tensors are torch.bfloat16, the mask is torch.uint8 [H]
(nonzero = channel in the sync set S), all on the same GPU and contiguous.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import LIBPATH

CAAT_OK = 0
CAAT_F32 = 0
CAAT_BF16 = 1
STATUS_NAMES = {
    0: "CAAT_OK",
    1: "CAAT_ERR_NULL",
    2: "CAAT_ERR_DIM",
    3: "CAAT_ERR_ALIGN",
    4: "CAAT_ERR_ALIAS",
    5: "CAAT_ERR_DTYPE",
    6: "CAAT_ERR_WORKSPACE",
    7: "CAAT_ERR_LAUNCH",
}

# (name, restype, argtypes) for every symbol the header declares.
_P, _I, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = [
    ("caat_abi_version", _I, []),
    ("caat_status_string", ctypes.c_char_p, [_I]),
    ("caat_rowpar_pcr_fwd", _I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _S, _P]),
    ("caat_rowpar_pcr_fwd_workspace_bytes", _S, [_I, _I, _I, _I]),
    ("caat_rowpar_pcr_fwd_noalloc", _I, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    ("caat_pcr_bwd", _I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _S, _P]),
    ("caat_pcr_bwd_workspace_bytes", _S, [_I, _I, _I, _I]),
    ("caat_colpar_fwd", _I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    ("caat_colpar_bwd", _I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    ("caat_residual_rmsnorm", _I, [_P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_float, _P]),
    ("caat_partial_channel_reduce", _I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    ("caat_partial_channel_reduce_residual_rmsnorm", _I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_float, _P]),
]


class CaatError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().caat_status_string(status).decode() if _LIB is not None else ""
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


_LIB = None
_LOCK = threading.Lock()


def lib(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    with _LOCK:
        p = path or LIBPATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is not built; run `python -m partial_channel_reduce_amd.build` "
                "(the HIP library is required; there is no CPU path)"
            )
        L = ctypes.CDLL(p)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _LIB = L
        return L


def _check(status: int, where: str):
    if status != CAAT_OK:
        raise CaatError(status, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _require(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd_workspace_bytes(T: int, M: int, Kr: int, H: int) -> int:
    return int(lib().caat_rowpar_pcr_fwd_workspace_bytes(T, M, Kr, H))


def bwd_workspace_bytes(T: int, M: int, Kr: int, H: int) -> int:
    return int(lib().caat_pcr_bwd_workspace_bytes(T, M, Kr, H))


def rowpar_pcr_fwd(X: torch.Tensor, W: torch.Tensor, mask: torch.Tensor, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """out[T,M,H] = partial channel-reduce of X[t] @ W[t] (see caat_pcr.h).

    A caller-supplied `workspace` (fwd_workspace_bytes of it; shapes served by
    the decode or split kernels need one) must be zeroed once before its first
    use; the library leaves its counters zero."""
    _require(X, "X", torch.bfloat16, 3)
    dev = X.device
    _require(W, "W", torch.bfloat16, 3, dev)
    _require(mask, "mask", torch.uint8, 1, dev)
    T, M, Kr = X.shape
    H = W.shape[2]
    if W.shape[0] != T or W.shape[1] != Kr or mask.shape[0] != H:
        raise ValueError(f"shape mismatch: X{tuple(X.shape)} W{tuple(W.shape)} mask{tuple(mask.shape)}")
    if out is None:
        out = torch.empty((T, M, H), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, 3, dev)
    if tuple(out.shape) != (T, M, H):
        raise ValueError(f"out must be {(T, M, H)}, got {tuple(out.shape)}")
    need = fwd_workspace_bytes(T, M, Kr, H)
    if workspace is None and need > 0:
        # the arrival counters at its head must start at zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().caat_rowpar_pcr_fwd(_ptr(X), _ptr(W), _ptr(mask), _ptr(out), T, M, Kr, H, _ptr(workspace), ws_bytes,
                                   _stream(dev))
    _check(st, "caat_rowpar_pcr_fwd")
    return out


def rowpar_pcr_fwd_noalloc(X: torch.Tensor, W: torch.Tensor, mask: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """rowpar_pcr_fwd into a caller-provided `out`, with no workspace: the
    library's per-GPU scratch serves the decode and split paths where their
    workspace fits it (see caat_pcr.h).  Calls that may overlap on one GPU
    must be serialised by the caller."""
    _require(X, "X", torch.bfloat16, 3)
    dev = X.device
    _require(W, "W", torch.bfloat16, 3, dev)
    _require(mask, "mask", torch.uint8, 1, dev)
    _require(out, "out", torch.bfloat16, 3, dev)
    T, M, Kr = X.shape
    H = W.shape[2]
    if W.shape[0] != T or W.shape[1] != Kr or mask.shape[0] != H or tuple(out.shape) != (T, M, H):
        raise ValueError(f"shape mismatch: X{tuple(X.shape)} W{tuple(W.shape)} mask{tuple(mask.shape)} "
                         f"out{tuple(out.shape)}")
    st = lib().caat_rowpar_pcr_fwd_noalloc(_ptr(X), _ptr(W), _ptr(mask), _ptr(out), T, M, Kr, H, _stream(dev))
    _check(st, "caat_rowpar_pcr_fwd_noalloc")
    return out


def pcr_bwd(dZ: torch.Tensor, X: torch.Tensor, W: torch.Tensor, mask: torch.Tensor,
            dX: torch.Tensor | None = None, dW: torch.Tensor | None = None,
            need_dx: bool = True, need_dw: bool = True, workspace: torch.Tensor | None = None):
    """(dX[T,M,Kr], dW[T,Kr,H]) for incoming per-rank gradients dZ[T,M,H]."""
    _require(dZ, "dZ", torch.bfloat16, 3)
    dev = dZ.device
    _require(X, "X", torch.bfloat16, 3, dev)
    _require(W, "W", torch.bfloat16, 3, dev)
    _require(mask, "mask", torch.uint8, 1, dev)
    T, M, H = dZ.shape
    Kr = X.shape[2]
    if tuple(X.shape) != (T, M, Kr) or tuple(W.shape) != (T, Kr, H) or mask.shape[0] != H:
        raise ValueError(f"shape mismatch: dZ{tuple(dZ.shape)} X{tuple(X.shape)} W{tuple(W.shape)}")
    if need_dx and dX is None:
        dX = torch.empty((T, M, Kr), dtype=torch.bfloat16, device=dev)
    if need_dw and dW is None:
        dW = torch.empty((T, Kr, H), dtype=torch.bfloat16, device=dev)
    if dX is not None:
        _require(dX, "dX", torch.bfloat16, 3, dev)
    if dW is not None:
        _require(dW, "dW", torch.bfloat16, 3, dev)
    need = bwd_workspace_bytes(T, M, Kr, H)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().caat_pcr_bwd(_ptr(dZ), _ptr(X), _ptr(W), _ptr(mask), _ptr(dX), _ptr(dW), T, M, Kr, H,
                            _ptr(workspace), ws_bytes, _stream(dev))
    _check(st, "caat_pcr_bwd")
    return dX, dW


def partial_channel_reduce(Y: torch.Tensor, mask: torch.Tensor, out: torch.Tensor | None = None,
                           inplace: bool = False) -> torch.Tensor:
    """The reduce alone on per-rank Y[T,M,H] (float32 or bfloat16)."""
    if Y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("Y must be float32 or bfloat16")
    _require(Y, "Y", Y.dtype, 3)
    dev = Y.device
    _require(mask, "mask", torch.uint8, 1, dev)
    T, M, H = Y.shape
    if mask.shape[0] != H:
        raise ValueError("mask length must equal H")
    if inplace:
        out = Y
    elif out is None:
        out = torch.empty_like(Y)
    _require(out, "out", Y.dtype, 3, dev)
    if out.shape != Y.shape:
        raise ValueError("out must have Y's shape")
    dt = CAAT_F32 if Y.dtype == torch.float32 else CAAT_BF16
    st = lib().caat_partial_channel_reduce(_ptr(Y), _ptr(mask), _ptr(out), T, M, H, dt, _stream(dev))
    _check(st, "caat_partial_channel_reduce")
    return out


def colpar_fwd(A: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """U[T,M,N] = A[t] @ W[t] for per-rank inputs A[T,M,K] (see caat_pcr.h)."""
    _require(A, "A", torch.bfloat16, 3)
    dev = A.device
    _require(W, "W", torch.bfloat16, 3, dev)
    T, M, K = A.shape
    N = W.shape[2]
    if W.shape[0] != T or W.shape[1] != K:
        raise ValueError(f"shape mismatch: A{tuple(A.shape)} W{tuple(W.shape)}")
    if out is None:
        out = torch.empty((T, M, N), dtype=torch.bfloat16, device=dev)
    _require(out, "out", torch.bfloat16, 3, dev)
    if tuple(out.shape) != (T, M, N):
        raise ValueError(f"out must be {(T, M, N)}, got {tuple(out.shape)}")
    st = lib().caat_colpar_fwd(_ptr(A), _ptr(W), _ptr(out), T, M, K, N, _stream(dev))
    _check(st, "caat_colpar_fwd")
    return out


def colpar_bwd(dU: torch.Tensor, A: torch.Tensor, W: torch.Tensor, dA: torch.Tensor | None = None,
               dW: torch.Tensor | None = None, need_da: bool = True, need_dw: bool = True):
    """(dA[T,M,K], dW[T,K,N]) for incoming per-rank gradients dU[T,M,N]."""
    _require(dU, "dU", torch.bfloat16, 3)
    dev = dU.device
    _require(A, "A", torch.bfloat16, 3, dev)
    _require(W, "W", torch.bfloat16, 3, dev)
    T, M, N = dU.shape
    K = A.shape[2]
    if tuple(A.shape) != (T, M, K) or tuple(W.shape) != (T, K, N):
        raise ValueError(f"shape mismatch: dU{tuple(dU.shape)} A{tuple(A.shape)} W{tuple(W.shape)}")
    if need_da and dA is None:
        dA = torch.empty((T, M, K), dtype=torch.bfloat16, device=dev)
    if need_dw and dW is None:
        dW = torch.empty((T, K, N), dtype=torch.bfloat16, device=dev)
    if dA is not None:
        _require(dA, "dA", torch.bfloat16, 3, dev)
    if dW is not None:
        _require(dW, "dW", torch.bfloat16, 3, dev)
    st = lib().caat_colpar_bwd(_ptr(dU), _ptr(A), _ptr(W), _ptr(dA), _ptr(dW), T, M, K, N, _stream(dev))
    _check(st, "caat_colpar_bwd")
    return dA, dW


def residual_rmsnorm(Z: torch.Tensor, R: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5,
                     r_out: torch.Tensor | None = None, n_out: torch.Tensor | None = None, inplace: bool = False):
    """(Rn, N): per-rank residual update Rn = R + Z and its RMS normalisation
    (see caat_pcr.h).  inplace=True writes Rn into R."""
    _require(Z, "Z", torch.bfloat16, 3)
    dev = Z.device
    _require(R, "R", torch.bfloat16, 3, dev)
    _require(gamma, "gamma", torch.bfloat16, 1, dev)
    T, M, H = Z.shape
    if tuple(R.shape) != (T, M, H) or gamma.shape[0] != H:
        raise ValueError(f"shape mismatch: Z{tuple(Z.shape)} R{tuple(R.shape)} gamma{tuple(gamma.shape)}")
    if inplace:
        r_out = R
    elif r_out is None:
        r_out = torch.empty_like(Z)
    if n_out is None:
        n_out = torch.empty_like(Z)
    _require(r_out, "r_out", torch.bfloat16, 3, dev)
    _require(n_out, "n_out", torch.bfloat16, 3, dev)
    if tuple(r_out.shape) != (T, M, H) or tuple(n_out.shape) != (T, M, H):
        raise ValueError("outputs must have Z's shape")
    st = lib().caat_residual_rmsnorm(_ptr(Z), _ptr(R), _ptr(gamma), _ptr(r_out), _ptr(n_out), T, M, H, float(eps),
                                     _stream(dev))
    _check(st, "caat_residual_rmsnorm")
    return r_out, n_out


def reduce_residual_rmsnorm(Y: torch.Tensor, mask: torch.Tensor, R: torch.Tensor, gamma: torch.Tensor,
                            eps: float = 1e-5, r_out: torch.Tensor | None = None, n_out: torch.Tensor | None = None,
                            inplace: bool = False):
    """(Rout, N): the partial channel-reduce of bf16 Y[T,M,H] with the residual
    update and RMS normalisation in its epilogue (see caat_pcr.h); Z is not
    materialised.  inplace=True writes Rout into R."""
    _require(Y, "Y", torch.bfloat16, 3)
    dev = Y.device
    _require(mask, "mask", torch.uint8, 1, dev)
    _require(R, "R", torch.bfloat16, 3, dev)
    _require(gamma, "gamma", torch.bfloat16, 1, dev)
    T, M, H = Y.shape
    if tuple(R.shape) != (T, M, H) or gamma.shape[0] != H or mask.shape[0] != H:
        raise ValueError(f"shape mismatch: Y{tuple(Y.shape)} R{tuple(R.shape)} gamma{tuple(gamma.shape)} "
                         f"mask{tuple(mask.shape)}")
    if inplace:
        r_out = R
    elif r_out is None:
        r_out = torch.empty_like(Y)
    if n_out is None:
        n_out = torch.empty_like(Y)
    _require(r_out, "r_out", torch.bfloat16, 3, dev)
    _require(n_out, "n_out", torch.bfloat16, 3, dev)
    if tuple(r_out.shape) != (T, M, H) or tuple(n_out.shape) != (T, M, H):
        raise ValueError("outputs must have Y's shape")
    st = lib().caat_partial_channel_reduce_residual_rmsnorm(_ptr(Y), _ptr(mask), _ptr(R), _ptr(gamma), _ptr(r_out),
                                                            _ptr(n_out), T, M, H, float(eps), _stream(dev))
    _check(st, "caat_partial_channel_reduce_residual_rmsnorm")
    return r_out, n_out
