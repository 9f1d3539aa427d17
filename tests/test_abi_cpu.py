"""CPU: the C-ABI library loads, exports every symbol the header declares, and
rejects invalid arguments on the host before any GPU work (no GPU needed)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from partial_channel_reduce_amd import build as pbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "caat_pcr.h")

OK, NULL, DIM, ALIGN, ALIAS, DTYPE, WS, LAUNCH = range(8)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pbuild.LIBPATH):
        pbuild.build()
    from partial_channel_reduce_amd import ops

    return ops.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(caat_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("caat_rowpar_pcr_fwd", "caat_pcr_bwd", "caat_partial_channel_reduce", "caat_colpar_fwd",
              "caat_colpar_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    from partial_channel_reduce_amd import ops

    declared = header_functions()
    assert sorted(n for n, _, _ in ops.SIGNATURES) == declared
    for n in declared:
        assert hasattr(L, n), n
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", pbuild.LIBPATH], capture_output=True, text=True).stdout
        exported = set(re.findall(r"\sT\s(caat_\w+)", out))
        assert set(declared) <= exported


def test_status_strings(L):
    assert L.caat_abi_version() == 1
    for s in range(8):
        assert L.caat_status_string(s).decode()
    assert L.caat_status_string(99).decode() == "unknown status"


# Fake but well-aligned device addresses: validation never dereferences them.
A = 0x7F0000000000
B = 0x7F0100000000
C = 0x7F0200000000
D = 0x7F0300000000
E = 0x7F0400000000


def fwd(L, X=A, W=B, mask=C, out=D, T=8, M=64, Kr=64, H=64, ws=None, wsb=0):
    return L.caat_rowpar_pcr_fwd(X, W, mask, out, T, M, Kr, H, ws, wsb, None)


def test_fwd_validation(L):
    assert fwd(L, X=None) == NULL
    assert fwd(L, W=None, M=0) == NULL
    assert fwd(L, X=None, out=None, M=0) == OK  # empty tensors may be NULL
    assert fwd(L, mask=None) == NULL
    assert fwd(L, T=0) == DIM
    assert fwd(L, T=65) == DIM
    assert fwd(L, M=-1) == DIM
    assert fwd(L, Kr=12) == DIM
    assert fwd(L, H=100) == DIM
    assert fwd(L, Kr=0) == DIM
    assert fwd(L, X=A + 8) == ALIGN
    assert fwd(L, out=D + 2) == ALIGN
    assert fwd(L, mask=C + 4) == ALIGN
    assert fwd(L, out=A) == ALIAS  # out over X
    assert fwd(L, out=B + 16) == ALIAS  # out over W
    # per-rank slice beyond 32-bit signed byte offsets (2^30 elements)
    assert fwd(L, T=1, M=1 << 20, Kr=4096, H=64) == DIM
    assert fwd(L, T=1, M=1 << 18, Kr=4096, H=64) == DIM
    # decode-shaped call without its workspace
    assert fwd(L, M=8) == WS
    need = L.caat_rowpar_pcr_fwd_workspace_bytes(8, 8, 64, 64)
    assert need >= 8 * 8 * 64 * 4
    assert fwd(L, M=8, ws=E, wsb=need - 4) == WS
    assert fwd(L, M=8, ws=E + 8, wsb=need) == WS  # workspace must be 16-byte aligned
    assert fwd(L, M=8, ws=D, wsb=need) == ALIAS  # workspace over out
    # empty input: nothing to do, nothing enqueued
    assert fwd(L, M=0) == OK


def test_noalloc_fwd_validation(L):
    """The no-allocation forward checks everything on the host first; shapes
    whose scratch would exceed the library's fixed area are refused."""
    na = L.caat_rowpar_pcr_fwd_noalloc
    assert na(A, B, None, D, 8, 32, 64, 64, None) == NULL
    assert na(None, B, C, D, 8, 32, 64, 64, None) == NULL
    assert na(A, B, C, D + 2, 8, 32, 64, 64, None) == ALIGN
    assert na(A, B, C, A, 8, 32, 64, 64, None) == ALIAS
    assert na(A, B, C, D, 0, 32, 64, 64, None) == DIM
    assert na(A, B, C, D, 8, 0, 64, 64, None) == OK  # empty: nothing enqueued
    # 64 ranks x 65536 channels: 16 MiB of fp32 partials + the counters > the scratch
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(64, 1, 8, 65536) > (16 << 20)
    assert na(A, B, C, D, 64, 1, 8, 65536, None) == WS
    assert na(A, B, C, D, 8, 32, 8, 16384, None) == WS  # 2048 + 8*32*16384*4 bytes


def test_workspace_sizes(L):
    T, Kr, H = 8, 1376, 4096
    # 33 .. 1280 tokens at this width (at most 3 x 176 + 128 = 656 fused
    # tiles of 128 x 64 for a walk of 8 x 22 chunks): the split forward's
    # fp32 products after the counter region -- two contraction slices of
    # them while there are at most 256 tiles of 128 x 64 (M <= 64 here)
    for M in (33, 64):
        assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, M, Kr, H) == 2048 + 2 * T * M * H * 4
    for M in (65, 100, 193, 1280):
        assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, M, Kr, H) == 2048 + T * M * H * 4
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(4, 128, Kr, H) == 2048 + 2 * 4 * 128 * H * 4  # 256 tiles
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(4, 129, Kr, H) == 2048 + 4 * 129 * H * 4  # 384 tiles
    # slices only for contractions of at least 16 chunks of 64
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 64, 960, H) == 2048 + T * 64 * H * 4  # 15 chunks
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 64, 968, H) == 2048 + 2 * T * 64 * H * 4  # 16 chunks
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 1281, Kr, H) == 0  # 672 tiles: fused, no workspace
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 640, 512, H) == 2048 + T * 640 * H * 4  # 320 tiles, walk 64
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 641, 512, H) == 0  # 352 tiles: fused
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(16, 832, 688, H) == 2048 + 16 * 832 * H * 4  # 416 = 2 x 176 + 64
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(16, 833, 688, H) == 0
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 256, 96, 768) == 2048 + T * 256 * 768 * 4  # 24 tiles
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(T, 1408, 96, 768) == 0  # 132 tiles, two-chunk walk: fused
    # one rank: chunked decode, 43 stages of 32 rows in two contraction slices
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(1, 100, Kr, H) == 2048 + 2 * 32 * H * 4
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(2, 8, 64, 65536) == 2048 + 2 * 8 * 65536 * 4
    assert L.caat_rowpar_pcr_fwd_workspace_bytes(2, 8, 64, 65544) == 0  # above 65536 channels: tiled
    for M in (1, 8, 32):
        need = L.caat_rowpar_pcr_fwd_workspace_bytes(T, M, Kr, H)
        assert need == 2048 + T * M * H * 4  # fixed arrival-counter region + fp32 partials
    # with one rank, 33 .. 192 tokens run 32 at a time and share one chunk's partials
    for M in (33, 100, 192):
        assert L.caat_rowpar_pcr_fwd_workspace_bytes(1, M, Kr, H) == L.caat_rowpar_pcr_fwd_workspace_bytes(1, 32, Kr, H)
    assert L.caat_pcr_bwd_workspace_bytes(T, 16384, Kr, H) >= T * 16384 * H * 2  # G for every rank
    assert L.caat_pcr_bwd_workspace_bytes(T, 16384, Kr, H) % 256 == 0
    assert L.caat_pcr_bwd_workspace_bytes(T, 0, Kr, H) == 0
    assert L.caat_pcr_bwd_workspace_bytes(0, 8, Kr, H) == 0  # invalid dims report 0


def test_decode_slice_workspace(L):
    """Below the split forward's start, few ranks cut each contraction into ks
    slices (T * ks <= 8, at most 256 workgroups of 128 channels, two 32-row
    stages per wave and slice); the workspace holds every slice's partials."""
    H = 4096
    ws = L.caat_rowpar_pcr_fwd_workspace_bytes
    assert ws(1, 8, 11008, H) == 2048 + 8 * 1 * 8 * H * 4   # 344 stages: 8 slices
    assert ws(1, 8, 4096, H) == 2048 + 8 * 1 * 8 * H * 4    # 128 stages: still 8
    assert ws(1, 8, 4064, H) == 2048 + 4 * 1 * 8 * H * 4    # 127 stages: 4
    assert ws(2, 15, 5504, H) == 2048 + 4 * 2 * 15 * H * 4  # T * ks <= 8
    assert ws(4, 8, 2752, H) == 2048 + 2 * 4 * 8 * H * 4
    assert ws(4, 8, 1024, H) == 2048 + 2 * 4 * 8 * H * 4    # 32 stages: two slices of 16
    assert ws(4, 8, 992, H) == 2048 + 4 * 8 * H * 4         # 31 stages: whole
    assert ws(8, 8, 11008, H) == 2048 + 8 * 8 * H * 4       # eight ranks: whole
    assert ws(2, 8, 5504, 16384) == 2048 + 2 * 8 * 16384 * 4  # 256 blocks already
    assert ws(2, 8, 5504, 8192) == 2048 + 2 * 2 * 8 * 8192 * 4  # 128 blocks: two slices
    assert ws(3, 7, 2000, 264) == 2048 + -(-2 * 3 * 7 * 264 * 4 // 256) * 256  # 63 stages, T = 3: two slices


def test_bwd_workspace_split_pieces(L):
    """The backward's workspace: G for every rank, then s fp32 pieces of dW
    when its tiles cannot fill 256 CUs and M spans at least 16 chunks of 64
    tokens.  Host-only (nothing is launched)."""
    L.caat_pcr_bwd_workspace_bytes.restype = ctypes.c_size_t

    def pieces(T, M, Kr, H):
        g = -(-(T * M * H * 2) // 256) * 256 + 256  # G, then the tile-class area
        extra = L.caat_pcr_bwd_workspace_bytes(T, M, Kr, H) - g
        assert extra >= 0 and extra % (T * Kr * H * 4) == 0
        return extra // (T * Kr * H * 4) or 1

    assert pieces(8, 16384, 1376, 4096) == 1  # 7B down-proj: 768 tiles of 256x256
    assert pieces(8, 16384, 512, 4096) == 1   # 7B out-proj: 256 of them
    assert pieces(8, 32768, 704, 2048) == 4   # 1.1B: 192 big tiles x 4 = 3 full rounds
    assert pieces(8, 32768, 256, 2048) == 4   # 64 big tiles x 4 = one round
    assert pieces(8, 8192, 384, 768) == 2     # 130M: 144 tiles of 128x128
    assert pieces(8, 8192, 96, 768) == 6      # 48 of them
    assert pieces(8, 960, 96, 768) == 1       # 15 chunks: too short to split
    assert pieces(8, 1024, 96, 768) == 2      # 16 chunks: two pieces of eight
    assert pieces(2, 256, 1536, 768) == 1     # the tiny layer: 4 chunks


def bwd(L, dZ=A, X=B, W=C, mask=D, dX=E, dW=E + (1 << 32), T=4, M=64, Kr=64, H=64, ws=E + (2 << 32), wsb=1 << 20):
    return L.caat_pcr_bwd(dZ, X, W, mask, dX, dW, T, M, Kr, H, ws, wsb, None)


def test_bwd_validation(L):
    assert bwd(L, dZ=None) == NULL
    assert bwd(L, mask=None) == NULL
    assert bwd(L, W=None) == NULL  # dX requested without W
    assert bwd(L, X=None) == NULL  # dW requested without X
    assert bwd(L, H=12) == DIM
    assert bwd(L, dX=E + 4) == ALIGN
    assert bwd(L, dX=A) == ALIAS  # dX over dZ
    assert bwd(L, dW=E) == ALIAS  # dW over dX
    assert bwd(L, ws=None) == WS
    assert bwd(L, wsb=16) == WS
    assert bwd(L, ws=A) == ALIAS  # workspace over dZ
    assert bwd(L, dX=None, dW=None) == OK  # nothing requested: nothing enqueued
    assert bwd(L, M=0, dW=None) == OK  # empty input, dX empty


def colf(L, A_=A, W=B, U=D, T=4, M=64, K=64, N=64):
    return L.caat_colpar_fwd(A_, W, U, T, M, K, N, None)


def colb(L, dU=A, A_=B, W=C, dA=E, dW=E + (1 << 32), T=4, M=64, K=64, N=64):
    return L.caat_colpar_bwd(dU, A_, W, dA, dW, T, M, K, N, None)


def test_colpar_validation(L):
    # host-side checks only: every call here returns before any launch
    assert colf(L, A_=None) == NULL
    assert colf(L, W=None) == NULL
    assert colf(L, T=0) == DIM
    assert colf(L, N=100) == DIM
    assert colf(L, K=12) == DIM
    assert colf(L, U=D + 2) == ALIGN
    assert colf(L, U=A) == ALIAS  # U over A
    assert colf(L, U=B + 16) == ALIAS  # U over W
    assert colf(L, M=0) == OK  # empty: nothing enqueued
    assert colb(L, dU=None) == NULL
    assert colb(L, W=None) == NULL  # dA requested without W
    assert colb(L, A_=None) == NULL  # dW requested without A
    assert colb(L, N=12) == DIM
    assert colb(L, dA=E + 4) == ALIGN
    assert colb(L, dA=A) == ALIAS  # dA over dU
    assert colb(L, dW=E) == ALIAS  # dW over dA
    assert colb(L, dA=None, dW=None) == OK  # nothing requested
    assert colb(L, M=0, dW=None) == OK  # empty input, dA empty


def rms(L, Z=A, R=B, g=C, Ro=D, N=E, T=4, M=64, H=64, eps=1e-5):
    return L.caat_residual_rmsnorm(Z, R, g, Ro, N, T, M, H, eps, None)


def test_residual_rmsnorm_validation(L):
    # host-side checks only: every call here returns before any launch
    assert rms(L, Z=None) == NULL
    assert rms(L, g=None) == NULL
    assert rms(L, N=None) == NULL
    assert rms(L, H=100) == DIM
    assert rms(L, H=8200) == DIM  # above 8192 channels
    assert rms(L, T=0) == DIM
    assert rms(L, eps=-1.0) == DIM
    assert rms(L, eps=float("nan")) == DIM
    assert rms(L, Ro=D + 2) == ALIGN
    assert rms(L, g=C + 8) == ALIGN
    assert rms(L, Ro=A) == ALIAS  # Rout over Z
    assert rms(L, Ro=B + 16) == ALIAS  # Rout partly over R (not in place)
    assert rms(L, N=B) == ALIAS  # N over R
    assert rms(L, N=D) == ALIAS  # N over Rout
    assert rms(L, R=A, Ro=A) == ALIAS  # in-place update of a residual that overlaps Z
    assert rms(L, M=0) == OK  # empty: nothing enqueued


def test_reduce_residual_rmsnorm_validation(L):
    """The reduce with the residual update and norm in its epilogue: host-side
    checks only, every call returns before any launch."""
    f = L.caat_partial_channel_reduce_residual_rmsnorm

    def call(Y=A, mask=B, R=C, g=D, Ro=E, N=E + (1 << 32), T=4, M=16, H=64, eps=1e-5):
        return f(Y, mask, R, g, Ro, N, T, M, H, eps, None)

    assert call(Y=None) == NULL
    assert call(mask=None) == NULL
    assert call(g=None) == NULL
    assert call(N=None) == NULL
    assert call(Y=None, R=None, Ro=None, N=None, M=0) == OK  # empty tensors may be NULL
    assert call(T=0) == DIM
    assert call(T=65) == DIM
    assert call(H=60) == DIM
    assert call(H=8200) == DIM  # above 8192 channels
    assert call(M=1 << 18, H=4096) == DIM  # one rank's slice of 2^30 elements
    assert call(eps=-1.0) == DIM
    assert call(eps=float("nan")) == DIM
    assert call(Ro=E + 2) == ALIGN
    assert call(mask=B + 4) == ALIGN
    assert call(Ro=A) == ALIAS  # Rout over Y
    assert call(N=A + 64) == ALIAS  # N over Y
    assert call(R=A + 128) == ALIAS  # R over Y
    assert call(Ro=C + 16) == ALIAS  # Rout partly over R (not in place)
    assert call(N=C) == ALIAS  # N over R
    assert call(N=E) == ALIAS  # N over Rout
    assert call(Ro=B) == ALIAS  # Rout over the mask
    assert call(M=0) == OK  # empty: nothing enqueued


def test_reduce_validation(L):
    red = L.caat_partial_channel_reduce
    assert red(None, C, D, 8, 16, 64, 0, None) == NULL
    assert red(A, None, D, 8, 16, 64, 0, None) == NULL
    assert red(None, C, None, 8, 0, 64, 0, None) == OK
    assert red(A, C, D, 8, 16, 64, 7, None) == DTYPE
    assert red(A, C, D, 0, 16, 64, 0, None) == DIM
    assert red(A, C, D, 8, 16, 60, 0, None) == DIM
    assert red(A + 4, C, D, 8, 16, 64, 0, None) == ALIGN
    assert red(A, C, A + 256, 8, 16, 64, 0, None) == ALIAS  # partial overlap
    assert red(A, C, D, 8, 0, 64, 0, None) == OK  # empty
    assert red(A, C, A, 8, 0, 64, 1, None) == OK  # in place, empty
    # one rank's slice must stay below 2^30 elements (the kernels count its
    # vectors in 32 bits); these sizes would wrap that count, so they are
    # rejected on the host, in place or not, fp32 or bf16
    big_m = (1 << 22) + 1  # M * 4096 = 2^34 + 4096 elements
    assert red(A, C, D, 1, big_m, 4096, 0, None) == DIM
    assert red(A, C, A, 1, big_m, 4096, 0, None) == DIM
    assert red(A, C, D, 1, 1 << 23, 4096, 1, None) == DIM  # 2^35 bf16 elements
    assert red(A, C, D, 2, 1 << 18, 4096, 0, None) == DIM  # exactly 2^30 per rank


def test_product_path_fails_loudly_without_library(tmp_path):
    """No silent fallback: a missing library raises."""
    from partial_channel_reduce_amd import ops

    with pytest.raises(RuntimeError, match="not built"):
        ops.lib(str(tmp_path / "missing.so"))


def test_binding_signatures_match_header_arity():
    from partial_channel_reduce_amd import ops

    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, _, args in ops.SIGNATURES:
        m = re.search(name + r"\s*\(([^)]*)\)", text)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), name
