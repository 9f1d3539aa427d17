"""Seeded random shapes for the GPU sweep test, with the forward path each
one takes (mirroring the library's dispatch rules, so the sweep can assert
that every path is covered)."""
import numpy as np


def decode_slices(T, Kr, H):
    """Contraction slices per rank the decode kernel takes (whole stages of 32
    rows): doubled while T * ks <= 8, the workgroups T * ceil(H/128) * ks stay
    within 256 and each of the 8 waves keeps two stages of every slice."""
    items, ns, ks = T * -(-H // 128), -(-Kr // 32), 1
    while 2 * ks <= 8 and 2 * ks * T <= 8 and 2 * ks * items <= 256 and ns >= 2 * ks * 16:
        ks *= 2
    return ks


def forward_path(T, M, Kr, H):
    """Which forward kernel the library runs for (T, M, Kr, H) with a mask."""
    tiles64 = -(-H // 128) * -(-M // 64)
    nk = -(-Kr // 64)
    walk = T * nk
    limit = 128 if nk <= 2 else (3 * walk + 128 if T <= 8 else 2 * walk + 64)
    min_m = 33 if T <= 8 else 24  # where the split takes over from the decode kernel
    if T >= 2 and M >= min_m and tiles64 <= limit:
        wg256 = T * -(-H // 256) * -(-M // 256)
        full = 4 * M >= 3 * 256 * -(-M // 256)  # token tiles at least 3/4 full
        if full and (wg256 % 256 == 0 or 192 <= wg256 < 256):
            return "split256"
        if T * -(-H // 128) * -(-M // 128) >= 512:
            return "split128"
        # two contraction slices per rank: few 128x64 tiles, long contractions
        return "split64x2" if tiles64 * T <= 256 and nk >= 16 else "split64"
    if M <= 192 and H <= 65536:
        base = "decode" if M <= 32 else "chunked"
        return base + "_sliced" if decode_slices(T, Kr, H) > 1 else base
    big = -(-M // 256) * -(-H // 256) >= 160
    small = not big and -(-H // 128) * -(-M // 128) < 512
    if small and T >= 2 and (T <= 4 or (T <= 8 and Kr <= 128)):
        return "queue"
    base = "fused256" if big else "fused128x64" if small else "fused128"
    # short contractions: the mask's mixed 256-channel groups go to the
    # register-queue kernel in a second launch
    return base + "+queue" if 2 <= T <= 8 and (nk <= 6 or (small and nk <= 12)) else base


def cases(n=64, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    kinds = [("random", 0.5), ("prefix", 0.5), ("strided", 0.5), ("random", 0.3), ("random", 0.0), ("random", 1.0)]
    while len(out) < n:
        T = int(rng.choice([1, 2, 3, 4, 5, 8, 8, 8, 13, 16]))
        M = int(rng.choice([1, 5, 17, 32, 33, 64, 100, 150, 193, 300, 700, 1000, 1500, 2100, 3000]))
        Kr = 8 * int(rng.integers(1, 200))
        H = 8 * int(rng.integers(1, 280))
        if T * M * Kr * H > 3e8:  # keep the fp64 oracle quick
            continue
        kind, p = kinds[int(rng.integers(len(kinds)))]
        out.append((T, M, Kr, H, kind, p, int(rng.integers(1 << 30))))
    # paths that need more tiles than the size cap usually allows: split with
    # 128-token tiles, fused 128x128 and 256x256 tiles, more register-queue
    # and fused 128x64 tiles
    out += [(8, 512, 192, 2048, "random", 0.5, 11), (2, 4096, 16, 2048, "strided", 0.5, 12),
            (2, 8192, 8, 2048, "random", 0.5, 13), (4, 3000, 40, 776, "prefix", 0.5, 14),
            (8, 3000, 96, 512, "random", 0.5, 15), (5, 2500, 200, 264, "random", 0.5, 16),
            # the largest rank count the library takes
            (64, 20, 16, 264, "random", 0.5, 17), (64, 100, 72, 128, "strided", 0.5, 18),
            (64, 900, 8, 64, "random", 0.5, 19), (64, 8256, 8, 64, "prefix", 0.5, 20),
            # split forward with 256x256 tiles: 192 of them (ragged tokens), 256
            # (ragged channels), 256 at T = 16
            (8, 1800, 136, 768, "random", 0.5, 21), (8, 1900, 200, 776, "strided", 0.5, 22),
            (16, 2000, 72, 512, "random", 0.5, 23),
            # split forward, two contraction slices per rank (17 chunks: 9 + 8)
            (4, 100, 1048, 512, "random", 0.5, 24),
            # tiled forwards with more ranks than the register queue holds (one
            # launch): 256x256 and 128x128 tiles; and 128x64 tiles with the
            # mixed groups in a second launch
            (9, 4096, 8, 4096, "random", 0.5, 25), (9, 2048, 16, 4096, "strided", 0.5, 26),
            (8, 4096, 256, 512, "random", 0.5, 27),
            # decode with contraction slices: 8 (one rank), 4 (two ranks, ragged
            # channel block), 2 (three ranks); one rank in 32-token chunks
            (1, 3, 4104, 520, "random", 0.5, 28), (2, 9, 2056, 776, "prefix", 0.5, 29),
            (3, 7, 2000, 264, "strided", 0.5, 30), (1, 70, 1032, 264, "random", 0.5, 31)]
    return out
