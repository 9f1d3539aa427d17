"""The forward's two-launch form: with 2 <= T <= 8 and at most six chunks of
64 per rank's contraction (twelve where the tiles are 128 x 64 anyway), the
tiled kernel takes the 256-channel groups of
the mask in which every 8-channel chunk is wholly synced or wholly local, and
the register-queue kernel the groups with a chunk that mixes the two.  Each
workgroup decides from its own group, so a mask with both kinds of group has
its output written by both kernels.  Integer inputs bit for bit against the
oracle, on every tiled base (256x256, 128x128, 128x64 tiles) and with masks
whose groups are all mixed, all uniform, alternating, none synced and all
synced."""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G
from tests.sweep_cases import forward_path

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _mask(H, kind, seed):
    if kind == "alternating":  # even groups: a random half; odd groups: the first 128 channels
        rng = np.random.default_rng(seed)
        m = np.zeros(H, dtype=np.uint8)
        for g0 in range(0, H, 256):
            n = min(256, H - g0)
            if (g0 // 256) % 2 == 0:
                m[g0:g0 + n] = rng.random(n) < 0.5
            else:
                m[g0:g0 + min(128, n)] = 1
        return m
    if kind == "none":
        return np.zeros(H, dtype=np.uint8)
    if kind == "all":
        return np.ones(H, dtype=np.uint8)
    return synth.make_mask(H, 0.5, kind, seed=seed)


def _mixed_groups(mask):
    H = mask.shape[0]
    ch = (mask.reshape(H // 8, 8) != 0)
    mixed_chunk = ch.any(1) & ~ch.all(1)
    return [bool(mixed_chunk[g * 32:(g + 1) * 32].any()) for g in range(-(-H // 256))]


# (T, M, Kr, H) and the tiled base each takes
SHAPES = [((2, 8192, 8, 2048), "fused256+queue"), ((2, 4096, 16, 2048), "fused128+queue"),
          ((8, 4096, 256, 520), "fused128x64+queue"), ((5, 3000, 136, 1032), "fused128x64+queue"),
          ((5, 6000, 456, 264), "fused128x64+queue")]  # 8 chunks: two launches with 128x64 tiles only
KINDS = ["random", "strided", "prefix", "alternating", "none", "all"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape,path", SHAPES, ids=[p + "-" + "x".join(map(str, s)) for s, p in SHAPES])
def test_two_launch_forward_bitwise(ops, shape, path, kind):
    T, M, Kr, H = shape
    assert forward_path(T, M, Kr, H) == path
    mask = _mask(H, kind, seed=T + M + Kr)
    mg = _mixed_groups(mask)
    if kind == "alternating":
        assert any(mg) and not all(mg)  # both launches write part of the output
    elif kind in ("random", "strided"):
        assert all(mg)
    elif kind in ("none", "all"):
        assert not any(mg)
    # (a contiguous S is uniform everywhere but in the group where it ends,
    # when that end is not a multiple of 8: with H = 520 the first 260
    # channels leave group 1 mixed)
    _announce(f"two-launch fwd T={T} M={M} Kr={Kr} H={H} {path} {kind}")
    zf = 1.0 - min(0.9, 6.0 / np.sqrt(T * Kr))
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=M + H, lo=-1, hi=1, x_zero_frac=zf)
    ref = oracle.rowpar_pcr_fwd(X, W, mask)
    assert np.abs(ref).max() <= 256
    out = torch.full((T, M, H), 7.0, dtype=torch.bfloat16, device=G.dev())  # every element must be written
    ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), out)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(out), ref)
