"""The backward's reduced gradient G with tiles of 256 channels classified:
wholly local tiles are read from dZ, wholly synced ones hold the one sum once,
mixed ones get every rank's copy.  Masks that mix all three classes (and a
partial last tile), integer inputs: dX and dW bit for bit against the oracle,
on the 256x256 and 128x128 kernels and the split dW."""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _class_mask(H, pattern, seed):
    """pattern[i] for tile i (256 channels): 's' all synced, 'l' all local, 'm' random half."""
    rng = np.random.default_rng(seed)
    mask = np.zeros(H, dtype=np.uint8)
    for i, k in enumerate(pattern):
        c0, c1 = 256 * i, min(H, 256 * (i + 1))
        if c0 >= H:
            break
        if k == "s":
            mask[c0:c1] = 1
        elif k == "m":
            mask[c0:c1] = (rng.random(c1 - c0) < 0.5).astype(np.uint8)
            mask[c0] = 1
            mask[c0 + 1] = 0  # surely mixed
    return mask


def _int_grad(T, M, H, seed, density=0.2):
    rng = np.random.default_rng(seed)
    dZ = rng.integers(-1, 2, size=(T, M, H)) * (rng.random((T, M, H)) < density)
    return synth.f32_to_bf16_bits(dZ.astype(np.float32))


CASES = [
    # T, M, Kr, H, tile pattern: 256x256 dX (288 tiles) and split 128x128 dW
    (3, 8192, 520, 1024, "slms"),
    # 128x128 dX and dW, a partial last tile (H = 776: three full tiles and 8 channels)
    (4, 300, 200, 776, "lsms"),
    (2, 520, 136, 776, "mslm"),
    # all synced / all local (every tile uniform)
    (8, 512, 384, 768, "sss"),
    (8, 512, 384, 768, "lll"),
    # big dW tiles without a split
    (8, 1024, 1376, 4096, "sslmsmllssllmsss"),
]


@pytest.mark.parametrize("T,M,Kr,H,pattern", CASES)
def test_bwd_tile_classes_bitwise(ops, T, M, Kr, H, pattern):
    _announce(f"bwd tile classes T={T} M={M} Kr={Kr} H={H} {pattern}")
    X, W = synth.make_integer_fwd_inputs(T, M, Kr, H, seed=T + M, lo=-1, hi=1, x_zero_frac=0.8)
    dZ = _int_grad(T, M, H, seed=T + H, density=0.05 if H >= 4096 else 0.2)
    mask = _class_mask(H, pattern, seed=M)
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    assert max(np.abs(rdX).max(), np.abs(rdW).max()) <= 256
    ws = torch.full((ops.bwd_workspace_bytes(T, M, Kr, H),), 0x7F, dtype=torch.uint8, device=G.dev())
    dX, dW = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask), workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(G.from_dev_bf16(dX), rdX), "dX differs from the oracle"
    assert np.array_equal(G.from_dev_bf16(dW), rdW), "dW differs from the oracle"
