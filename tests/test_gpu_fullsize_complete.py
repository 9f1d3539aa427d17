"""Complete element-by-element parity at the other full-size layer shapes, in
the launch configuration the benchmark times (the Llama2-7B down-projection
forward is in test_gpu_fullsize_7b.py):

* forwards of the 7B attention out-projection (Kr = 512), the TinyLlama-1.1B
  down- and out-projections (contiguous and strided S) and the 130M layers:
  every output against the fp64 oracle, block by block, under both bars;
  synced channels bitwise identical across ranks;
* the 130M layers' backward: every element of dX and dW, with the allowance
  for the bf16 rounding of the reduced gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from partial_channel_reduce_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BLOCK = 2048


@pytest.fixture(scope="module")
def ops():
    from partial_channel_reduce_amd import ops as _ops

    _ops.lib()
    return _ops


def _announce(msg):
    print(f"[case] {msg}", flush=True)


FWD = [
    ("Llama2-7B out-proj", 8, 16384, 512, 4096, "random", 0.5),
    ("TinyLlama-1.1B down-proj, S = first half", 8, 32768, 704, 2048, "prefix", 0.5),
    ("TinyLlama-1.1B down-proj, even channels", 8, 32768, 704, 2048, "strided", 0.5),
    ("TinyLlama-1.1B out-proj, even channels", 8, 32768, 256, 2048, "strided", 0.5),
    ("130M down-proj", 8, 8192, 384, 768, "random", 0.5),
    ("130M out-proj, p = 0.25", 8, 8192, 96, 768, "random", 0.25),
]


@pytest.mark.parametrize("name,T,M,Kr,H,kind,p", FWD)
def test_fwd_every_element(ops, name, T, M, Kr, H, kind, p):
    _announce(f"every element, fwd {name}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=9)
    mask = synth.make_mask(H, p, kind, seed=9)
    out = ops.rowpar_pcr_fwd(G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    bits = G.bf16_bits(out)
    del out
    S = mask != 0
    for t in range(1, T):
        assert np.array_equal(bits[t][:, S], bits[0][:, S]), f"synced channels differ between rank 0 and {t}"
    bar = G.Bf16Bar(f"fwd {name}")
    for m0 in range(0, M, BLOCK):
        ref = oracle.rowpar_pcr_fwd(X[:, m0:m0 + BLOCK], W, mask)
        bar.add(oracle.bf16_to_f64(bits[:, m0:m0 + BLOCK]), ref, S[None, None, :])
    print(f"[result] {bar.finish()}", flush=True)


@pytest.mark.parametrize("name,Kr,p", [("130M down-proj", 384, 0.5), ("130M out-proj", 96, 0.75)])
def test_bwd_130m_every_element(ops, name, Kr, p):
    T, M, H = 8, 8192, 768
    _announce(f"every element, bwd {name}")
    X, W = synth.make_fwd_inputs(T, M, Kr, H, seed=10)
    dZ = synth.make_grad(T, M, H, seed=10)
    mask = synth.make_mask(H, p, "random", seed=10)
    dX, dW = ops.pcr_bwd(G.to_dev_bf16(dZ), G.to_dev_bf16(X), G.to_dev_bf16(W), G.to_dev_u8(mask))
    torch.cuda.synchronize()
    rdX, rdW = oracle.pcr_bwd(dZ, X, W, mask)
    ax, aw = G.bwd_g_allowance(dZ, X, W, mask)
    print(G.check_bf16(G.from_dev_bf16(dX), rdX, None, f"dX {name}", extra=ax))
    print(G.check_bf16(G.from_dev_bf16(dW), rdW, (mask != 0)[None, None, :], f"dW {name}", extra=aw))
