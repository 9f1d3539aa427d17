"""Benchmark of the row-parallel GEMM + partial channel-reduce on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (one step): the Llama2-7B MLP down-projection as a row-parallel layer
with partial channel-reduce, forward + backward: T = 8 ranks resident on the
GPU, M = 4 x 4096 = 16384 tokens, K = 11008 (Kr = 1376 per rank), H = 4096,
sync fraction p = 0.5 with a seeded random channel mask, bf16 inputs
X ~ N(0,1), W ~ N(0,0.02), dZ ~ N(0,1), fp32 accumulation.  Inputs are
synthetic and resident in HBM before timing starts.

Printed: one JSON line.  `value` is the step's algorithmic TFLOP/s
(fwd 2MKH + bwd 4MKH flops).  Beside it: per-kernel times, the roofline of the
dominant kernel, the standalone reduce in GB/s, the decode-shaped forward in
GB/s, the attention out-projection (Kr = 512) and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused rowpar GEMM+partial-reduce TFLOP/s (% MFMA peak); reduce GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

T, M, KR, H, P = 8, 16384, 1376, 4096, 0.5
KR_OUT = 512
# The smaller models' row-parallel layers (name, T, M, Kr, H, mask kind), all at p = 0.5:
# the 130M model (h = 768, 8 x 1024 tokens) and TinyLlama-1.1B (h = 2048, 16 x 2048 tokens).
MODEL_SHAPES = (
    ("130M down-proj", 8, 8192, 384, 768, "random"),
    ("130M out-proj", 8, 8192, 96, 768, "random"),
    ("1.1B down-proj", 8, 32768, 704, 2048, "prefix"),
    ("1.1B down-proj", 8, 32768, 704, 2048, "strided"),
    ("1.1B out-proj", 8, 32768, 256, 2048, "prefix"),
    ("1.1B out-proj", 8, 32768, 256, 2048, "strided"),
)
COPY_ELEMS = 1 << 28           # fp32 elements of the calibration kernel (1 GiB each way)
PAYLOAD_P = (0.25, 0.5, 0.75, 1.0)  # sync fractions of the payload leg (prefix masks)
PAYLOAD_CALLS = 3                   # in-place reduce calls per p before its timing
COPY_KERNEL_KEY = "neg_kernel"  # substring naming torch's elementwise negation kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_7b_down_proj.txt")
MASK_ORDER = ("random", "prefix", "strided")  # the fwd_masks leg's order


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096,
                    help="tokens of the CPU oracle sample (about 10 s on 16 host threads)")
    ap.add_argument("--reduce-m", default="16384,4096,1,8,32",
                    help="token counts of the reduce leg (<= 32: latency points; counter runs take one at a time)")
    ap.add_argument("--decode-m", default="1,8,32", help="token counts of the decode legs (counter runs take one at a time)")
    ap.add_argument("--only", default="", help="comma list of legs: train,context,out,shapes,reduce,decode,decode_out,mid,tsweep,colpar,norm,reduce_norm,payload,copy (profiling runs)")
    ap.add_argument("--rocprof-stats", metavar="DIR", help="print a summary of a rocprofv3 --stats csv run and exit")
    ap.add_argument("--rocprof-mfma", metavar="DIR",
                    help="print per-kernel MfmaUtil and performed bf16 MFMA flops from a rocprofv3 "
                         "--pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 csv run of the train leg, and exit")
    ap.add_argument("--rocprof-payload", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the in-place reduce's calibrated bytes per dispatch for each p of the payload leg "
                         "from two rocprofv3 --pmc csv runs of `--only payload,copy`, and exit")
    ap.add_argument("--rocprof-stall", nargs=3, metavar=("SQ_DIR", "TCP_DIR", "TA_DIR"),
                    help="print where the GEMMs' memory path waits (L1 stalls on L2 data, TA/TD busy, L2 hit rate, "
                         "LDS bank conflicts, wave waits) from three rocprofv3 --pmc csv runs of the train leg, and exit")
    ap.add_argument("--rocprof-masks", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="forward HBM traffic per sync-set kind from two --pmc runs of `--only fwd_masks,copy`, and exit")
    ap.add_argument("--rocprof-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print per-kernel HBM bytes from two rocprofv3 --pmc csv runs (FETCH_SIZE, WRITE_SIZE), "
                         "calibrated against the copy leg's kernel, and exit")
    ap.add_argument("--rocprof-channel-yaml", metavar="PATH",
                    help="write the per-L2-channel counter definitions (for rocprofv3 -E) to PATH, and exit")
    ap.add_argument("--rocprof-channels", nargs="+", metavar="DIR",
                    help="per-L2-channel totals and spread of the fp32 reduce (its largest launch) from rocprofv3 "
                         "--pmc csv runs made with the --rocprof-channel-yaml counters, and exit")
    return ap.parse_args()


# Per-L2-channel counters: each TCC counter below has one value per channel
# (16 per XCD) and per XCD; a derived counter per channel sums one channel
# over the eight XCDs.  Two passes (at most four TCC base counters each): the
# DRAM credit stalls with the busy cycles, and the requests.
CHANNEL_PASSES = ((("RST", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL"), ("WST", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL"),
                   ("BUSY", "TCC_BUSY")),
                  (("RD", "TCC_EA0_RDREQ"), ("WR", "TCC_EA0_WRREQ")))
CHANNEL_COUNTERS = tuple(c for p in CHANNEL_PASSES for c in p)
N_L2_CHANNELS = 16


def channel_counter_yaml() -> str:
    out = ["rocprofiler-sdk:", "  counters-schema-version: 1", "  counters:"]
    for tag, base in CHANNEL_COUNTERS:
        for k in range(N_L2_CHANNELS):
            out += [f"  - name: {tag}_CH{k}", f"    description: {base} of L2 channel {k}, summed over the XCDs",
                    "    properties: []", "    definitions:", "    - architectures:", "      - gfx950",
                    f"      expression: reduce(select({base},[DIMENSION_INSTANCE=[{k}]]),sum)"]
    return "\n".join(out) + "\n"


def channel_counter_names() -> str:
    """One line per pass: the derived counters to hand to --pmc."""
    return "\n".join(" ".join(f"{tag}_CH{k}" for tag, _ in p for k in range(N_L2_CHANNELS)) for p in CHANNEL_PASSES)


def rocprof_channels_summary(dirs) -> str:
    """Per-channel medians over the fp32 reduce's largest launches, one block per run."""
    import statistics as st
    out = []
    for d in dirs:
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv"))
                if "pcr_reduce_f32" in r["Kernel_Name"]]
        if not rows:
            out.append(f"{d}: no fp32 reduce launch")
            continue
        g = max(int(r["Grid_Size"]) for r in rows)
        per, dur = {}, {}
        for r in rows:
            if int(r["Grid_Size"]) != g:
                continue
            per.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
            dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        out.append(f"{d}: {len(dur)} launches of {g} threads, profiled duration median {st.median(dur.values()):.0f} us")
        out.append("| counter | total (M) | max / mean | min / mean | cv | per channel (M) |")
        out.append("|---|---|---|---|---|---|")
        for tag, base in CHANNEL_COUNTERS:
            if f"{tag}_CH0" not in per:
                continue
            v = [st.median(per[f"{tag}_CH{k}"].values()) for k in range(N_L2_CHANNELS)]
            m = st.mean(v)
            out.append(f"| {base} | {sum(v) / 1e6:.2f} | {max(v) / m:.3f} | {min(v) / m:.3f} | "
                       f"{st.pstdev(v) / m:.3f} | " + " ".join(f"{x / 1e6:.2f}" for x in v) + " |")
        out.append("")
    return "\n".join(out)


# The sources each counted kernel is compiled from (its device code; the host
# dispatch that picks it is the bench's fixed configuration).
_GEMM_SOURCES = ("common.hpp", "gemm_core.hpp", "gemm_kernels.hpp", "reduce_kernels.hpp")
KERNEL_SOURCES = {
    "rowpar_pcr_fwd_kernel": _GEMM_SOURCES,
    "pcr_bwd_dx_kernel": _GEMM_SOURCES,
    "pcr_bwd_dw_kernel": _GEMM_SOURCES,
    "pcr_reduce_bf16_kernel": ("common.hpp", "reduce_kernels.hpp"),
    "pcr_reduce_bf16_runs8_kernel": ("common.hpp", "reduce_kernels.hpp"),
    "pcr_reduce_f32_runs8_kernel": ("common.hpp", "reduce_kernels.hpp"),
    "pcr_reduce_bf16_runs16_kernel": ("common.hpp", "reduce_kernels.hpp"),
}


def src_hash(files=None) -> str:
    """Hash of the kernel sources (all of them, or the given files)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "partial_channel_reduce_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def kernel_src_hash(kernel: str) -> str:
    return src_hash(KERNEL_SOURCES.get(kernel))


def main():
    args = parse()
    if args.rocprof_stats:
        print(rocprof_stats_summary(args.rocprof_stats))
        return
    if args.rocprof_mfma:
        print(rocprof_mfma_summary(args.rocprof_mfma))
        return
    if args.rocprof_payload:
        print(rocprof_payload_summary(*args.rocprof_payload))
        return
    if args.rocprof_stall:
        print(rocprof_stall_summary(*args.rocprof_stall))
        return
    if args.rocprof_masks:
        print(rocprof_masks_summary(*args.rocprof_masks))
        return
    if args.rocprof_traffic:
        print(rocprof_traffic_summary(*args.rocprof_traffic))
        return
    if args.rocprof_channel_yaml:
        with open(args.rocprof_channel_yaml, "w") as f:
            f.write(channel_counter_yaml())
        print(channel_counter_names())
        return
    if args.rocprof_channels:
        print(rocprof_channels_summary(args.rocprof_channels))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            "bench.py measures one GPU: the T tensor-parallel ranks are resident shards on a single "
            "MI355X; a run across several GPUs is not measured here.",
            file=sys.stderr,
        )
        sys.exit(2)

    import numpy as np
    import torch

    from partial_channel_reduce_amd import ops, synth

    ops.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    legs = set(args.only.split(",")) if args.only else {"train", "context", "out", "reduce", "decode", "tsweep",
                                                         "colpar", "norm", "reduce_norm", "fwd_masks", "payload", "decode_out", "shapes",
                                                         "mid"}
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def randn_bf16(shape, scale=1.0):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * scale).to(torch.bfloat16)

    def mask_dev(Hh, seed=0, kind="random"):
        return torch.from_numpy(synth.make_mask(Hh, P, kind, seed=seed)).to(dev)

    def time_call(fn, iters, warm=2):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / iters  # ms

    res = {}
    K = T * KR
    flops_fwd = 2.0 * M * K * H
    flops_step = 3.0 * flops_fwd

    # ------------------------------------------------------------------ train
    if "train" in legs:
        log("allocating 7B down-proj inputs")
        X = randn_bf16((T, M, KR))
        W = randn_bf16((T, KR, H), 0.02)
        dZ = randn_bf16((T, M, H))
        mk = mask_dev(H)
        out = torch.empty((T, M, H), dtype=torch.bfloat16, device=dev)
        dX = torch.empty_like(X)
        dW = torch.empty_like(W)
        ws = torch.empty(ops.bwd_workspace_bytes(T, M, KR, H), dtype=torch.uint8, device=dev)

        def step():
            ops.rowpar_pcr_fwd(X, W, mk, out=out)
            ops.pcr_bwd(dZ, X, W, mk, dX=dX, dW=dW, workspace=ws)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        log(f"timing {args.steps} steps")
        # Events on the launch stream around the forward and the backward of
        # every timed step: the per-launch kernel times quoted below come from
        # the timed region itself.
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(args.steps):
            evs[i][0].record()
            ops.rowpar_pcr_fwd(X, W, mk, out=out)
            evs[i][1].record()
            ops.pcr_bwd(dZ, X, W, mk, dX=dX, dW=dW, workspace=ws)
            evs[i][2].record()
        e.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_step = s.elapsed_time(e) / args.steps
        res["ms_per_step"] = ms_step
        res["wall_s"] = wall
        log(f"step {ms_step:.3f} ms")
        t_fwd = sum(ev[0].elapsed_time(ev[1]) for ev in evs) / args.steps
        t_bwd_step = sum(ev[1].elapsed_time(ev[2]) for ev in evs) / args.steps

        # dX and dW separated by timing the backward with one product off
        it = max(3, args.steps // 2)
        t_bwd = time_call(lambda: ops.pcr_bwd(dZ, X, W, mk, dX=dX, dW=dW, workspace=ws), it)
        t_bdx = time_call(lambda: ops.pcr_bwd(dZ, X, W, mk, dX=dX, need_dw=False, workspace=ws), it)
        t_bdw = time_call(lambda: ops.pcr_bwd(dZ, X, W, mk, dW=dW, need_dx=False, workspace=ws), it)
        k = {
            "rowpar_pcr_fwd_kernel": t_fwd,
            "pcr_bwd_dw_kernel": t_bwd - t_bdx,
            "pcr_bwd_dx_kernel": t_bwd - t_bdw,
            "pcr_reduce_bf16_kernel (G)": max(t_bdx + t_bdw - t_bwd, 0.0),
        }
        res["kernels_ms"] = {n: round(v, 4) for n, v in k.items()}
        per_flops = {"rowpar_pcr_fwd_kernel": flops_fwd, "pcr_bwd_dw_kernel": flops_fwd, "pcr_bwd_dx_kernel": flops_fwd}
        dom = max(per_flops, key=lambda n: k[n])
        ach = per_flops[dom] / (k[dom] * 1e-3) / 1e12
        res["dominant"] = dom
        res["roofline"] = {
            "bound": "mfma",
            "kernel": dom,
            "achieved": round(ach, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic(dom),
        }
        res["fwd_tflops"] = round(flops_fwd / (t_fwd * 1e-3) / 1e12, 2)
        res["bwd_tflops"] = round(2 * flops_fwd / (t_bwd_step * 1e-3) / 1e12, 2)

    if "train" in legs and "context" in legs:
        # The same step with S = the first half of the channels.  A contiguous
        # S (reachable for any S by one model-wide channel permutation) lets
        # the forward write the synced sums as whole lines.
        mkp = mask_dev(H, kind="prefix")
        t_pf = time_call(lambda: ops.rowpar_pcr_fwd(X, W, mkp, out=out), it)
        t_pb = time_call(lambda: ops.pcr_bwd(dZ, X, W, mkp, dX=dX, dW=dW, workspace=ws), it)
        res["prefix_mask"] = {"fwd_ms": round(t_pf, 4), "bwd_ms": round(t_pb, 4),
                              "tflops": round(flops_step / ((t_pf + t_pb) * 1e-3) / 1e12, 2)}

        # Context only (not part of the path): the vendor GEMM library
        # (hipBLASLt through torch.bmm) on the three plain per-rank products of
        # the same shapes, without any reduce.  Both operands contiguous.
        yb = torch.empty((T, M, H), dtype=torch.bfloat16, device=dev)
        wt = W.transpose(1, 2).contiguous()
        xt = X.transpose(1, 2).contiguous()
        t_lf = time_call(lambda: torch.bmm(X, W, out=yb), it)
        t_lx = time_call(lambda: torch.bmm(dZ, wt, out=dX), it)
        t_lw = time_call(lambda: torch.bmm(xt, dZ, out=dW), it)
        res["library_gemm"] = {
            "what": "torch.bmm (hipBLASLt), plain products of the same shapes, no reduce",
            "fwd_ms": round(t_lf, 4), "dx_ms": round(t_lx, 4), "dw_ms": round(t_lw, 4),
            "tflops": round(flops_step / ((t_lf + t_lx + t_lw) * 1e-3) / 1e12, 2),
        }
        del yb, wt, xt
    if "train" in legs:
        del X, W, dZ, out, dX, dW, ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------- out-projection
    if "out" in legs:
        Ko = T * KR_OUT
        Xo = randn_bf16((T, M, KR_OUT))
        Wo = randn_bf16((T, KR_OUT, H), 0.02)
        dZo = randn_bf16((T, M, H))
        mk = mask_dev(H)
        outo = torch.empty((T, M, H), dtype=torch.bfloat16, device=dev)
        dXo, dWo = torch.empty_like(Xo), torch.empty_like(Wo)
        wso = torch.empty(ops.bwd_workspace_bytes(T, M, KR_OUT, H), dtype=torch.uint8, device=dev)
        tf = time_call(lambda: ops.rowpar_pcr_fwd(Xo, Wo, mk, out=outo), 10)
        tb = time_call(lambda: ops.pcr_bwd(dZo, Xo, Wo, mk, dX=dXo, dW=dWo, workspace=wso), 10)
        fo = 2.0 * M * Ko * H
        res["out_proj"] = {
            "Kr": KR_OUT,
            "fwd_ms": round(tf, 4),
            "bwd_ms": round(tb, 4),
            "fwd_bwd_tflops": round(3 * fo / ((tf + tb) * 1e-3) / 1e12, 2),
        }
        del Xo, Wo, dZo, outo, dXo, dWo, wso
        torch.cuda.empty_cache()

    # -------------------------------------------- the smaller models' layers
    if "shapes" in legs:
        # Forward and backward of each layer against its roofline: algorithmic
        # flops 2*M*(T*Kr)*H (backward twice that) and bytes X + W + out
        # (backward dZ + X + W read, dX + dW written); the bound is the
        # larger of flops / bf16 peak and bytes / HBM peak.  Buffer sets are
        # rotated so that every call streams at least 600 MB: operands do not
        # sit in the 256 MB last-level cache between calls.
        rows = []
        for name, Ts, Ms, Ks, Hs, kind in MODEL_SHAPES:
            bf = 2 * (Ts * Ms * Ks + Ts * Ks * Hs + Ts * Ms * Hs)
            bb = 2 * (Ts * Ms * Hs + 2 * Ts * Ms * Ks + 2 * Ts * Ks * Hs)
            nset = max(1, min(4, -(-600_000_000 // bf)))
            sets = []
            for _ in range(nset):
                sets.append((randn_bf16((Ts, Ms, Ks)), randn_bf16((Ts, Ks, Hs), 0.02), randn_bf16((Ts, Ms, Hs)),
                             torch.empty((Ts, Ms, Hs), dtype=torch.bfloat16, device=dev),
                             torch.empty((Ts, Ms, Ks), dtype=torch.bfloat16, device=dev),
                             torch.empty((Ts, Ks, Hs), dtype=torch.bfloat16, device=dev)))
            mks = mask_dev(Hs, kind=kind)
            wss = torch.empty(ops.bwd_workspace_bytes(Ts, Ms, Ks, Hs), dtype=torch.uint8, device=dev)
            ctr = [0]

            def fwd_call():
                Xs, Ws, _, Os, _, _ = sets[ctr[0] % nset]
                ctr[0] += 1
                ops.rowpar_pcr_fwd(Xs, Ws, mks, out=Os)

            def bwd_call():
                Xs, Ws, dZs, _, dXs, dWs = sets[ctr[0] % nset]
                ctr[0] += 1
                ops.pcr_bwd(dZs, Xs, Ws, mks, dX=dXs, dW=dWs, workspace=wss)

            iters = 4 * nset
            tf = time_call(fwd_call, iters, warm=nset)
            tb = time_call(bwd_call, iters, warm=nset)
            ff = 2.0 * Ms * (Ts * Ks) * Hs
            roof_f = max(ff / (PEAK_BF16_TFLOPS * 1e9), bf / (PEAK_HBM_GBS * 1e6))  # ms
            roof_b = max(2 * ff / (PEAK_BF16_TFLOPS * 1e9), bb / (PEAK_HBM_GBS * 1e6))
            rows.append({
                "layer": name, "T": Ts, "M": Ms, "Kr": Ks, "H": Hs, "mask": kind, "p": P,
                "fwd_us": round(tf * 1e3, 1), "bwd_us": round(tb * 1e3, 1),
                "fwd_bound": "mfma" if ff / bf > PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3 else "hbm",
                "fwd_tflops": round(ff / (tf * 1e-3) / 1e12, 1), "fwd_GBs": round(bf / (tf * 1e-3) / 1e9, 1),
                "fwd_frac_roof": round(roof_f / tf, 3),
                "bwd_tflops": round(2 * ff / (tb * 1e-3) / 1e12, 1), "bwd_frac_roof": round(roof_b / tb, 3),
            })
            log(f"{name} ({kind}): fwd {tf * 1e3:.1f} us ({roof_f / tf:.2f} of roofline), bwd {tb * 1e3:.1f} us")
            del sets, mks, wss
            torch.cuda.empty_cache()
        res["model_shapes"] = rows

    # ------------------------------------------------------ reduce-only fp32
    if "reduce" in legs:
        red = {}
        mk = mask_dev(H, seed=1)
        red_m = [int(x) for x in args.reduce_m.split(",") if x]
        for Mr in [m for m in red_m if m > 32]:
            Y = torch.randn((T, Mr, H), generator=gen, device=dev, dtype=torch.float32)
            o = torch.empty_like(Y)
            t = time_call(lambda: ops.partial_channel_reduce(Y, mk, out=o), 10)
            nbytes = 2.0 * T * Mr * H * 4
            gbs = nbytes / (t * 1e-3) / 1e9
            red[f"M{Mr}"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
            del Y, o
        # decode-sized reduces: latency-bound, rotate 64 buffer sets (> the 256 MB last-level cache)
        for Mr in [m for m in red_m if m <= 32]:
            sets = [torch.randn((T, Mr, H), generator=gen, device=dev) for _ in range(64)]
            outs = [torch.empty_like(x) for x in sets]
            idx = [0]

            def call():
                i = idx[0] % len(sets)
                idx[0] += 1
                ops.partial_channel_reduce(sets[i], mk, out=outs[i])

            t = time_call(call, 128)
            nbytes = 2.0 * T * Mr * H * 4
            red[f"M{Mr}"] = {"us": round(t * 1e3, 2), "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1), "bound": "latency"}
            del sets, outs
        res["reduce_only_f32"] = red
        # bf16 variant (the form the backward uses for G), out of place
        Yb = randn_bf16((T, 16384, H))
        ob = torch.empty_like(Yb)
        t = time_call(lambda: ops.partial_channel_reduce(Yb, mk, out=ob), 10)
        gbs = 2.0 * T * 16384 * H * 2 / (t * 1e-3) / 1e9
        res["reduce_only_bf16"] = {"M16384": {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1),
                                              "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}}
        del Yb, ob
        torch.cuda.empty_cache()

    # -------------------------------------------------- decode-shaped forward
    if "decode" in legs:
        dec = {}
        mk = mask_dev(H)
        nsets = 6  # 6 x 90 MB of weights: beyond the 256 MB last-level cache
        Ws = [randn_bf16((T, KR, H), 0.02) for _ in range(nsets)]
        dec_m = [int(x) for x in args.decode_m.split(",") if x]
        for Md in dec_m:
            Xs = [randn_bf16((T, Md, KR)) for _ in range(nsets)]
            outs = [torch.empty((T, Md, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
            wsd = torch.zeros(max(1, ops.fwd_workspace_bytes(T, Md, KR, H)), dtype=torch.uint8, device=dev)
            idx = [0]

            def call():
                i = idx[0] % nsets
                idx[0] += 1
                ops.rowpar_pcr_fwd(Xs[i], Ws[i], mk, out=outs[i], workspace=wsd)

            t = time_call(call, 60, warm=6)
            nbytes = 2.0 * (T * Md * KR + T * KR * H + T * Md * H)
            gbs = nbytes / (t * 1e-3) / 1e9
            dec[f"M{Md}"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        res["decode_down_proj"] = dec
        del Ws
        torch.cuda.empty_cache()

    if "mid" in legs:
        # forward of the 7B down-projection at a few hundred tokens (the split
        # forward: one workgroup per rank and tile, then a reduce pass);
        # weight sets rotate past the last-level cache
        mk = mask_dev(H)
        nsets = 6
        Ws = [randn_bf16((T, KR, H), 0.02) for _ in range(nsets)]
        mid = {}
        for Mm in (64, 128, 256, 512):
            Xs = [randn_bf16((T, Mm, KR)) for _ in range(nsets)]
            outs = [torch.empty((T, Mm, H), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
            wsm = torch.zeros(max(1, ops.fwd_workspace_bytes(T, Mm, KR, H)), dtype=torch.uint8, device=dev)
            idx = [0]

            def callm():
                i = idx[0] % nsets
                idx[0] += 1
                ops.rowpar_pcr_fwd(Xs[i], Ws[i], mk, out=outs[i], workspace=wsm)

            t = time_call(callm, 30, warm=6)
            flops = 2.0 * Mm * K * H
            nbytes = 2.0 * (T * Mm * KR + T * KR * H + T * Mm * H)
            roof_ms = max(flops / (PEAK_BF16_TFLOPS * 1e9), nbytes / (PEAK_HBM_GBS * 1e6))
            mid[f"M{Mm}"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(flops / (t * 1e-3) / 1e12, 1),
                             "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1), "frac_roof": round(roof_ms / t, 4)}
            del Xs, outs
        res["mid_tokens_fwd"] = mid
        del Ws
        torch.cuda.empty_cache()

    if "decode_out" in legs:
        # the attention out-projection (Kr = 512): 33.6 MB of weights; 16 sets
        # rotate (537 MB, beyond the last-level cache)
        mk = mask_dev(H)
        dec_m = [int(x) for x in args.decode_m.split(",") if x]
        deco = {}
        nso = 16
        Wo = [randn_bf16((T, KR_OUT, H), 0.02) for _ in range(nso)]
        for Md in dec_m:
            Xo = [randn_bf16((T, Md, KR_OUT)) for _ in range(nso)]
            oo = [torch.empty((T, Md, H), dtype=torch.bfloat16, device=dev) for _ in range(nso)]
            wso = torch.zeros(max(1, ops.fwd_workspace_bytes(T, Md, KR_OUT, H)), dtype=torch.uint8, device=dev)
            idx = [0]

            def callo():
                i = idx[0] % nso
                idx[0] += 1
                ops.rowpar_pcr_fwd(Xo[i], Wo[i], mk, out=oo[i], workspace=wso)

            t = time_call(callo, 64, warm=16)
            nbytes = 2.0 * (T * Md * KR_OUT + T * KR_OUT * H + T * Md * H)
            gbs = nbytes / (t * 1e-3) / 1e9
            deco[f"M{Md}"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        res["decode_out_proj"] = deco
        del Wo
        torch.cuda.empty_cache()

    # ------------------------------------------------ tensor-parallel sweep
    if "tsweep" in legs:
        # The same layer (M = 16384, K = 11008, H = 4096, p = 0.5 random mask)
        # split over T = 2, 4, 8, 16 ranks: Kr = K / T; the product's flops
        # stay 2MKH, the output (and the synced payload) grow with T.
        sweep = {}
        mk = mask_dev(H)
        K_all = T * KR
        for Ts in (2, 4, 8, 16):
            Krs = K_all // Ts
            Xs = randn_bf16((Ts, M, Krs))
            Ws = randn_bf16((Ts, Krs, H), 0.02)
            dZs = randn_bf16((Ts, M, H))
            outs = torch.empty((Ts, M, H), dtype=torch.bfloat16, device=dev)
            dXs, dWs = torch.empty_like(Xs), torch.empty_like(Ws)
            wss = torch.empty(ops.bwd_workspace_bytes(Ts, M, Krs, H), dtype=torch.uint8, device=dev)
            tf = time_call(lambda: ops.rowpar_pcr_fwd(Xs, Ws, mk, out=outs), 5)
            tb = time_call(lambda: ops.pcr_bwd(dZs, Xs, Ws, mk, dX=dXs, dW=dWs, workspace=wss), 5)
            sweep[f"T{Ts}"] = {"Kr": Krs, "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
                               "tflops": round(flops_step / ((tf + tb) * 1e-3) / 1e12, 2)}
            del Xs, Ws, dZs, outs, dXs, dWs, wss
            torch.cuda.empty_cache()
        res["t_sweep"] = sweep

    # ------------------------------------ column-parallel layer (per-rank input)
    if "colpar" in legs:
        # The Llama2-7B MLP up-projection as the column-parallel layer after
        # a partial channel-reduce: rank t multiplies its own activation
        # A_t [M, 4096] by its column slice [4096, 1376]; fwd + bwd.
        Kc, Nc = H, KR
        A = randn_bf16((T, M, Kc))
        W1 = randn_bf16((T, Kc, Nc), 0.02)
        dU = randn_bf16((T, M, Nc))
        U = torch.empty((T, M, Nc), dtype=torch.bfloat16, device=dev)
        dA, dW1 = torch.empty_like(A), torch.empty_like(W1)
        tf = time_call(lambda: ops.colpar_fwd(A, W1, out=U), 10)
        tb = time_call(lambda: ops.colpar_bwd(dU, A, W1, dA=dA, dW=dW1), 10)
        fc = 2.0 * M * Kc * Nc * T
        res["colpar_up_proj"] = {"K": Kc, "N_per_rank": Nc, "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
                                 "fwd_bwd_tflops": round(3 * fc / ((tf + tb) * 1e-3) / 1e12, 2)}
        del A, W1, dU, U, dA, dW1
        torch.cuda.empty_cache()

    # ------------------------------- residual update + RMS norm (per rank)
    if "norm" in legs:
        # The step after the partial reduce at the Llama2-7B shape: each rank
        # adds its activation to its residual stream and RMS-normalises it;
        # reads Z and R, writes the new residual and the normalised rows.
        Zn = randn_bf16((T, M, H))
        Rn = randn_bf16((T, M, H))
        gn = (1.0 + 0.1 * torch.randn((H,), generator=gen, device=dev)).to(torch.bfloat16)
        ro, no = torch.empty_like(Zn), torch.empty_like(Zn)
        t = time_call(lambda: ops.residual_rmsnorm(Zn, Rn, gn, 1e-5, r_out=ro, n_out=no), 10)
        nbytes = 4.0 * T * M * H * 2
        gbs = nbytes / (t * 1e-3) / 1e9
        res["residual_rmsnorm"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        del Zn, Rn, gn, ro, no
        torch.cuda.empty_cache()

    if "fwd_masks" in legs:
        # The 7B forward with the three kinds of sync set, in this order (a
        # counter run splits the forward's dispatches into three equal groups
        # by dispatch order): a random S, the first half of the channels, the
        # even channels.  Each kind: 2 warm-up calls, then 5 timed ones.
        Xm = randn_bf16((T, M, KR))
        Wm = randn_bf16((T, KR, H), 0.02)
        om = torch.empty((T, M, H), dtype=torch.bfloat16, device=dev)
        fm = {}
        for kind in MASK_ORDER:
            mkk = mask_dev(H, kind=kind)
            fm[kind] = round(time_call(lambda: ops.rowpar_pcr_fwd(Xm, Wm, mkk, out=om), 5), 4)
        res["fwd_masks_ms"] = fm
        log(f"forward by sync-set kind (ms): {fm}")
        del Xm, Wm, om
        torch.cuda.empty_cache()

    if "reduce_norm" in legs:
        # The partial channel-reduce of bf16 per-rank activations with the
        # residual update + RMS norm in its epilogue, against the two-kernel
        # chain it replaces (bf16 reduce writing Z, then the norm pass reading
        # it).  Algorithmic bytes: Y and R read, Rout and N written.
        Yr = randn_bf16((T, M, H))
        Rr = randn_bf16((T, M, H))
        gr = (1.0 + 0.1 * torch.randn((H,), generator=gen, device=dev)).to(torch.bfloat16)
        mkr = mask_dev(H)
        ro, no, zr = torch.empty_like(Yr), torch.empty_like(Yr), torch.empty_like(Yr)
        t_f = time_call(lambda: ops.reduce_residual_rmsnorm(Yr, mkr, Rr, gr, 1e-5, r_out=ro, n_out=no), 10)

        def chain():
            ops.partial_channel_reduce(Yr, mkr, out=zr)
            ops.residual_rmsnorm(zr, Rr, gr, 1e-5, r_out=ro, n_out=no)

        t_c = time_call(chain, 10)
        nbytes = 4.0 * T * M * H * 2
        gbs = nbytes / (t_f * 1e-3) / 1e9
        res["reduce_residual_rmsnorm"] = {
            "us": round(t_f * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "chain_us": round(t_c * 1e3, 2), "chain_bytes": 6.0 * T * M * H * 2, "bytes": nbytes,
        }
        log(f"reduce+residual+norm fused {t_f*1e3:.1f} us vs chain {t_c*1e3:.1f} us")
        del Yr, Rr, gr, ro, no, zr
        torch.cuda.empty_cache()

    # ------------------------------------ payload of the in-place reduce vs p
    if "payload" in legs:
        # In place with S = the first p*H channels, the reduce touches only
        # the synced channels: its traffic should scale with p (the payload
        # cut the pages claim for the partial reduce).  PAYLOAD_CALLS calls
        # per p, in the order of PAYLOAD_P (the counter summary relies on it).
        pay = {}
        Yp = torch.randn((T, 4096, H), generator=gen, device=dev, dtype=torch.float32)
        for pp in PAYLOAD_P:
            mkp = torch.from_numpy(synth.make_mask(H, pp, "prefix")).to(dev)
            for _ in range(PAYLOAD_CALLS):
                ops.partial_channel_reduce(Yp, mkp, inplace=True)
            torch.cuda.synchronize()
            t = time_call(lambda: ops.partial_channel_reduce(Yp, mkp, inplace=True), 5, warm=0)
            pay[f"p{pp}"] = {"us": round(t * 1e3, 2),
                             "GB/s_synced": round(2.0 * T * 4096 * H * 4 * pp / (t * 1e-3) / 1e9, 1)}
        res["payload_inplace_reduce"] = pay
        del Yp
        torch.cuda.empty_cache()

    # ------------------------------------------- copy of known size (counters)
    if "copy" in legs:
        # A plain streaming kernel of known size (1 GiB read, 1 GiB written;
        # an elementwise negation, so it is a kernel dispatch rather than a DMA
        # copy): the reference against which the HBM byte counters of the other
        # kernels are scaled.
        xs = torch.empty(COPY_ELEMS, dtype=torch.float32, device=dev).uniform_(generator=gen)
        ys = torch.empty_like(xs)
        t = time_call(lambda: torch.neg(xs, out=ys), 5)
        res["copy"] = {"bytes": 2 * COPY_ELEMS * 4, "us": round(t * 1e3, 1),
                       "GB/s": round(2 * COPY_ELEMS * 4 / (t * 1e-3) / 1e9, 1)}
        del xs, ys
        torch.cuda.empty_cache()

    # ------------------------------------------------------- CPU oracle leg
    cpu = None
    if not args.no_cpu_baseline and "train" in legs:
        cpu = cpu_baseline(args.cpu_sample_tokens)

    value = None
    if "ms_per_step" in res:
        value = flops_step / (res["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2) if value is not None else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res.get("ms_per_step", float("nan")), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Llama2-7B MLP down-projection, row-parallel + partial channel-reduce, fwd+bwd",
            "T": T, "M": M, "K": K, "Kr": KR, "H": H, "p": P, "mask": "random",
        },
        "mfma_frac": round(value / PEAK_BF16_TFLOPS, 4) if value is not None else None,
        "roofline": res.get("roofline"),
        "cpu_baseline": cpu,
        "kernels_ms": res.get("kernels_ms"),
        "fwd_tflops": res.get("fwd_tflops"),
        "bwd_tflops": res.get("bwd_tflops"),
        "prefix_mask": res.get("prefix_mask"),
        "library_gemm": res.get("library_gemm"),
        "out_proj": res.get("out_proj"),
        "model_shapes": res.get("model_shapes"),
        "reduce_only_f32": res.get("reduce_only_f32"),
        "reduce_only_bf16": res.get("reduce_only_bf16"),
        "t_sweep": res.get("t_sweep"),
        "colpar_up_proj": res.get("colpar_up_proj"),
        "residual_rmsnorm": res.get("residual_rmsnorm"),
        "reduce_residual_rmsnorm": res.get("reduce_residual_rmsnorm"),
        "fwd_masks_ms": res.get("fwd_masks_ms"),
        "decode_down_proj": res.get("decode_down_proj"),
        "decode_out_proj": res.get("decode_out_proj"),
        "mid_tokens_fwd": res.get("mid_tokens_fwd"),
        "payload_inplace_reduce": res.get("payload_inplace_reduce"),
        "copy": res.get("copy"),
        "src": src_hash(),
    }
    print(json.dumps(line), flush=True)


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` as recorded from the FETCH_SIZE and
    WRITE_SIZE counters (calibrated), if they were taken on the current kernel
    sources; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    cur = kernel_src_hash(kernel)
    for ln in lines:
        f = ln.strip().strip("`").split()
        if len(f) >= 4 and f[0] == "traffic" and f[1] == kernel and f[2] == f"src={cur}":
            return int(f[3].split("=")[1])
    return None


def _read_csv(path):
    import csv

    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def _short(name: str) -> str:
    n = name.split("(")[0]
    return n.replace("void ", "").replace("caat::", "")


def rocprof_stats_summary(d: str) -> str:
    """Markdown table of a `rocprofv3 --kernel-trace --stats --output-format csv` run."""
    rows = _read_csv(_find(d, "kernel_stats.csv"))
    out = ["| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| {} | {} | {:.1f} | {:.1f} | {:.1f} | {:.2f} |".format(
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def rocprof_mfma_summary(d: str) -> str:
    """Per-kernel MFMA busy fraction (MfmaUtil: MFMA busy cycles over all SIMDs'
    active cycles) and performed bf16 MFMA flops (SQ_INSTS_VALU_MFMA_MOPS_BF16
    x 512) per dispatch, the latter beside the GEMM's algorithmic 2*M*K*H."""
    acc = {}
    for r in _read_csv(_find(d, "counter_collection.csv")):
        acc.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    algo = 2.0 * M * (T * KR) * H
    out = ["| kernel | dispatches | MfmaUtil % | MFMA GFLOP per dispatch | / algorithmic 2MKH |",
           "|---|---|---|---|---|"]
    for k in sorted({k for k, _ in acc}):
        util = acc.get((k, "MfmaUtil"))
        mops = acc.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
        if not util or not mops or max(mops) == 0:
            continue
        fl = sum(mops) / len(mops) * 512
        out.append(f"| {_short(k)} | {len(util)} | {sum(util) / len(util):.1f} | {fl / 1e9:.1f} | {fl / algo:.3f} |")
    return "\n".join(out)


STALL_PASSES = (
    ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS",
     "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
    ("TCP_PENDING_STALL_CYCLES_sum", "TCP_TCP_TA_DATA_STALL_CYCLES_sum", "TCP_TCR_TCP_STALL_CYCLES_sum",
     "TCP_READ_TAGCONFLICT_STALL_CYCLES_sum", "GRBM_GUI_ACTIVE"),
    ("TA_TA_BUSY_sum", "TA_BUFFER_READ_LDS_WAVEFRONTS_sum", "TD_TD_BUSY_sum", "TCC_HIT_sum", "TCC_MISS_sum",
     "TCC_TAG_STALL_sum", "GRBM_GUI_ACTIVE"),
)


def rocprof_stall_summary(*dirs: str) -> str:
    """Where the products' copy path waits, from three counter passes
    (STALL_PASSES, one per directory).  GRBM_GUI_ACTIVE sums the 8 XCDs'
    active cycles, so one XCD's = GUI / 8; per-CU units (TCP, TA, TD, LDS) are
    normalised by 256 x that, SIMD-wide ones by 1024 x that."""
    per = []
    for d in dirs:
        acc = {}
        for r in _read_csv(_find(d, "counter_collection.csv")):
            acc.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        per.append({k: sum(v) / len(v) for k, v in acc.items()})
    kernels = sorted({k for k, _ in per[0]} & {k for k, _ in per[1]} & {k for k, _ in per[2]})
    kernels = [k for k in kernels if any(s in k for s in ("pcr_fwd", "pcr_bwd", "pcr_reduce"))]
    out = ["| kernel | MFMA busy | L1 stalled on L2 data | TA busy | TD busy | L2 hit rate | "
           "LDS bank-conflict cycles | wave cycles waiting (any / for issue) |",
           "|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        g = lambda i, c: per[i].get((k, c), float("nan"))
        cyc = [g(i, "GRBM_GUI_ACTIVE") / 8 for i in range(3)]
        hit, miss = g(2, "TCC_HIT_sum"), g(2, "TCC_MISS_sum")
        wc = g(0, "SQ_WAVE_CYCLES")
        out.append(
            f"| {_short(k)} | {g(0, 'SQ_VALU_MFMA_BUSY_CYCLES') / (cyc[0] * 1024):.2f} "
            f"| {g(1, 'TCP_PENDING_STALL_CYCLES_sum') / (cyc[1] * 256):.2f} "
            f"| {g(2, 'TA_TA_BUSY_sum') / (cyc[2] * 256):.2f} | {g(2, 'TD_TD_BUSY_sum') / (cyc[2] * 256):.2f} "
            f"| {hit / (hit + miss):.3f} | {g(0, 'SQ_LDS_BANK_CONFLICT') / (cyc[0] * 256):.4f} "
            f"| {g(0, 'SQ_WAIT_ANY') / wc:.2f} / {g(0, 'SQ_WAIT_INST_ANY') / wc:.2f} |")
    return "\n".join(out)


def rocprof_payload_summary(fetch_dir: str, write_dir: str) -> str:
    """Bytes per dispatch of the in-place fp32 reduce for each p of the payload
    leg (dispatches in order, PAYLOAD_CALLS + 5 per p, see the leg), scaled
    by what the counters read for the calibration kernel."""
    def series(d, counter):
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv")) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0))))
        red = [float(r["Counter_Value"]) for r in rows if "pcr_reduce_f32_kernel" in r["Kernel_Name"]]
        cal = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL_KEY in r["Kernel_Name"]]
        return red, sum(cal) / len(cal)

    fr, fc = series(fetch_dir, "FETCH_SIZE")
    wr, wc = series(write_dir, "WRITE_SIZE")
    known_kib = COPY_ELEMS * 4 / 1024.0
    sf, sw = known_kib / fc, known_kib / wc
    per = PAYLOAD_CALLS + 5  # dispatches per p: the untimed calls, then 5 timed ones (no warm-up)
    if len(fr) != per * len(PAYLOAD_P) or len(wr) != len(fr):
        raise SystemExit(f"unexpected reduce dispatch count {len(fr)} / {len(wr)}")
    full = 2.0 * T * 4096 * H * 4  # out-of-place bytes of the whole tensor
    out = [f"scale: FETCH_SIZE x{sf:.4f}, WRITE_SIZE x{sw:.4f} (calibration kernel, {COPY_ELEMS * 4} bytes each way)", "",
           "| p | HBM read MB | HBM write MB | total MB | / total at p = 1 | synced bytes 2*T*M*H*4*p, MB |",
           "|---|---|---|---|---|---|"]
    tot = {}
    for i, pp in enumerate(PAYLOAD_P):
        f = sum(fr[i * per:(i + 1) * per]) / per * sf * 1024
        w = sum(wr[i * per:(i + 1) * per]) / per * sw * 1024
        tot[pp] = (f, w)
    t1 = sum(tot[1.0])
    for pp in PAYLOAD_P:
        f, w = tot[pp]
        out.append(f"| {pp} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / 1e6:.1f} | {(f + w) / t1:.3f} | {full * pp / 1e6:.1f} |")
    return "\n".join(out)


def rocprof_traffic_summary(fetch_dir: str, write_dir: str) -> str:
    """Per-kernel FETCH_SIZE / WRITE_SIZE averages (KiB per dispatch) and the
    HBM bytes per launch they imply once scaled by what the same counters read
    for the calibration kernel (known to move COPY_ELEMS*4 bytes each way)."""
    def per_kernel(d, counter):
        acc = {}
        for r in _read_csv(_find(d, "counter_collection.csv")):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            acc.setdefault(k, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    fetch, nf = per_kernel(fetch_dir, "FETCH_SIZE")
    write, _ = per_kernel(write_dir, "WRITE_SIZE")
    copy_k = [k for k in fetch if COPY_KERNEL_KEY in k]
    if not copy_k:
        raise SystemExit("calibration kernel not found in the FETCH_SIZE run")
    ck = copy_k[0]
    known_kib = COPY_ELEMS * 4 / 1024.0
    sf, sw = known_kib / fetch[ck], known_kib / write[ck]
    out = [
        f"calibration kernel: {_short(ck)} moving {COPY_ELEMS * 4} bytes each way",
        f"FETCH_SIZE reads {fetch[ck]:.0f} KiB -> scale {sf:.4f}; WRITE_SIZE reads {write[ck]:.0f} KiB -> scale {sw:.4f}",
        "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |",
        "|---|---|---|---|---|---|",
    ]
    lines = []
    for k in sorted(fetch, key=lambda k: -fetch[k]):
        if k not in write:
            continue
        rb, wb = fetch[k] * sf * 1024, write[k] * sw * 1024
        out.append(f"| {_short(k)} | {nf[k]} | {fetch[k]:.0f} | {write[k]:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
        base = _short(k).split("<")[0]
        if base in KERNEL_SOURCES:
            lines.append(f"`traffic {base} src={kernel_src_hash(base)} bytes={int(rb + wb)} read={int(rb)} write={int(wb)}`")
    return "\n".join(out + ["", "Machine-readable (kernel, hash of that kernel's sources, calibrated bytes per dispatch):", ""]
                     + [ln + "  " for ln in lines])


def rocprof_masks_summary(fetch_dir: str, write_dir: str) -> str:
    """The 256x256 forward's FETCH_SIZE / WRITE_SIZE per sync-set kind: its
    dispatches in dispatch order split into len(MASK_ORDER) equal groups
    (the fwd_masks leg runs one kind after the other), scaled by what the
    counters read for the calibration kernel."""
    def series(d, counter):
        rows = [r for r in _read_csv(_find(d, "counter_collection.csv")) if r["Counter_Name"] == counter]
        fw = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                    if "rowpar_pcr_fwd_kernel<256, 256, 8>" in r["Kernel_Name"])
        cp = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL_KEY in r["Kernel_Name"]]
        return [v for _, v in fw], sum(cp) / len(cp)

    fetch, cf = series(fetch_dir, "FETCH_SIZE")
    write, cw = series(write_dir, "WRITE_SIZE")
    known_kib = COPY_ELEMS * 4 / 1024.0
    sf, sw = known_kib / cf, known_kib / cw
    n = len(fetch) // len(MASK_ORDER)
    out_b = T * M * H * 2
    algo = 2.0 * M * T * KR + 2.0 * T * KR * H + out_b
    lines = [f"calibration: FETCH_SIZE scale {sf:.4f}, WRITE_SIZE scale {sw:.4f}; {n} dispatches per kind",
             "",
             "| sync set | HBM read MB | HBM write MB | write / output bytes | read + write / algorithmic bytes |",
             "|---|---|---|---|---|"]
    for i, kind in enumerate(MASK_ORDER):
        f = fetch[i * n:(i + 1) * n]
        w = write[i * n:(i + 1) * n]
        rb = sum(f) / len(f) * sf * 1024
        wb = sum(w) / len(w) * sw * 1024
        lines.append(f"| {kind} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {wb / out_b:.3f} | {(rb + wb) / algo:.3f} |")
    return "\n".join(lines)


def cpu_baseline(tokens: int):
    """The CPU oracle (fp64 numpy) on a bounded sample of the same workload:
    forward + backward of the down-projection for `tokens` of the 16384 tokens."""
    import numpy as np

    import oracle
    from partial_channel_reduce_amd import synth

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    host_cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    log(f"cpu oracle on {tokens} tokens, {threads} BLAS threads of {host_cores} host cores ({model})")
    X, W = synth.make_fwd_inputs(T, tokens, KR, H, seed=0)
    dZ = synth.make_grad(T, tokens, H, seed=0)
    mask = synth.make_mask(H, P, "random", seed=0)
    t0 = time.perf_counter()
    oracle.rowpar_pcr_fwd(X, W, mask)
    oracle.pcr_bwd(dZ, X, W, mask)
    dt = time.perf_counter() - t0
    flops = 6.0 * tokens * (T * KR) * H
    return {
        "value": round(flops / dt / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cores": host_cores,
        "cpu_model": model,
        "elementwise_threads": 1,
        "kind": "oracle",
        "sample": f"fwd+bwd of {tokens} of {M} tokens (T={T}, Kr={KR}, H={H}, p={P}), fp64 numpy, {dt:.1f} s",
    }


if __name__ == "__main__":
    main()
