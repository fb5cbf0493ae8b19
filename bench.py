#!/usr/bin/env python3
"""Benchmark of the fine-grained-scaled FP8 GEMM path on one MI355X.

Default workload (one "step"): the dense NT sweep -- M in {64, 4096} x the six
(N, K) shapes (2112,7168) (24576,1536) (32768,512) (7168,16384) (4096,7168)
(7168,2048), e4m3 A/B with 1x128 / 128x128 fp32 scales, C bf16 -- twelve
dg_fp8_gemm_nt calls, each on its own resident inputs.  Value = algorithmic
flops of the step / step time, in TFLOPS.

Other workloads (--config): 0 the single M=128 N=2112 K=7168 GEMM, 2 the
contiguous grouped GEMM (8 groups), 3 the masked grouped GEMM (32 groups),
4 the FP8xFP4 expert FFN.

Caches: one step touches more than 1 GB of distinct inputs and outputs, so no
shape's operands survive in the 4 MB L2s or the 256 MB Infinity Cache until
that shape runs again; --flush additionally writes a 512 MB buffer before
every step (outside the timed region is impossible per call, so it is only
used with --per-call timing).

Prints ONE JSON line (rank 0, N=1).
"""

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense FP4/FP6 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--shape", type=str, default=None,
                    help="M,N,K: time only this dense shape (C bf16), for profiling")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("fp8_gemm.hip", "dg_device.hpp", "ffn.hip"):
        p = os.path.join(ROOT, "fp4_gemm_dense_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def dense_shapes(config):
    import synth
    if config == 0:
        return [(128, 2112, 7168, False, synth.seed_for(0, 0))]
    out = []
    for mi, M in enumerate(synth.DENSE_M):
        for j, (N, K) in enumerate(synth.DENSE_NK):
            out.append((M, N, K, True, synth.seed_for(1, mi * 6 + j)))
    return out


def build_dense(config, only=None):
    import torch
    import synth
    items = []
    shapes = dense_shapes(config)
    if only is not None:
        M, N, K = (int(v) for v in only.split(","))
        shapes = [(M, N, K, True, 12345)]
    for (M, N, K, with_c, seed) in shapes:
        g = synth.gen_dense(M, N, K, seed, with_c=with_c, backend="torch", device="cuda")
        g["d"] = torch.empty(M, N, dtype=torch.int16, device="cuda")
        flops = 2.0 * M * N * K
        nbytes = M * K + N * K + 4 * (K // 128) * M + 4 * ((N + 127) // 128) * (K // 128) + 2 * M * N * (2 if with_c else 1)
        items.append(dict(g=g, flops=flops, bytes=nbytes, label=f"M{M}_N{N}_K{K}", shape=(M, N, K)))
    return items


def run_dense_item(dg, it):
    g = it["g"]
    dg.dg_fp8_gemm_nt(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], g["d"])


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# ----------------------------------------------------------------------------

def cpu_baseline_dense(items, budget_s):
    import numpy as np
    import synth
    from oracle import ref as R
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = 1
    rows_per_shape = 64
    host = []
    for it in items:
        g = it["g"]
        M, N, K = it["shape"]
        r = min(M, rows_per_shape)
        host.append(dict(a=synth.to_numpy(g["a"][:r]), sfa=synth.to_numpy(g["sfa"][:, :r]),
                         b=synth.to_numpy(g["b"]), sfb=synth.to_numpy(g["sfb"]),
                         c=None if g["c"] is None else synth.to_numpy(g["c"][:r]),
                         flops=2.0 * r * N * K))
    flops = 0.0
    t0 = time.perf_counter()
    done = 0
    for h in host:
        R.fp8_gemm_nt(h["a"], h["sfa"], h["b"], h["sfb"], h["c"])
        flops += h["flops"]
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"numpy fp64 oracle (dequantise + matmul) on the first {rows_per_shape} rows of "
                      f"{done} of the {len(items)} sweep shapes, full N and K; {dt:.1f} s",
            "seconds": dt}


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import fp4_gemm_dense_amd as dg
    dg.load_library()
    torch.cuda.init()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calib:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n}))
        return

    if args.config not in (0, 1):
        raise SystemExit("configs 2-4 are benchmarked by their own scripts in this version")

    items = build_dense(args.config, args.shape)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        for it in items:
            run_dense_item(dg, it)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    n = len(items)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, it in enumerate(items):
            run_dense_item(dg, it)
            ev[s][i + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    per = []
    for i, it in enumerate(items):
        durs = [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]
        med = statistics.median(durs)
        per.append(dict(shape=it["label"], ms=med, tflops=it["flops"] / med / 1e9,
                        gbs=it["bytes"] / med / 1e6,
                        roofline_frac=max(it["flops"] / 1e12 / PEAK_FP8_TFLOPS, it["bytes"] / 1e9 / PEAK_HBM_GBS)
                        / (med / 1e3)))
    step_flops = sum(it["flops"] for it in items)
    value = step_flops / (ms_per_step / 1e3) / 1e12

    # dominant kernel: the launches that use the largest tile (the M=4096 shapes)
    plans = [dg.dg_query_plan(*it["shape"]) for it in items]
    dom_kid = max(set(p["kernel_id"] for p in plans),
                  key=lambda k: sum(per[i]["ms"] for i, p in enumerate(plans) if p["kernel_id"] == k))
    dom = [i for i, p in enumerate(plans) if p["kernel_id"] == dom_kid]
    dom_flops = sum(items[i]["flops"] for i in dom) / len(dom)
    dom_ms = sum(statistics.mean(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) for i in dom) / len(dom)
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            if tj.get("kernel_source_hash") == kernel_source_hash() and tj.get("config") == args.config:
                traffic = tj.get("bytes_per_launch")
        except Exception:
            traffic = None
    bm, bn = plans[dom[0]]["block_m"], plans[dom[0]]["block_n"]
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
                "kernel": f"fp8_gemm_kernel tile {bm}x{bn} (dense)", "launches_per_step": len(dom)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(items, args.cpu_budget_s)

    workload = ("dense NT sweep M{64,4096} x (N,K){(2112,7168),(24576,1536),(32768,512),(7168,16384),"
                "(4096,7168),(7168,2048)}, e4m3 1x128/128x128 fp32 scales, C bf16"
                if args.config == 1 else "dense NT M128 N2112 K7168, e4m3 1x128/128x128 fp32 scales, C=0")
    out = {
        "metric": "block-scaled FP8 GEMM TFLOPS + % MFMA peak (dense, grouped, masked)",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp8e4m3 -> f32 acc, bf16 out",
        "data": "synthetic (seeded N(0,1), quantised per 1x128 / 128x128)",
        "config": {"workload": workload, "gemms_per_step": len(items), "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "mfma_peak_frac": round(value / PEAK_FP8_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "per_shape": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in p.items()} for p in per],
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
