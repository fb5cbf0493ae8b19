#!/usr/bin/env python3
"""Benchmark of the fine-grained-scaled FP8 / FP8xFP4 GEMM path on one MI355X.

Default workload (--config all), one "step" = every FP8 form the metric names,
each call on its own resident inputs:
  * dense M=128 N=2112 K=7168, C = 0 (the pages' featured shape);
  * the dense NT sweep -- M in {64, 4096} x the six (N, K) shapes (2112,7168)
    (24576,1536) (32768,512) (7168,16384) (4096,7168) (7168,2048); C bf16;
  * the M-grouped contiguous GEMM, 8 groups from 32768 routed rows, (N,K) in
    {(4096,7168), (7168,2048)};
  * the M-grouped masked GEMM, 32 groups x 256 rows, masked_m ~ U{0..256}, the
    same (N,K) pairs;
all with e4m3 A/B and 1x128 / 128x128 fp32 scales: seventeen calls.
value = algorithmic flops of the step / the summed time of its calls (TFLOPS);
"forms" reports each form on its own with its roofline.

Other workloads (one form per run):
  --config 0  dense M=128 N=2112 K=7168, C = 0
  --config 1  the dense NT sweep alone
  --config 2  M-grouped contiguous, 8 groups from 32768 routed rows, (N,K) in
              {(4096,7168), (7168,2048)}
  --config 3  M-grouped masked, 32 groups x 256 rows, masked_m ~ U{0..256},
              same (N,K) pairs
  --config 4  FP8xFP4 expert FFN, 4096 tokens, hidden 7168, intermediate 2048,
              32 local experts of 256, top-8
  --config 5  M-grouped FP8xFP4 GEMM, contiguous, 8 groups from 32768 routed rows,
              (N,K) in {(4096,7168), (7168,2048)}: config 2 with E2M1 weights
              (UE8M0 per 1x32) and UE8M0 activation scales per 1x128
  --config 6  the config-1 dense sweep with packed UE8M0 scales (power-of-two,
              A per 1x128, B per 128x128), applied by the scaled matrix instruction
  --config 7  config 2 in the NN layout (each group's B stored [K, N])
  --config 8  K-grouped GEMM in the TN layout: 8 groups from 32768 tokens (a
              weight-gradient shape), (M,N) in {(4096,7168), (7168,2048)}

Caches: each call is timed in a batch over rotating copies of its inputs and
outputs (as many as make 768 MB of distinct data, at least one), so no call
finds its operands in the 4 MB L2s or the 256 MB Infinity Cache: every call
starts from HBM.  A timed batch needs one pair of events (which alone read
about 4.6 us on this system) for many calls.

Algorithmic work: flops = 2 * (valid rows) * N * K (the FFN counts linear1 and
linear2 over routed pairs); bytes = every distinct operand and scale byte read
once plus valid outputs written once (re-reads, padding rows and workspace
traffic excluded).  Timing: HIP events on the launch stream around each
call's batch, inside one timed region of K steps bracketed by device
synchronisation; per call the median and the minimum over the steps are
reported, and ms_per_step is the mean over the steps of the summed per-call
times (step_wall_ms, the whole region over K, is reported too).

Prints ONE JSON line.
"""

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense FP4/FP6 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

METRIC = "block-scaled FP8 GEMM TFLOPS + % MFMA peak (dense, grouped, masked)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=str, default="all", choices=["all"] + [str(i) for i in range(9)])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--shape", type=str, default=None,
                    help="M,N,K: time only this dense shape (C bf16), for profiling")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--only", type=str, default=None,
                    help="time only the calls of one kernel group (e.g. 'contiguous 128x256'), for counter runs")
    ap.add_argument("--summarize-counters", nargs=5,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CALIB_FETCH_DIR", "CALIB_WRITE_DIR", "KEY"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of `--only KEY` and one of "
                         "--copy-calib into calibrated HBM bytes per call, stored under KEY in "
                         "profiles/traffic.json")
    return ap.parse_args()


def kernel_source_hash(kind):
    """Hash of the sources that decide the kernels (and their plans) a workload kind runs."""
    h = hashlib.sha256()
    files = (("ffn.hip", "dg_device.hpp", "dg_internal.hpp") if kind in ("ffn", "fp4_contiguous")
             else ("fp8_gemm.hip", "fp8_gemm_wide.hip", "skinny.hip", "planner.cpp", "api.cpp", "dg_device.hpp",
                   "dg_internal.hpp"))
    for f in files:
        p = os.path.join(ROOT, "fp4_gemm_dense_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def nb(n):
    return (n + 127) // 128


def _ws(form, m, n, k, groups=1, expected_m=0):
    """Workspace for one call, allocated once outside the timed region (None: not needed)."""
    import torch
    import fp4_gemm_dense_amd as dg
    need = dg.dg_fp8_gemm_workspace_bytes(form, m, n, k, groups, expected_m)
    return torch.empty(need, dtype=torch.uint8, device="cuda") if need else None


def _tile(plan):
    return f"{plan['block_m']}x{plan['block_n']}"


# Calls are timed in batches over rotating copies of their inputs and outputs:
# a batch touches at least this many distinct bytes (three times the 256 MB
# Infinity Cache), so every call finds its operands in HBM, not in a cache.
ROTATE_BYTES = 768 << 20


def _replicas(g, d, nbytes):
    """[(inputs, output)] copies for one call: g and d, then device copies of them."""
    import torch
    n = max(1, min(64, -(-ROTATE_BYTES // max(int(nbytes), 1))))
    out = [(g, d)]
    for _ in range(n - 1):
        out.append(({k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in g.items()}, torch.empty_like(d)))
    return out


# ----------------------------------------------------------------------------
# workloads: each item = one library call with its algorithmic flops / bytes
# ----------------------------------------------------------------------------

def items_dense(config, only=None):
    import torch
    import synth
    import fp4_gemm_dense_amd as dg
    if only is not None:
        M, N, K = (int(v) for v in only.split(","))
        shapes = [(M, N, K, True, 12345)]
    elif config == 0:
        shapes = [(128, 2112, 7168, False, synth.seed_for(0, 0))]
    else:
        shapes = [(M, N, K, True, synth.seed_for(config, mi * 6 + j))
                  for mi, M in enumerate(synth.DENSE_M) for j, (N, K) in enumerate(synth.DENSE_NK)]
    ue = config == 6          # packed UE8M0 scales
    kind = "dense_ue8m0" if ue else ("dense_small" if config == 0 else "dense")
    items = []
    for (M, N, K, with_c, seed) in shapes:
        gen = synth.gen_dense_ue8m0 if ue else synth.gen_dense
        g = gen(M, N, K, seed, with_c=with_c, backend="torch", device="cuda")
        d = torch.empty(M, N, dtype=torch.int16, device="cuda")
        kw = (K // 128 + 3) // 4
        sf_bytes = 4 * kw * (M + nb(N)) if ue else 4 * (K // 128) * (M + nb(N))
        nbytes = M * K + N * K + sf_bytes + 2 * M * N * (2 if with_c else 1)
        gemm = dg.dg_fp8_gemm_nt_ue8m0 if ue else dg.dg_fp8_gemm_nt
        ws = _ws(dg.FORM_NT_UE8M0 if ue else dg.FORM_NT, M, N, K)
        plan = dg.dg_query_plan_form(dg.FORM_NT_UE8M0 if ue else dg.FORM_NT, M, N, K)

        def mk(g, d, gemm=gemm, ws=ws):
            return lambda: gemm(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d, workspace=ws)
        items.append(dict(kind=kind, runs=[mk(*r) for r in _replicas(g, d, nbytes)], g=g, flops=2.0 * M * N * K, bytes=nbytes, label=f"M{M}_N{N}_K{K}",
                          shape=(M, N, K), plan=plan, kernel=f"{kind} {_tile(plan)}"))
    return items


def items_contiguous(nn=False):
    import torch
    import synth
    import fp4_gemm_dense_amd as dg
    items = []
    gen = synth.gen_contiguous_nn if nn else synth.gen_contiguous
    gemm = dg.dg_m_grouped_fp8_gemm_nn_contiguous if nn else dg.dg_m_grouped_fp8_gemm_nt_contiguous
    kind = "contiguous_nn" if nn else "contiguous"
    for j, (N, K) in enumerate(synth.GROUPED_NK):
        g = gen(8, 32768, N, K, synth.seed_for(7 if nn else 2, j), backend="torch", device="cuda")
        M = g["M"]
        d = torch.empty(M, N, dtype=torch.int16, device="cuda")
        valid = sum(g["counts"])
        groups_hit = sum(1 for c in g["counts"] if c > 0)
        nbytes = valid * K + groups_hit * (N * K + 4 * nb(N) * (K // 128)) + 4 * (K // 128) * valid + 4 * M + 2 * valid * N
        ws = _ws(dg.FORM_CONTIGUOUS_NN if nn else dg.FORM_CONTIGUOUS_NT, M, N, K, 8)
        plan = dg.dg_query_plan_form(dg.FORM_CONTIGUOUS_NN if nn else dg.FORM_CONTIGUOUS_NT, M, N, K, 8)

        def mk(g, d, ws=ws):
            return lambda: gemm(g["a"], g["sfa"], g["b"], g["sfb"], g["m_indices"], d, workspace=ws)
        items.append(dict(kind=kind, runs=[mk(*r) for r in _replicas(g, d, nbytes)], g=g, flops=2.0 * valid * N * K, bytes=nbytes,
                          label=f"G8_contig{'_nn' if nn else ''}_N{N}_K{K}", shape=(M, N, K), plan=plan,
                          kernel=f"{kind} {_tile(plan)}"))
    return items


def items_kgrouped():
    import torch
    import synth
    import fp4_gemm_dense_amd as dg
    items = []
    for j, (M, N) in enumerate(synth.GROUPED_NK):
        g = synth.gen_kgrouped_tn(8, 32768, M, N, synth.seed_for(8, j), backend="torch", device="cuda")
        K = g["K"]
        d = torch.empty(8, M, N, dtype=torch.int16, device="cuda")
        valid = sum(g["counts"])
        nbytes = K * (M + N) + 4 * (K // 128) * (M + nb(N)) + 4 * 8 + 2 * 8 * M * N

        def mk(g, d):
            return lambda: dg.dg_k_grouped_fp8_gemm_tn_contiguous(g["a"], g["sfa"], g["b"], g["sfb"], g["ks"], d)
        items.append(dict(kind="kgrouped", runs=[mk(*r) for r in _replicas(g, d, nbytes)], g=g, flops=2.0 * valid * M * N, bytes=nbytes,
                          label=f"G8_kgrouped_tn_M{M}_N{N}", shape=(M, N, K), kernel="kgrouped"))
    return items


def items_masked():
    import torch
    import synth
    import fp4_gemm_dense_amd as dg
    items = []
    for j, (N, K) in enumerate(synth.GROUPED_NK):
        g = synth.gen_masked(32, 256, N, K, synth.seed_for(3, j), backend="torch", device="cuda")
        mm = [int(v) for v in g["masked_m"].cpu()]
        d = torch.empty(32, 256, N, dtype=torch.int16, device="cuda")
        valid = sum(mm)
        groups_hit = sum(1 for v in mm if v > 0)
        nbytes = valid * K + groups_hit * (N * K + 4 * nb(N) * (K // 128)) + 4 * (K // 128) * valid + 4 * 32 + 2 * valid * N
        ws = _ws(dg.FORM_MASKED_NT, 256, N, K, 32, 128)

        def mk(g, d, ws=ws):
            return lambda: dg.dg_m_grouped_fp8_gemm_nt_masked(g["a"], g["sfa"], g["b"], g["sfb"], g["masked_m"], d,
                                                              128, workspace=ws)
        items.append(dict(kind="masked", runs=[mk(*r) for r in _replicas(g, d, nbytes)], g=g, flops=2.0 * valid * N * K, bytes=nbytes,
                          label=f"G32_masked_N{N}_K{K}", shape=(256, N, K), masked_m=mm, kernel="masked"))
    return items


def items_fp4_contiguous():
    import torch
    import synth
    import fp4_gemm_dense_amd as dg
    items = []
    for j, (N, K) in enumerate(synth.GROUPED_NK):
        g = synth.gen_fp4_contiguous(8, 32768, N, K, synth.seed_for(5, j), backend="torch", device="cuda")
        M = g["M"]
        d = torch.empty(M, N, dtype=torch.int16, device="cuda")
        valid = sum(g["counts"])
        groups_hit = sum(1 for c in g["counts"] if c > 0)
        nbytes = (valid * K + groups_hit * (N * K // 2 + N * (K // 32)) + valid * 4 * ((K // 128 + 3) // 4)
                  + 4 * M + 2 * valid * N)
        g["b_sf_t"] = dg.dg_transform_fp4_weight_sf(g["b_sf"])     # weight pre-transform, once per weight set

        def mk(g, d):
            return lambda: dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(g["a"], g["a_sf"], g["b"], g["b_sf_t"],
                                                                      g["m_indices"], d)
        items.append(dict(kind="fp4_contiguous", runs=[mk(*r) for r in _replicas(g, d, nbytes)], g=g, flops=2.0 * valid * N * K, bytes=nbytes,
                          label=f"G8_fp4_contig_N{N}_K{K}", shape=(M, N, K), kernel="fp4_contiguous"))
    return items


def items_ffn():
    import torch
    import synth
    import fp4_gemm_dense_amd as dg
    T, H, I, E = 4096, 7168, 2048, 32
    g = synth.gen_ffn(T=T, H=H, I=I, num_local=E, num_experts=256, topk=8, seed=synth.seed_for(4, 0),
                      backend="torch", device="cuda")
    idx = g["topk_idx"]
    local = (idx >= 0) & (idx < E)
    P = int(local.sum())
    hit = torch.bincount(idx[local].long(), minlength=E)
    experts_hit = int((hit > 0).sum())
    k = idx.shape[1]
    ws = torch.empty(dg.dg_fp8_fp4_expert_ffn_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, H, dtype=torch.int16, device="cuda")
    w_bytes = experts_hit * (2 * I * H // 2 + 2 * I * (H // 32) + H * I // 2 + H * (I // 32))
    nbytes = w_bytes + T * H + T * (H // 128) + T * k * 8 + T * H * 2

    # weight pre-transform, once per weight set (outside the timed step)
    (g["w1t"], g["w1_sft"]), (g["w2t"], g["w2_sft"]) = dg.transform_weights_for_expert_ffn(
        (g["w1"], g["w1_sf"]), (g["w2"], g["w2_sf"]))

    def mk(g, y):
        return lambda: dg.dg_fp8_fp4_expert_ffn(g["x"], g["x_sf"], g["topk_idx"], g["topk_w"], g["w1t"], g["w1_sft"],
                                                g["w2t"], g["w2_sft"], y, 0, ws)
    return [dict(kind="ffn", runs=[mk(*r) for r in _replicas(g, y, nbytes)], g=g, flops=2.0 * P * (2 * I * H + H * I), bytes=nbytes,
                 label=f"ffn_T{T}_H{H}_I{I}_E{E}_pairs{P}", shape=(T, H, I), pairs=P, kernel="ffn")]


# ----------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the same workload)
# ----------------------------------------------------------------------------

def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def cpu_baseline(items, budget_s):
    """Time the oracle, as it stands, on a bounded sample of the same inputs: passes over
    successive row slices until about 0.7 x budget_s seconds of oracle time."""
    t_total = 0.0
    flops = 0.0
    desc = []
    t_start = time.perf_counter()
    target_s = 0.7 * budget_s        # oracle seconds to aim for; passes take further row slices
    npass = 0
    while t_total < target_s and time.perf_counter() - t_start < budget_s:
        t_total, flops = _cpu_pass(items, budget_s, t_start, npass, t_total, flops, desc)
        npass += 1
    return {"value": flops / max(t_total, 1e-9) / 1e12, "unit": "TFLOPS", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"numpy fp64 oracle (dequantise + matmul), {npass} pass(es) over: " + "; ".join(desc) +
                      f"; {t_total:.1f} s of oracle time; input generation and host copies excluded",
            "cpu": cpu_model(), "seconds": round(t_total, 2)}


def _cpu_pass(items, budget_s, t_start, npass, t_total, flops, desc):
    """One pass of the oracle over a slice of every item; pass p takes the p-th slice of rows."""
    import numpy as np
    import synth
    from oracle import ref as R
    for it in items:
        if time.perf_counter() - t_start > budget_s:
            break
        g = it["g"]
        kind = it["kind"]
        if kind in ("dense_small", "dense", "dense_ue8m0"):
            ue = kind == "dense_ue8m0"
            M, N, K = it["shape"]
            r = min(M, 64)
            r0 = (npass * r) % M
            r = min(r, M - r0)
            if "_np_b" not in it:      # B is copied to the host once, not per pass
                it["_np_b"] = (synth.to_numpy(g["b"]), synth.to_numpy(g["sfb"]))
            b, sfb = it["_np_b"]
            a = synth.to_numpy(g["a"][r0:r0 + r])
            sfa = synth.to_numpy(g["sfa"][r0:r0 + r] if ue else g["sfa"][:, r0:r0 + r])
            c = None if g["c"] is None else synth.to_numpy(g["c"][r0:r0 + r])
            t0 = time.perf_counter()
            (R.fp8_gemm_nt_ue8m0 if ue else R.fp8_gemm_nt)(a, sfa, b, sfb, c)
            t_total += time.perf_counter() - t0
            flops += 2.0 * r * N * K
            if npass == 0:
                desc.append(f"{r} rows of {it['label']}")
        elif kind == "kgrouped":
            M, N, K = it["shape"]
            ks = synth.to_numpy(g["ks"]).tolist()
            rows = np.arange(16 * npass, 16 * npass + 16) % M
            k0 = 0
            for kg in ks:
                if time.perf_counter() - t_start > budget_s:
                    break
                if kg > 0:
                    b0, b1 = k0 // 128, (k0 + kg) // 128
                    a = synth.to_numpy(g["a"][k0:k0 + kg][:, rows])
                    sfa = synth.to_numpy(g["sfa"][b0:b1][:, rows])
                    b = synth.to_numpy(g["b"][k0:k0 + kg])
                    sfb = synth.to_numpy(g["sfb"][:, b0:b1])
                    t0 = time.perf_counter()
                    R.fp8_gemm_tn(a, sfa, b, sfb)
                    t_total += time.perf_counter() - t0
                    flops += 2.0 * len(rows) * N * kg
                k0 += kg
            if npass == 0:
                desc.append(f"16 output rows of every group of {it['label']}")
        elif kind == "fp4_contiguous":
            M, N, K = it["shape"]
            mi = synth.to_numpy(g["m_indices"])
            for grp in range(8):
                if time.perf_counter() - t_start > budget_s:
                    break
                rows = np.nonzero(mi == grp)[0][16 * npass:16 * npass + 16]
                if len(rows) == 0:
                    continue
                a, a_sf = synth.to_numpy(g["a"][rows]), synth.to_numpy(g["a_sf"][rows])
                b, b_sf = synth.to_numpy(g["b"][grp]), synth.to_numpy(g["b_sf"][grp])
                t0 = time.perf_counter()
                R.fp8_fp4_gemm_nt(a, a_sf, b, b_sf)
                t_total += time.perf_counter() - t0
                flops += 2.0 * len(rows) * N * K
            if npass == 0:
                desc.append(f"up to 16 valid rows per group of {it['label']}")
        elif kind in ("contiguous", "contiguous_nn", "masked"):
            M, N, K = it["shape"]
            masked = kind == "masked"
            G = 32 if masked else 8
            for grp in range(G):
                if time.perf_counter() - t_start > budget_s:
                    break
                if not masked:
                    rows = np.nonzero(synth.to_numpy(g["m_indices"]) == grp)[0]
                    rows = rows[16 * npass:16 * npass + 16]
                    a, sfa = synth.to_numpy(g["a"][rows]), synth.to_numpy(g["sfa"][:, rows])
                else:
                    r0 = min(16 * npass, it["masked_m"][grp])
                    r1 = min(r0 + 16, it["masked_m"][grp])
                    rows = np.arange(r0, r1)
                    a, sfa = synth.to_numpy(g["a"][grp, r0:r1]), synth.to_numpy(g["sfa"][grp][:, r0:r1])
                if len(rows) == 0:
                    continue
                b, sfb = synth.to_numpy(g["b"][grp]), synth.to_numpy(g["sfb"][grp])
                t0 = time.perf_counter()
                (R.fp8_gemm_nn if kind == "contiguous_nn" else R.fp8_gemm_nt)(a, sfa, b, sfb)
                t_total += time.perf_counter() - t0
                flops += 2.0 * len(rows) * N * K
            if npass == 0:
                desc.append(f"up to 16 valid rows per group of {it['label']}")
        else:
            T, H, I = it["shape"]
            idx = synth.to_numpy(g["topk_idx"])
            toks = np.nonzero((idx < 32).any(1))[0][12 * npass:12 * npass + 12]
            sub = {k: synth.to_numpy(g[k][toks]) for k in ("x", "x_sf", "topk_idx", "topk_w")}
            w = {k: synth.to_numpy(g[k]) for k in ("w1", "w1_sf", "w2", "w2_sf")}
            pairs = int((sub["topk_idx"] < 32).sum())
            t0 = time.perf_counter()
            R.expert_ffn(sub["x"], sub["x_sf"], sub["topk_idx"], sub["topk_w"], w["w1"], w["w1_sf"], w["w2"],
                         w["w2_sf"], 0, 32)
            t_total += time.perf_counter() - t0
            flops += 2.0 * pairs * (2 * I * H + H * I)
            if npass == 0:
                desc.append(f"{len(toks)} tokens ({pairs} local pairs) per pass of {it['label']}")
    return t_total, flops


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------

WORKLOADS = {
    "all": "one step of every FP8 form: dense NT M128 N2112 K7168 (C=0); dense NT sweep M{64,4096} x "
           "(N,K){(2112,7168),(24576,1536),(32768,512),(7168,16384),(4096,7168),(7168,2048)} (C bf16); "
           "M-grouped contiguous, 8 groups from 32768 routed rows (multinomial, padded to 128), "
           "(N,K){(4096,7168),(7168,2048)}; M-grouped masked, 32 groups x 256 rows, masked_m ~ U{0..256}, "
           "(N,K){(4096,7168),(7168,2048)}; e4m3 1x128 / 128x128 fp32 scales",
    "0": "dense NT M128 N2112 K7168, e4m3 1x128 / 128x128 fp32 scales, C=0",
    "1": "dense NT sweep M{64,4096} x (N,K){(2112,7168),(24576,1536),(32768,512),(7168,16384),(4096,7168),"
         "(7168,2048)}, e4m3 1x128 / 128x128 fp32 scales, C bf16",
    "2": "M-grouped contiguous, 8 groups from 32768 routed rows (multinomial, padded to 128), "
         "(N,K){(4096,7168),(7168,2048)}, e4m3 1x128 / 128x128 fp32 scales",
    "3": "M-grouped masked, 32 groups x 256 rows, masked_m ~ U{0..256}, (N,K){(4096,7168),(7168,2048)}, "
         "e4m3 1x128 / 128x128 fp32 scales",
    "4": "FP8xFP4 expert FFN, 4096 tokens, hidden 7168, intermediate 2048, 32 local experts of 256, top-8, "
         "e4m3 activations (UE8M0/128), E2M1 weights (UE8M0/32)",
    "5": "M-grouped FP8xFP4 GEMM, contiguous, 8 groups from 32768 routed rows (multinomial, padded to 128), "
         "(N,K){(4096,7168),(7168,2048)}, e4m3 activations (UE8M0/128), E2M1 weights (UE8M0/32)",
    "6": "dense NT GEMM sweep, M{64,4096} x (N,K){(2112,7168),(24576,1536),(32768,512),(7168,16384),(4096,7168),"
         "(7168,2048)}, C bf16, e4m3 with packed UE8M0 scales (A 1x128, B 128x128, power-of-two amax/448)",
    "7": "M-grouped contiguous GEMM in the NN layout (B stored [K,N]), 8 groups from 32768 routed rows "
         "(multinomial, padded to 128), (N,K){(4096,7168),(7168,2048)}, e4m3 1x128 / 128x128 fp32 scales",
    "8": "K-grouped GEMM, TN layout (A [K,M], B [K,N], one D per group), 8 groups from 32768 tokens "
         "(multinomial, padded to 128), (M,N){(4096,7168),(7168,2048)}, e4m3 1x128 / 128x128 fp32 scales",
}

FORM_NAMES = {"dense_small": "dense M128 N2112 K7168", "dense": "dense sweep", "contiguous": "contiguous grouped",
              "masked": "masked grouped", "ffn": "FP8xFP4 expert FFN", "fp4_contiguous": "FP8xFP4 contiguous grouped",
              "dense_ue8m0": "dense sweep, UE8M0 scales", "contiguous_nn": "contiguous grouped, NN layout",
              "kgrouped": "K-grouped TN"}


def build_items(cfg, shape=None):
    if shape is not None:
        return items_dense(1, shape)
    if cfg == "all":
        return items_dense(0) + items_dense(1) + items_contiguous() + items_masked()
    c = int(cfg)
    if c in (0, 1, 6):
        return items_dense(c)
    if c in (2, 7):
        return items_contiguous(nn=c == 7)
    if c == 3:
        return items_masked()
    if c == 5:
        return items_fp4_contiguous()
    if c == 8:
        return items_kgrouped()
    return items_ffn()


def roofline_time(it):
    """Seconds the call takes at the roofline: the larger of its MFMA and HBM times."""
    return max(it["flops"] / 1e12 / PEAK_FP8_TFLOPS, it["bytes"] / 1e9 / PEAK_HBM_GBS)


def bound_of(it):
    return "mfma" if it["flops"] / 1e12 / PEAK_FP8_TFLOPS >= it["bytes"] / 1e9 / PEAK_HBM_GBS else "hbm"


def roofline_of(group, traffic=None):
    """Roofline of a group of launches of one kernel: algorithmic flops (MFMA-bound) or
    bytes (HBM-bound) per launch over the group's mean launch time."""
    t_ms = sum(it["mean_ms"] for it in group) / len(group)
    time_mfma = sum(it["mean_ms"] for it in group if bound_of(it) == "mfma")
    bound = "mfma" if time_mfma * 2 >= sum(it["mean_ms"] for it in group) else "hbm"
    if bound == "mfma":
        per_launch = sum(it["flops"] for it in group) / len(group)
        achieved = per_launch / (t_ms / 1e3) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
             "frac": round(achieved / PEAK_FP8_TFLOPS, 4)}
    else:
        per_launch = sum(it["bytes"] for it in group) / len(group)
        achieved = per_launch / (t_ms / 1e3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved / PEAK_HBM_GBS, 4)}
    r.update({"traffic": traffic, "kernel": group[0]["kernel"], "launches_per_step": len(group),
              "avg_launch_ms": round(t_ms, 5), "algorithmic_per_launch": per_launch})
    return r


def lookup_traffic(key, kind):
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(tfile):
        return None
    try:
        entry = json.load(open(tfile)).get(key)
    except (ValueError, OSError):
        return None
    if entry and entry.get("kernel_source_hash") == kernel_source_hash(kind):
        return entry.get("bytes_per_launch")
    return None


def summarize_counters(fetch_dir, write_dir, calib_fetch_dir, calib_write_dir, key):
    """Calibrated HBM bytes per call of the kernel group `key` (e.g. "contiguous 128x256"),
    from two rocprofv3 --pmc runs of `bench.py --only <key>` (FETCH_SIZE, then WRITE_SIZE)
    and two of `bench.py --copy-calib` (the same two counters).  The library's dispatches of a
    call (GEMM plus split-K reduce, or the FFN's four kernels) are summed; torch's own
    kernels (the cache flush, input generation) are left out.  Each counter is scaled by
    what it reads for the plain 1 GiB copy."""
    import csv
    import glob

    def per_kernel(d, counter):
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter:
                    acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return acc

    def copy_bytes(acc):
        vals = [v for k, vs in acc.items() if "copy" in k.lower() or "elementwise" in k.lower() for v in vs]
        return statistics.median(vals) if vals else float("nan")

    n = 1 << 30
    fetch_scale = n / copy_bytes(per_kernel(calib_fetch_dir, "FETCH_SIZE"))
    write_scale = n / copy_bytes(per_kernel(calib_write_dir, "WRITE_SIZE"))
    kind = key.split(" ")[0]
    # one dispatch per call names the call: the FFN's routing kernel, else the GEMM
    # kernel (square, wide, skinny or FP8xFP4); split-K reduces and the K-grouped
    # zeroing kernel ride along
    primary = ("route",) if kind == "ffn" else ("gemm_kernel", "gemm_wide_kernel")

    def per_call(acc):
        lib = {k: v for k, v in acc.items() if "dg::" in k and "transpose" not in k}   # (weight set-up excluded)
        calls = sum(len(v) for k, v in lib.items() if any(s in k for s in primary) and "reduce" not in k)
        return sum(sum(v) for v in lib.values()) / max(calls, 1), sorted(lib)
    fb, kernels = per_call(per_kernel(fetch_dir, "FETCH_SIZE"))
    wb, _ = per_call(per_kernel(write_dir, "WRITE_SIZE"))
    entry = {"kernel_source_hash": kernel_source_hash(kind),
             "bytes_per_launch": int(fb * fetch_scale + wb * write_scale),
             "fetch_bytes": int(fb * fetch_scale), "write_bytes": int(wb * write_scale),
             "kernels": kernels, "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)}
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    tj = json.load(open(tfile)) if os.path.exists(tfile) else {}
    tj[key] = entry
    with open(tfile, "w") as f:
        json.dump(tj, f, indent=1)
    print(json.dumps({key: entry}))


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only (no multi-GPU path); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import fp4_gemm_dense_amd as dg
    dg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calib:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "dispatches": 3}))
        return

    cfg = args.config
    items = build_items(cfg, args.shape)
    if args.only is not None:
        items = [it for it in items if it["kernel"] == args.only]
        if not items:
            sys.exit(f"--only {args.only!r}: no call of this workload uses that kernel group")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for w in range(args.warmup):
        for it in items:
            for run in it["runs"]:
                run()
    torch.cuda.synchronize()

    n = len(items)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        for i, it in enumerate(items):
            ev[s][i][0].record(stream)
            for run in it["runs"]:
                run()
            ev[s][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_wall_ms = t_start.elapsed_time(t_end) / args.steps

    per = []
    for i, it in enumerate(items):
        durs = [ev[s][i][0].elapsed_time(ev[s][i][1]) / len(it["runs"]) for s in range(args.steps)]
        it["durs"] = durs
        it["mean_ms"] = statistics.mean(durs)
        it["med_ms"] = med = statistics.median(durs)
        it["min_ms"] = mn = min(durs)
        per.append(dict(shape=it["label"], form=it["kind"], kernel=it["kernel"], batch=len(it["runs"]), ms=med,
                        min_ms=mn,
                        tflops=it["flops"] / med / 1e9, gbs=it["bytes"] / med / 1e6,
                        mfma_frac=it["flops"] / med / 1e9 / PEAK_FP8_TFLOPS,
                        hbm_frac=it["bytes"] / med / 1e6 / PEAK_HBM_GBS,
                        bound=bound_of(it), roofline_frac=roofline_time(it) / (med / 1e3)))
    ms_per_step = statistics.mean(sum(ev[s][i][0].elapsed_time(ev[s][i][1]) / len(items[i]["runs"])
                                      for i in range(n)) for s in range(args.steps))
    step_flops = sum(it["flops"] for it in items)
    value = step_flops / (ms_per_step / 1e3) / 1e12

    # per-form results, each with the roofline of its dominant kernel
    forms = {}
    for kind in dict.fromkeys(it["kind"] for it in items):
        group = [it for it in items if it["kind"] == kind]
        t_med = sum(it["med_ms"] for it in group)
        t_min = sum(it["min_ms"] for it in group)
        kern = max(dict.fromkeys(it["kernel"] for it in group),
                   key=lambda k: sum(it["mean_ms"] for it in group if it["kernel"] == k))
        dom = [it for it in group if it["kernel"] == kern]
        forms[kind] = {
            "name": FORM_NAMES[kind], "calls": len(group),
            "tflops": round(sum(it["flops"] for it in group) / t_med / 1e9, 2),
            "tflops_min_time": round(sum(it["flops"] for it in group) / t_min / 1e9, 2),
            "gbs": round(sum(it["bytes"] for it in group) / t_med / 1e6, 1),
            "ms_median": round(t_med, 4), "ms_min": round(t_min, 4),
            "roofline_frac": round(sum(roofline_time(it) for it in group) / (t_med / 1e3), 4),
            "roofline": roofline_of(dom, lookup_traffic(kern, kind)),
        }
    # the step's dominant kernel: the largest share of the step's time
    kern = max(dict.fromkeys(it["kernel"] for it in items),
               key=lambda k: sum(it["mean_ms"] for it in items if it["kernel"] == k))
    dom = [it for it in items if it["kernel"] == kern]
    roof = roofline_of(dom, lookup_traffic(kern, dom[0]["kind"]))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(items, args.cpu_budget_s)

    fp4 = cfg in ("4", "5")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 -> f32" if fp4 else "fp8e4m3 x fp8e4m3 -> f32",
        "data": "synthetic (seeded N(0,1), quantised as the workload states)",
        "config": {"workload": WORKLOADS[cfg] if args.shape is None else f"dense NT {args.shape}",
                   "calls_per_step": n, "parallelism": "none (1 GPU)",
                   "cache": "cold: each call timed in a batch over rotating copies of >= 768 MB of operands"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "forms": forms,
        "mfma_peak_frac": round(value / PEAK_FP8_TFLOPS, 4),
        "step_wall_ms": round(step_wall_ms, 4),
        "wall_s_timed": round(wall, 3),
        "per_call": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in p.items()} for p in per],
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
