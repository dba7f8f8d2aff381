#!/usr/bin/env python3
"""Benchmark of the decoupled-head attention forward on one MI355X.

One step = one attention forward (QK^T, mask, online softmax, P.V, output) of
the chosen workload variant over inputs already resident in HBM.  Prints one
JSON line with throughput (TFLOP/s of algorithmic work), the roofline
position of the kernel, tokens/s, the same measurement for the comparator
head configurations at the same shape (SQA speedup vs MHA/GQA), and the fp64
CPU oracle timed on a bounded sample of the same workload on the host cores.

Default workload: encoder_s32k (B=1, S=32768, d=128, non-causal), SQA variant
H_q=H_kv=8, with the 16-head MHA run as the comparator.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_BYTES_PER_S = 8.0e12
KERNEL_SOURCES = ["reduced_query_head_amd/csrc/attn_fwd.hip", "reduced_query_head_amd/csrc/device_common.h"]


def algorithmic_flops(B, S, H_q, d, causal):
    """2*d flops for q.k plus 2*d for p*v per visible (query, key) pair."""
    pairs = S * (S + 1) // 2 if causal else S * S
    return 4 * B * H_q * d * pairs


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, variant):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_bf16_{workload}_{variant}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def time_variant(sqa, torch, w, variant, steps, warmup):
    import inputs.configs as cfg
    v = w.variant(variant)
    q, k, vv, _ = cfg.make_inputs(w, variant)
    dq, dk, dv = (torch.from_numpy(a).view(torch.bfloat16).to("cuda") for a in (q, k, vv))
    del q, k, vv
    out = torch.empty_like(dq)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        sqa.attn_fwd(dq, dk, dv, out=out, scale=w.scale, causal=w.causal, stream=stream)
    torch.cuda.synchronize()
    # per-launch HIP events on the launch stream, plus the whole timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        sqa.attn_fwd(dq, dk, dv, out=out, scale=w.scale, causal=w.causal, stream=stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    flops = algorithmic_flops(w.B, w.S, v.H_q, w.d, w.causal)
    total_ms = ev[0].elapsed_time(ev[steps])
    res = dict(H_q=v.H_q, H_kv=v.H_kv, flops=flops, ms_per_step=total_ms / steps,
               avg_launch_ms=sum(per_launch) / steps, min_launch_ms=min(per_launch),
               max_launch_ms=max(per_launch), wall_s=wall)
    res["tflops"] = flops / (res["ms_per_step"] * 1e-3) / 1e12
    res["tokens_per_s"] = w.B * w.S / (res["ms_per_step"] * 1e-3)
    del dq, dk, dv, out
    torch.cuda.empty_cache()
    return res


def time_backward(sqa, torch, w, variant, steps, warmup):
    """Times sqa.attn_bwd (row statistics, dq kernel, dk/dv kernel) on the
    forward's own output and log-normaliser, with a seeded N(0,1) upstream
    gradient.  Credited work: 10*d flops per visible (query, key) pair -- the
    score recompute, dP = dO.V^T, dQ, dK and dV products -- 2.5x the forward."""
    import inputs
    import inputs.configs as cfg
    v = w.variant(variant)
    q, k, vv, _ = cfg.make_inputs(w, variant)
    g = inputs.normal(w.seed(variant), 5, q.shape, "bf16", 1.0)
    dq_, dk_, dv_, dg = (torch.from_numpy(a).view(torch.bfloat16).to("cuda") for a in (q, k, vv, g))
    del q, k, vv, g
    stream = torch.cuda.current_stream()
    out, lse = sqa.attn_fwd(dq_, dk_, dv_, scale=w.scale, causal=w.causal, stream=stream, return_lse=True)
    gq, gk, gv = torch.empty_like(dq_), torch.empty_like(dk_), torch.empty_like(dv_)
    ws = torch.empty(sqa.attn_bwd_workspace_size(w.B, w.S, v.H_q), dtype=torch.uint8, device="cuda")

    def run():
        sqa.attn_bwd(dq_, dk_, dv_, out, dg, lse, scale=w.scale, causal=w.causal, stream=stream,
                     dq=gq, dk=gk, dv=gv, workspace=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    flops = algorithmic_flops(w.B, w.S, v.H_q, w.d, w.causal) * 10 // 4
    ms = ev[0].elapsed_time(ev[steps]) / steps
    del dq_, dk_, dv_, dg, out, lse, gq, gk, gv, ws
    torch.cuda.empty_cache()
    return {"workload": f"{w.name}/{variant}", "flops_credited": flops, "ms_per_step": round(ms, 4),
            "min_ms": round(min(per), 4), "max_ms": round(max(per), 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "pct_peak": round(100 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "kernels": "bwd_stats_bf16 + bwd_dq_bf16 + bwd_dkdv_bf16 (one sqa_attn_bwd call)"}


def time_decode(sqa, torch, wname, steps, warmup):
    """Decode (one token per sequence against its K/V cache) for every head
    configuration of the decode workload, on the same cache lengths.
    Algorithmic bytes per call: the valid part of the K and V caches
    (sum_b len_b * H_kv * d * 2 tensors * 2 bytes) plus q, out and lse; the
    call is bound by HBM bandwidth (8 TB/s)."""
    from inputs.configs import DECODE_WORKLOADS, decode_lengths, make_decode_inputs
    w = DECODE_WORKLOADS[wname]
    res = {}
    for var in w.variants:
        q, k, v, lens = make_decode_inputs(w, var.name)
        dq_, dk_, dv_ = (torch.from_numpy(a).view(torch.bfloat16).to("cuda") for a in (q, k, v))
        dl = torch.from_numpy(lens.astype("int32")).to("cuda")
        del q, k, v
        out = torch.empty_like(dq_)
        lse = torch.empty((w.B, var.H_q), dtype=torch.float32, device="cuda")
        ws = torch.empty(sqa.attn_decode_workspace_size(w.B, w.S_max, var.H_q, var.H_kv, w.d), dtype=torch.uint8,
                         device="cuda")
        stream = torch.cuda.current_stream()

        def run():
            sqa.attn_decode(dq_, dk_, dv_, seqlens=dl, out=out, lse=lse, scale=w.scale, stream=stream, workspace=ws)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            run()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        ms = sum(per) / steps
        nbytes = int(lens.sum()) * var.H_kv * w.d * 2 * 2 + 2 * w.B * var.H_q * w.d * 2 + w.B * var.H_q * 4
        res[var.name] = {"H_q": var.H_q, "H_kv": var.H_kv, "ms_per_call": round(ms, 4), "min_ms": round(min(per), 4),
                         "bytes_per_call": nbytes, "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                         "frac_hbm_peak": round(nbytes / (ms * 1e-3) / PEAK_HBM_BYTES_PER_S, 4),
                         "tokens_per_s": round(w.B / (ms * 1e-3), 1)}
        del dq_, dk_, dv_, dl, out, lse, ws
        torch.cuda.empty_cache()
    return {"workload": w.name, "B": w.B, "S_max": w.S_max, "d": w.d,
            "cache_lengths": [int(x) for x in decode_lengths(w.seed(w.variants[0].name), w.B, w.S_max,
                                                             w.min_len_frac)], "variants": res,
            "kernels": "attn_decode_split_bf16 + attn_decode_combine_bf16 (one sqa_attn_decode call)"}


def time_layer(sqa, torch, wname, steps, warmup):
    """Full attention layer (fused q/k/v projection GEMM, attention, output
    projection GEMM) for every head configuration of the layer workload.
    Credited work: 2*M*d_model*(H_q + 2 H_kv)*d + 2*M*H_q*d*d_model for the
    projections (M = B*S tokens) plus the attention's 4*d flops per visible
    (query, key) pair and query head."""
    from inputs.configs import LAYER_WORKLOADS, make_layer_inputs
    w = LAYER_WORKLOADS[wname]
    res = {}
    for var in w.variants:
        x, wq, wo = make_layer_inputs(w, var.name)
        dx, dwq, dwo = (torch.from_numpy(a).view(torch.bfloat16).to("cuda") for a in (x, wq, wo))
        del x, wq, wo
        out = torch.empty_like(dx)
        ws = torch.empty(sqa.layer_workspace_size(w.B, w.S, var.H_q, var.H_kv, w.d), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream()

        def run():
            sqa.layer_fwd(dx, dwq, dwo, var.H_q, var.H_kv, out=out, scale=w.scale, causal=w.causal, stream=stream,
                          workspace=ws)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            run()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[steps]) / steps
        M = w.B * w.S
        proj = 2 * M * w.d_model * (var.H_q + 2 * var.H_kv) * w.d + 2 * M * var.H_q * w.d * w.d_model
        att = algorithmic_flops(w.B, w.S, var.H_q, w.d, w.causal)
        res[var.name] = {"H_q": var.H_q, "H_kv": var.H_kv, "ms_per_layer": round(ms, 4),
                         "tokens_per_s": round(M / (ms * 1e-3), 1), "flops": proj + att,
                         "tflops": round((proj + att) / (ms * 1e-3) / 1e12, 2)}
        del dx, dwq, dwo, out, ws
        torch.cuda.empty_cache()
    if "mha" in res:
        for k, r in res.items():
            r["speedup_vs_mha"] = round(res["mha"]["ms_per_layer"] / r["ms_per_layer"], 3)
    return {"workload": w.name, "B": w.B, "S": w.S, "d_model": w.d_model, "d": w.d, "causal": w.causal,
            "variants": res, "kernels": "hipBLASLt GEMM + attn_fwd_bf16 + hipBLASLt GEMM (one sqa_layer_fwd call)"}


def gemm_context(torch, n=8192, iters=10):
    """A plain bf16 GEMM from the vendor library on random N(0,1) data, as a
    practical reference for dense bf16 throughput on this GPU (the chip is
    power-limited, so random operands run below the nominal peak)."""
    g = torch.Generator(device="cuda").manual_seed(1)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del a, b
    torch.cuda.empty_cache()
    return {"op": f"torch.matmul bf16 {n}x{n}x{n}, random N(0,1)", "tflops": round(2 * n ** 3 / ms / 1e9, 1)}


def cpu_baseline(w, variant, budget_s):
    """The fp64 oracle, unchanged, on a bounded sample of query positions of
    the same workload (all batches and heads of each sampled position)."""
    import numpy as np

    import inputs.configs as cfg
    import oracle

    v = w.variant(variant)
    q, k, vv, _ = cfg.make_inputs(w, variant)
    rng = np.random.default_rng(w.seed(variant))
    rows_all = rng.permutation(w.S)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    done, flops, t_used, i = [], 0, 0.0, 0
    chunk = max(threads, 8)
    while t_used < budget_s and i < w.S:
        rows = np.sort(rows_all[i:i + chunk])
        t0 = time.perf_counter()
        oracle.attention(q, k, vv, w.scale, causal=w.causal, rows=rows, n_threads=threads)
        t_used += time.perf_counter() - t0
        keys = (rows + 1) if w.causal else np.full(rows.size, w.S)
        flops += int(4 * w.B * v.H_q * w.d * keys.sum())
        done.append(rows.size)
        i += chunk
    n_rows = sum(done)
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_rows} of {w.S} query positions (seeded random, all {w.B} batch x {v.H_q} "
                      f"heads each) of {w.name}/{variant}; {t_used:.1f} s of oracle time; "
                      f"full run extrapolated: {algorithmic_flops(w.B, w.S, v.H_q, w.d, w.causal) / (flops / t_used):.0f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="encoder_s32k")
    ap.add_argument("--variant", default="sqa")
    ap.add_argument("--comparators", default="auto",
                    help="comma list of variants timed beside it, 'auto' = all others, 'none'")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--backward", choices=["auto", "none", "only"], default="auto",
                    help="time the backward too (auto: bf16 workloads), or only it")
    ap.add_argument("--long", choices=["auto", "none"], default="auto",
                    help="also time the 131k causal and 200k ragged workloads (SQA and comparators)")
    ap.add_argument("--decode", choices=["auto", "none", "only"], default="auto",
                    help="time the decode workload too (auto), or only it")
    ap.add_argument("--decode-workload", default="decode_s128k")
    ap.add_argument("--layer", choices=["auto", "none", "only"], default="auto",
                    help="time the full attention layer too (auto), or only it")
    ap.add_argument("--layer-workload", default="layer_s32k")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: libsqa runs on one GPU only; --gpus must be 1 "
              "(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import reduced_query_head_amd as sqa
    from inputs.configs import WORKLOADS

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    w = WORKLOADS[args.workload]
    sqa.load_library()
    if args.layer == "only":
        print(json.dumps({"layer": time_layer(sqa, torch, args.layer_workload, args.steps, args.warmup)}),
              flush=True)
        return
    if args.decode == "only":
        print(json.dumps({"decode": time_decode(sqa, torch, args.decode_workload, args.steps, args.warmup)}),
              flush=True)
        return
    if args.backward == "only":
        print(json.dumps({"backward": time_backward(sqa, torch, w, args.variant, args.steps, args.warmup)}),
              flush=True)
        return
    main_res = time_variant(sqa, torch, w, args.variant, args.steps, args.warmup)
    comps = {}
    names = [v.name for v in w.variants if v.name != args.variant] if args.comparators == "auto" else (
        [] if args.comparators == "none" else args.comparators.split(","))
    for name in names:
        comps[name] = time_variant(sqa, torch, w, name, max(3, args.steps // 2), args.warmup)
        comps[name]["sqa_speedup"] = comps[name]["ms_per_step"] / main_res["ms_per_step"]
        comps[name]["ideal_speedup"] = comps[name]["H_q"] / main_res["H_q"]

    achieved = main_res["flops"] / (main_res["avg_launch_ms"] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_from_profile(w.name, args.variant),
                "kernel": f"attn_fwd_bf16<d={w.d},causal={int(w.causal)}>",
                "flops_per_launch": main_res["flops"], "avg_launch_ms": round(main_res["avg_launch_ms"], 4)}
    longctx = None
    if args.long == "auto" and args.workload == "encoder_s32k":
        longctx = {}
        for wn in ("causal_s131k", "ragged_s200k"):
            lw = WORKLOADS[wn]
            rs = {vv.name: time_variant(sqa, torch, lw, vv.name, 5, 2) for vv in lw.variants}
            first = lw.variants[0].name
            longctx[wn] = {k: {"H_q": r["H_q"], "H_kv": r["H_kv"], "ms_per_step": round(r["ms_per_step"], 3),
                               "tflops": round(r["tflops"], 1),
                               "pct_peak": round(100 * r["tflops"] / PEAK_BF16_TFLOPS, 2),
                               "tokens_per_s": round(r["tokens_per_s"], 1),
                               "sqa_speedup": round(r["ms_per_step"] / rs[first]["ms_per_step"], 3) if k != first else 1.0}
                           for k, r in rs.items()}
    bwd = (time_backward(sqa, torch, w, args.variant, max(3, args.steps // 2), args.warmup)
           if args.backward == "auto" and w.dtype == "bf16" else None)
    dec = time_decode(sqa, torch, args.decode_workload, 20, 3) if args.decode == "auto" else None
    lay = time_layer(sqa, torch, args.layer_workload, 5, 2) if args.layer == "auto" else None
    cpu = cpu_baseline(w, args.variant, args.cpu_budget) if args.cpu_budget > 0 else None
    gemm = gemm_context(torch) if args.cpu_budget > 0 else None
    v = w.variant(args.variant)
    line = {
        "metric": "attn-fwd TFLOP/s (% bf16 MFMA peak) + tokens/s at 32k-200k, SQA vs MHA/GQA",
        "value": round(main_res["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}/{args.variant}", "B": w.B, "S": w.S, "H_q": v.H_q, "H_kv": v.H_kv,
                   "d": w.d, "causal": w.causal, "scale": w.scale},
        "pct_peak": round(100 * main_res["tflops"] / peak, 2),
        "tokens_per_s": round(main_res["tokens_per_s"], 1),
        "comparators": {k: {"H_q": c["H_q"], "H_kv": c["H_kv"], "tflops": round(c["tflops"], 2),
                            "ms_per_step": round(c["ms_per_step"], 4),
                            "tokens_per_s": round(c["tokens_per_s"], 1),
                            "sqa_speedup": round(c["sqa_speedup"], 3), "ideal_speedup": c["ideal_speedup"]}
                        for k, c in comps.items()},
        "roofline": roofline,
        "long_context": longctx,
        "backward": bwd,
        "decode": dec,
        "layer": lay,
        "cpu_baseline": cpu,
        "pages_claim": "SQA abstract: up to 3x throughput on 32k-200k sequences; hardware not named",
        "context_library_gemm": gemm,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
