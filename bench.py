#!/usr/bin/env python3
"""Benchmark: sparsely-gated MoE layer forward on one MI355X.

One step = one whole layer forward (moe_forward: route -> dispatch -> expert
FFN -> combine, plus the balancing losses) over one batch of seeded synthetic
tokens already resident in HBM. Default workload: the Switch-style top-1 layer
(T=16384, d_model=768, d_ff=3072, E=128, capacity factor 1.25, GELU, bf16).

Prints ONE JSON line with throughput (tokens/s), the roofline of the dominant
step (the expert FFN: both grouped GEMM launches and the tile map, timed with
HIP events on the stream they run on) and the CPU oracle's throughput on a
bounded sample of the same workload, timed on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 78.6  # fp32 FMA without packed-fp32 instructions (157.3 with them)
METRIC = "MoE layer fwd tokens/s (1 GPU) + % bf16 MFMA peak in expert GEMM"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="switch_top1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0, help="target CPU seconds for the oracle sample")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per expert-FFN launch measured with rocprofv3 counters")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain copy kernel of this size before timing (counter calibration)")
    ap.add_argument("--pmc-report", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into --traffic-json")
    ap.add_argument("--stats-report", metavar="KERNEL_STATS_CSV",
                    help="print a rocprofv3 --stats kernel_stats.csv as a markdown table")
    return ap.parse_args()


def ffn_algorithmic(cfg, counts_kept, elt):
    """Algorithmic work of one moe_expert_ffn launch: the weights of every expert
    that has rows (W1 + W2), the permuted input rows read and the output rows
    written; the hidden activations are an intermediate and not counted."""
    import numpy as np

    R = int(np.sum(counts_kept))
    live = int(np.count_nonzero(counts_kept))
    w_bytes = live * 2 * cfg.d_model * cfg.d_ff * elt
    io_bytes = 2 * R * cfg.d_model * elt
    flops = 4.0 * R * cfg.d_model * cfg.d_ff
    return R, w_bytes + io_bytes, flops


def cpu_baseline(cfg, inp, budget_s):
    """The oracle as it stands, on a bounded sample: routing and dispatch of the
    whole batch, then the expert FFN and combine of the first n tokens; the
    whole-batch time is extrapolated linearly in n."""
    import numpy as np

    import oracle

    spec = oracle.LayerSpec.of(cfg)
    t0 = time.perf_counter()
    r = oracle.route(spec, inp)
    C = oracle.capacity(cfg.T, cfg.E, cfg.k, cfg.capacity_factor)
    disp = oracle.dispatch(r["topk_idx"], cfg.E, C)
    t_route = time.perf_counter() - t0

    def ffn_combine(n):
        tokens = np.arange(n, dtype=np.int32)
        slots = disp["slot_dest"][tokens]
        kept = slots >= 0
        rows_tok = np.repeat(tokens, cfg.k).reshape(-1, cfg.k)[kept]
        rows_exp = r["topk_idx"][tokens][kept]
        t = time.perf_counter()
        yp = oracle.expert_ffn_rows(inp["x"], rows_tok, rows_exp, inp["w1"], inp["w2"], cfg.act, cfg.dtype)
        row_of_slot = np.full(max(disp["R"], 1), -1, np.int32)
        row_of_slot[slots[kept]] = np.arange(rows_tok.shape[0], dtype=np.int32)
        oracle.combine(tokens, disp["slot_dest"], r["topk_gate"], yp if yp.size else np.zeros((1, cfg.d_model)),
                       row_of_slot)
        return time.perf_counter() - t

    n0 = min(cfg.T, 64)
    t_probe = ffn_combine(n0)
    per_tok = t_probe / n0
    n = int(min(cfg.T, max(n0, (budget_s - t_route) / max(per_tok, 1e-9))))
    t_ffn = ffn_combine(n) if n > n0 else t_probe
    total = t_route + t_ffn * cfg.T / n
    return {
        "value": cfg.T / total,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"routing + dispatch of all {cfg.T} tokens ({t_route:.2f} s), expert FFN + combine of the "
                   f"first {n} tokens ({t_ffn:.2f} s), whole-batch time extrapolated linearly in tokens"),
    }


def source_hash() -> str:
    """Hash of the HIP sources: counter data taken on other sources is stale."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparsely_gated_mixture_gate_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def pmc_report(fetch_dir, write_dir, out_json, config, calib_mib):
    """Per-launch HBM bytes of the expert FFN (GEMM1 + GEMM2 + tile map) from
    two rocprofv3 --pmc runs, each scaled by what the counter reads for a
    plain copy kernel of calib_mib MiB (which reads and writes that much)."""
    import csv
    import glob

    def per_kernel(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(f)))
        out = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def mean(d, pred):
        vals = [v for k, vs in d.items() if pred(k) for v in vs]
        return sum(vals) / len(vals) if vals else None

    is_copy = lambda k: "elementwise_kernel" in k and "MulFunctor" in k  # noqa: E731
    kib = calib_mib * 1024.0
    f_scale = kib / mean(fetch, is_copy)
    w_scale = kib / mean(write, is_copy)
    def applies_act(k):
        # grouped_gemm_bf16_kernel<BM, BN, BK, NSTAGE, ACT, APPLY_ACT, SKIP> / grouped_gemm_f32_kernel<ACT, APPLY_ACT>
        targs = [t.strip() for t in k[k.index("<") + 1:k.index(">")].split(",")]
        return targs[5] == "true" if "bf16" in k else targs[1] == "true"

    parts = {}
    for tag, pred in (("gemm1", lambda k: "grouped_gemm" in k and applies_act(k)),
                      ("gemm2", lambda k: "grouped_gemm" in k and not applies_act(k)),
                      ("tile_map", lambda k: "tile_map_kernel" in k)):
        f_kib, w_kib = mean(fetch, pred), mean(write, pred)
        parts[tag] = {"fetch_bytes": f_kib * 1024 * f_scale, "write_bytes": w_kib * 1024 * w_scale,
                      "fetch_kib_raw": f_kib, "write_kib_raw": w_kib}
    total = sum(p["fetch_bytes"] + p["write_bytes"] for p in parts.values())
    try:
        with open(out_json) as fh:
            tj = json.load(fh)
    except (OSError, ValueError):
        tj = {}
    tj["current_hash"] = source_hash()
    tj[config] = {"source_hash": source_hash(), "bytes_per_launch": total, "parts": parts,
                  "copy_calibration": {"mib": calib_mib, "fetch_scale": f_scale, "write_scale": w_scale}}
    with open(out_json, "w") as fh:
        json.dump(tj, fh, indent=1)
    print(json.dumps(tj[config], indent=1))


def stats_report(path):
    import csv

    rows = list(csv.DictReader(open(path)))
    print("| kernel | calls | average us | min us | max us | share % |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        name = r["Name"].replace("moe::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")


def main():
    args = parse()
    if args.stats_report:
        stats_report(args.stats_report)
        return
    if args.pmc_report:
        pmc_report(args.pmc_report[0], args.pmc_report[1], args.traffic_json, args.config,
                   args.copy_calibration_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparsely_gated_mixture_gate_amd as moe
    from sparsely_gated_mixture_gate_amd.buffers import ForwardBuffers, StepBuffers, to_device, to_numpy
    from synthetic import get_config, make_inputs

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg)
    d = {k: to_device(v, dev) for k, v in inp.items()}
    p = moe.make_params(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k, cfg.dtype, cfg.act, cfg.renormalize,
                        cfg.capacity_factor)
    fb = ForwardBuffers.alloc(p, dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def forward():
        moe.moe_forward(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], d["w1"], d["w2"], fb.y,
                        fb.aux, fb.topk_idx, fb.topk_gate, fb.counts_routed, fb.counts_kept, fb.slot_dest, fb.ws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    tokens_per_s = cfg.T * args.steps / (ms_total / 1e3)
    print(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step (wall {t_wall:.3f} s)", file=sys.stderr, flush=True)

    # ---- per-step breakdown and the dominant step (expert FFN), events on the same stream
    sb = StepBuffers.alloc(p, dev)
    moe.moe_route(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], sb.topk_idx, sb.topk_gate,
                  sb.counts_routed, sb.aux, None, sb.ws_route)
    moe.moe_dispatch(p, d["x"], sb.topk_idx, sb.counts_kept, sb.offsets, sb.slot_dest, sb.row_src, sb.x_perm,
                     sb.ws_dispatch)
    torch.cuda.synchronize()
    steps = {
        "route": lambda: moe.moe_route(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"],
                                       sb.topk_idx, sb.topk_gate, sb.counts_routed, sb.aux, None, sb.ws_route),
        "dispatch": lambda: moe.moe_dispatch(p, d["x"], sb.topk_idx, sb.counts_kept, sb.offsets, sb.slot_dest,
                                             sb.row_src, sb.x_perm, sb.ws_dispatch),
        "expert_ffn": lambda: moe.moe_expert_ffn(p, sb.x_perm, sb.offsets, d["w1"], d["w2"], sb.y_perm, sb.ws_ffn),
        "combine": lambda: moe.moe_combine(p, sb.y_perm, sb.slot_dest, sb.topk_gate, sb.y),
    }
    breakdown = {}
    for name, fn in steps.items():
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        breakdown[name] = a.elapsed_time(b) / args.steps
    print(f"[bench] breakdown ms: {breakdown}", file=sys.stderr, flush=True)

    elt = 2 if cfg.dtype == "bf16" else 4
    counts_kept = to_numpy(sb.counts_kept)
    R, ffn_bytes, ffn_flops = ffn_algorithmic(cfg, counts_kept, elt)
    t_ffn = breakdown["expert_ffn"] / 1e3
    mfma_tflops = ffn_flops / t_ffn / 1e12
    hbm_gbs = ffn_bytes / t_ffn / 1e9
    if cfg.dtype != "bf16":
        bound, achieved, peak, unit = "alu", mfma_tflops, FP32_VALU_PEAK_TFLOPS, "TFLOP/s"
    elif ffn_flops / ffn_bytes > (BF16_MFMA_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9):
        bound, achieved, peak, unit = "mfma", mfma_tflops, BF16_MFMA_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", hbm_gbs, HBM_PEAK_GBS, "GB/s"
    traffic = None
    try:
        with open(args.traffic_json) as fh:
            tj = json.load(fh)
        entry = tj.get(cfg.name)
        if entry and entry.get("source_hash") == source_hash():
            traffic = entry["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    roofline = {
        "kernel": "moe_expert_ffn (tile map + grouped GEMM1 with activation + grouped GEMM2)",
        "bound": bound,
        "achieved": round(achieved, 3),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": traffic,
        "algorithmic_bytes": ffn_bytes,
        "algorithmic_flops": ffn_flops,
        "launch_ms": round(breakdown["expert_ffn"], 5),
    }

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, inp, args.cpu_budget_s)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens and N(0,1/fan_in) weights, random init)",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "T": cfg.T, "d_model": cfg.d_model, "d_ff": cfg.d_ff, "E": cfg.E, "k": cfg.k,
            "capacity_factor": cfg.capacity_factor, "kept_rows": R, "parallelism": "none (1 GPU)",
        },
        "mfma_frac_expert_gemm": round(mfma_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        "breakdown_ms": {k: round(v, 5) for k, v in breakdown.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
