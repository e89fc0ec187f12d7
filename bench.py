#!/usr/bin/env python3
"""Benchmark: sparsely-gated MoE layer forward on one MI355X.

One step = one whole layer forward (moe_forward: route -> dispatch -> expert
FFN -> combine, plus the balancing losses) over one batch of seeded synthetic
tokens already resident in HBM. Default workload: the large-expert dropless
top-1 layer (T=65536, d_model=2048, d_ff=8192, E=64, Zipf(1.2) segment sizes,
GELU, bf16) -- the largest layer of the five, the one the headline is quoted on.

Timing protocol: W untimed warm-up forwards; then K timed forwards, each
preceded by a write of a 512 MiB buffer (evicts the L2s and the Infinity Cache,
so every step starts cold) and bracketed by HIP events on the stream the layer
runs on; ms_per_step is the mean of the K cold steps, with median / p10 / p90
beside it, and the back-to-back warm mean of K more forwards. A third pass of K
cold forwards records the forward's own phase events (moe_set_phase_events:
route, dispatch, expert layer 1, expert layer 2, combine) to give each step's
time, its algorithmic bytes or flops, and its fraction of the MI355X peak (HBM
8 TB/s; dense bf16 MFMA 2.5 PFLOP/s). The step entry points moe_route,
moe_dispatch (with the row permutation the bf16 forward leaves to the expert
GEMM) and moe_combine are timed the same way on their own.

Prints ONE JSON line (per workload with --config all).
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
DEFAULT_CONFIG = "dropless_top1"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=DEFAULT_CONFIG, help="workload name, or 'all' for one line per workload")
    ap.add_argument("--flush-mib", type=int, default=512, help="buffer written before every cold step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-steps", action="store_true", help="skip the standalone step entry points")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0, help="target CPU seconds for the oracle sample")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM traffic per launch of the dominant kernel, from rocprofv3 counters")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain copy kernel of this size first (counter calibration)")
    ap.add_argument("--pmc-report", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into --traffic-json")
    ap.add_argument("--stats-report", metavar="KERNEL_STATS_CSV",
                    help="print a rocprofv3 --stats kernel_stats.csv as a markdown table")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor GEMM library (torch.matmul / torch.bmm, bf16) on dense and uniformly "
                         "batched GEMMs with the workload's expert-layer shapes, as a point of comparison")
    return ap.parse_args()


# --------------------------------------------------------------------------
# algorithmic work of each step (bytes that must cross HBM at least once, flops)
# --------------------------------------------------------------------------
def algorithmic(cfg, counts_routed, counts_kept):
    import numpy as np

    e = 2 if cfg.dtype == "bf16" else 4
    T, d, f, E, k = cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k
    R = int(np.sum(counts_kept))
    live = int(np.count_nonzero(counts_kept))
    dropped_tokens = 0  # rows of y the dispatch zeroes (top-1 only) -- counted below from counts
    if k == 1:
        dropped_tokens = int(np.sum(counts_routed) - R)
    wg = d * E * e * (2 if cfg.noisy else 1)
    out = {
        # gate: x once, the gate (and noise) weights, the noise tensor, the ids and gates written
        "route": {"bytes": T * d * e + wg + (4 * T * E if cfg.noisy else 0) + 8 * T * k},
        # index work: ids read; slot_dest, row_src, counts, offsets written; dropped rows of y zeroed
        "dispatch": {"bytes": 4 * T * k + 4 * T * k + 4 * R + 12 * E + dropped_tokens * d * e},
        "gemm1": {"flops": 2.0 * R * d * f, "bytes": live * d * f * e + R * d * e + R * f * e},
        "gemm2": {"flops": 2.0 * R * f * d, "bytes": live * f * d * e + R * f * e + R * d * e},
        "combine": {"bytes": R * d * e + 8 * T * k + T * d * e},
        # standalone moe_dispatch: the index work plus the permuted copy of the kept rows
        "dispatch_permute": {"bytes": 4 * T * k + 4 * T * k + 4 * R + 12 * E + 2 * R * d * e},
    }
    return R, live, out


def rate(ms, work):
    """GB/s and TFLOP/s of a step with its fraction of the matching peak."""
    s = ms / 1e3
    r = {"ms": round(ms, 5)}
    if "bytes" in work:
        gbs = work["bytes"] / s / 1e9 if s > 0 else None
        r.update(bytes=work["bytes"], GB_s=round(gbs, 1) if gbs else None,
                 frac_hbm=round(gbs / HBM_PEAK_GBS, 4) if gbs else None)
    if "flops" in work:
        tf = work["flops"] / s / 1e12 if s > 0 else None
        r.update(flops=work["flops"], TFLOP_s=round(tf, 2) if tf else None,
                 frac_mfma=round(tf / BF16_MFMA_PEAK_TFLOPS, 4) if tf else None)
    return r


def pct(vals, q):
    import numpy as np

    return float(np.percentile(np.asarray(vals, dtype=np.float64), q))


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# --------------------------------------------------------------------------
def cpu_baseline(cfg, inp, budget_s):
    """Routing and dispatch of the whole batch, then the expert FFN and combine
    of the first n tokens; the whole-batch time is extrapolated linearly in n."""
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


# --------------------------------------------------------------------------
# rocprofv3 summaries
# --------------------------------------------------------------------------
GEMM_SOURCES = ("expert_gemm.hip", "lds_dma.h", "common.h")


def source_hash() -> str:
    """Hash of the expert GEMM's sources: counter data taken on another version of
    the kernel is stale."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparsely_gated_mixture_gate_amd", "csrc")
    for f in GEMM_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _is_layer1(kernel_name: str) -> bool:
    # grouped_gemm_bf16_kernel<BM, BN, BK, NSTAGE, ACT, APPLY_ACT, ...> / grouped_gemm_f32_kernel<ACT, APPLY_ACT>
    targs = [t.strip() for t in kernel_name[kernel_name.index("<") + 1:kernel_name.index(">")].split(",")]
    return targs[5] == "true" if "bf16" in kernel_name else targs[1] == "true"


def pmc_report(fetch_dir, write_dir, out_json, config, calib_mib):
    """Per-launch HBM bytes of the two expert GEMM kernels from two rocprofv3
    --pmc runs (FETCH_SIZE, WRITE_SIZE), each scaled by what the counter reads
    for a plain copy kernel of calib_mib MiB (which reads and writes that much)."""
    import csv
    import glob

    def per_kernel(dd, counter):
        rows = []
        for fn in glob.glob(os.path.join(dd, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(fn)))
        out = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")

    def mean(dd, pred):
        vals = [v for kk, vs in dd.items() if pred(kk) for v in vs]
        return sum(vals) / len(vals) if vals else None

    is_copy = lambda kk: "elementwise_kernel" in kk and "MulFunctor" in kk  # noqa: E731
    kib = calib_mib * 1024.0
    f_scale = kib / mean(fetch, is_copy)
    w_scale = kib / mean(write, is_copy)
    parts = {}
    for tag, pred in (("gemm1", lambda kk: "grouped_gemm" in kk and _is_layer1(kk)),
                      ("gemm2", lambda kk: "grouped_gemm" in kk and not _is_layer1(kk))):
        f_kib, w_kib = mean(fetch, pred), mean(write, pred)
        if f_kib is None or w_kib is None:
            continue
        parts[tag] = {"fetch_bytes": f_kib * 1024 * f_scale, "write_bytes": w_kib * 1024 * w_scale,
                      "fetch_kib_raw": f_kib, "write_kib_raw": w_kib}
    try:
        with open(out_json) as fh:
            tj = json.load(fh)
    except (OSError, ValueError):
        tj = {}
    tj[config] = {"source_hash": source_hash(), "parts": parts,
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


def gpu_clock():
    """Shader clock levels from sysfs (the current one marked '*'), read right after
    the timed loops; a file read, no child process. None where sysfs does not show them."""
    import glob

    out = {}
    for fn in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            levels = open(fn).read().split("\n")
        except OSError:
            continue
        cur = [ln.strip() for ln in levels if ln.strip().endswith("*")]
        out[fn.split("/")[4]] = {"current": cur[0] if cur else None,
                                 "levels": [ln.strip() for ln in levels if ln.strip()]}
    return out or None


# --------------------------------------------------------------------------
# one workload
# --------------------------------------------------------------------------
def run_config(args, name):
    import numpy as np
    import torch

    import sparsely_gated_mixture_gate_amd as moe
    from sparsely_gated_mixture_gate_amd.buffers import ForwardBuffers, StepBuffers, to_device, to_numpy
    from synthetic import get_config, make_inputs

    cfg = get_config(name)
    dev = torch.device("cuda:0")
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg)
    d = {k: to_device(v, dev) for k, v in inp.items()}
    p = moe.make_params(cfg.T, cfg.d_model, cfg.d_ff, cfg.E, cfg.k, cfg.dtype, cfg.act, cfg.renormalize,
                        cfg.capacity_factor)
    fb = ForwardBuffers.alloc(p, dev)
    stream = torch.cuda.current_stream()
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def forward():
        moe.moe_forward(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], d["w1"], d["w2"], fb.y,
                        fb.aux, fb.topk_idx, fb.topk_gate, fb.counts_routed, fb.counts_kept, fb.slot_dest, fb.ws)

    def cold_loop(fn, n, extra=None):
        """n runs of fn, each after a cache-evicting write, bracketed by events; ms each."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            flush.fill_(i & 0x7F)
            if extra:
                extra(i)
            evs[i][0].record(stream)
            fn()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()

    # ---- headline: K cold forwards
    t_wall = time.perf_counter()
    step_ms = cold_loop(forward, args.steps)
    t_wall = time.perf_counter() - t_wall
    ms_step = sum(step_ms) / len(step_ms)
    tokens_per_s = cfg.T / (ms_step / 1e3)
    print(f"[bench] {args.steps} cold steps: mean {ms_step:.4f} ms, median {pct(step_ms, 50):.4f} ms "
          f"(wall {t_wall:.3f} s incl. flushes)", file=sys.stderr, flush=True)

    # ---- warm: K back-to-back forwards
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        forward()
    b.record(stream)
    torch.cuda.synchronize()
    warm_ms = a.elapsed_time(b) / args.steps
    clock = gpu_clock()

    # ---- phases of the forward (its own kernels), K cold forwards with phase events
    ph = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    cold_loop(forward, args.steps, extra=lambda i: moe.moe_set_phase_events(ph[i]))
    moe.moe_set_phase_events(None)
    names = ["route", "dispatch", "gemm1", "gemm2", "combine"]
    phase_ms = {nm: [ph[i][j].elapsed_time(ph[i][j + 1]) for i in range(args.steps)] for j, nm in enumerate(names)}
    ck, cr = to_numpy(fb.counts_kept), to_numpy(fb.counts_routed)
    R, live, work = algorithmic(cfg, cr, ck)
    phases = {nm: rate(pct(v, 50), work[nm]) for nm, v in phase_ms.items()}
    if cfg.dtype == "bf16" and cfg.k == 1:
        phases["combine"] = {"ms": round(pct(phase_ms["combine"], 50), 5),
                             "note": "top-1: layer 2 writes the gated rows into y; no combine kernel"}
    if cfg.dtype == "bf16":
        phases["dispatch"]["note"] = "index work only: layer 1 gathers its rows from x (no permuted copy)"
    print(f"[bench] phases (median ms): { {k: v['ms'] for k, v in phases.items()} }", file=sys.stderr, flush=True)

    # ---- the step entry points on their own (route, dispatch with the permuted copy, combine)
    standalone = None
    if not args.no_steps:
        sb = StepBuffers.alloc(p, dev)
        moe.moe_route(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"], sb.topk_idx, sb.topk_gate,
                      sb.counts_routed, sb.aux, None, sb.ws_route)
        moe.moe_dispatch(p, d["x"], sb.topk_idx, sb.counts_kept, sb.offsets, sb.slot_dest, sb.row_src, sb.x_perm,
                         sb.ws_dispatch)
        torch.cuda.synchronize()
        fns = {
            "route": (lambda: moe.moe_route(p, d["x"], d["w_gate"], d["gate_bias"], d["w_noise"], d["noise"],
                                            sb.topk_idx, sb.topk_gate, sb.counts_routed, sb.aux, None, sb.ws_route),
                      work["route"]),
            "dispatch_permute": (lambda: moe.moe_dispatch(p, d["x"], sb.topk_idx, sb.counts_kept, sb.offsets,
                                                          sb.slot_dest, sb.row_src, sb.x_perm, sb.ws_dispatch),
                                 work["dispatch_permute"]),
            "combine": (lambda: moe.moe_combine(p, sb.y_perm, sb.slot_dest, sb.topk_gate, sb.y), work["combine"]),
        }
        standalone = {}
        for nm, (fn, wk) in fns.items():
            for _ in range(2):
                fn()
            standalone[nm] = rate(pct(cold_loop(fn, args.steps), 50), wk)
        print(f"[bench] standalone (median ms): { {k: v['ms'] for k, v in standalone.items()} }", file=sys.stderr,
              flush=True)
        del sb

    # ---- roofline of the dominant kernel: expert layer 1 inside the forward
    g1, g2 = phases["gemm1"], phases["gemm2"]
    if cfg.dtype == "bf16":
        t_gemm = (g1["ms"] + g2["ms"]) / 1e3
        mfma_frac = (work["gemm1"]["flops"] + work["gemm2"]["flops"]) / t_gemm / 1e12 / BF16_MFMA_PEAK_TFLOPS
        intensity = work["gemm1"]["flops"] / work["gemm1"]["bytes"]
        if intensity > (BF16_MFMA_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9):
            bound, achieved, peak, unit, frac = "mfma", g1["TFLOP_s"], BF16_MFMA_PEAK_TFLOPS, "TFLOP/s", g1["frac_mfma"]
        else:
            bound, achieved, peak, unit, frac = "hbm", g1["GB_s"], HBM_PEAK_GBS, "GB/s", g1["frac_hbm"]
    else:
        mfma_frac = None
        tf = work["gemm1"]["flops"] / (g1["ms"] / 1e3) / 1e12
        bound, achieved, peak, unit, frac = "alu", round(tf, 3), FP32_VALU_PEAK_TFLOPS, "TFLOP/s", \
            round(tf / FP32_VALU_PEAK_TFLOPS, 4)
    traffic = None
    try:
        with open(args.traffic_json) as fh:
            entry = json.load(fh).get(cfg.name)
        if entry and entry.get("source_hash") == source_hash() and "gemm1" in entry.get("parts", {}):
            traffic = round(entry["parts"]["gemm1"]["fetch_bytes"] + entry["parts"]["gemm1"]["write_bytes"])
    except (OSError, ValueError):
        pass
    roofline = {
        "kernel": "expert layer 1 (grouped_gemm_bf16_kernel, APPLY_ACT) inside moe_forward",
        "bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": frac, "traffic": traffic,
        "algorithmic_bytes": work["gemm1"]["bytes"], "algorithmic_flops": work["gemm1"]["flops"],
        "launch_ms": g1["ms"],
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
            "capacity_factor": cfg.capacity_factor, "kept_rows": R, "experts_with_rows": live,
            "parallelism": "none (1 GPU)",
        },
        "step_ms": {"mean_cold": round(ms_step, 5), "median_cold": round(pct(step_ms, 50), 5),
                    "p10_cold": round(pct(step_ms, 10), 5), "p90_cold": round(pct(step_ms, 90), 5),
                    "mean_warm": round(warm_ms, 5), "flush_mib_before_each_cold_step": args.flush_mib},
        "mfma_frac_expert_gemm": round(mfma_frac, 4) if mfma_frac is not None else None,
        "phases": phases,
        "standalone_steps": standalone,
        "roofline": roofline,
        "gpu_clock": clock,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    del d, fb, flush
    torch.cuda.empty_cache()


def library_gemm(name, iters):
    """Dense and uniformly batched bf16 GEMMs of the workload's expert layers through the vendor library
    (torch.matmul / torch.bmm): M = T * k rows, layer 1 [M, d] x [d, f], layer 2 [M, f] x [f, d]; batched:
    E segments of M / E rows, each against its own weight matrix. A reference point for the grouped GEMM,
    which does the same work on ragged segments with the row gather, activation and gate fused."""
    import torch
    from synthetic.configs import CONFIGS

    cfg = CONFIGS[name]
    if cfg.dtype != "bf16":
        sys.exit(f"--library-gemm: {name} is not a bf16 workload")
    dev = torch.device("cuda:0")
    M, E, d, f = cfg.T * cfg.k, cfg.E, cfg.d_model, cfg.d_ff
    shapes = [(f"dense layer 1: [{M}, {d}] x [{d}, {f}]", (M, d), (d, f)),
              (f"dense layer 2: [{M}, {f}] x [{f}, {d}]", (M, f), (f, d)),
              (f"batched layer 1: {E} x [{M // E}, {d}] x [{d}, {f}]", (E, M // E, d), (E, d, f)),
              (f"batched layer 2: {E} x [{M // E}, {f}] x [{f}, {d}]", (E, M // E, f), (E, f, d))]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    print(f"library GEMMs, {name} shapes, bf16 in / bf16 out, {iters} back-to-back calls each")
    print("| GEMM | ms | TFLOP/s | fraction of 2.5 PFLOP/s |")
    print("|---|---:|---:|---:|")
    for label, sa, sb in shapes:
        a = torch.randn(sa, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        b = (torch.randn(sb, generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16).contiguous()
        fn = (lambda: torch.bmm(a, b)) if a.dim() == 3 else (lambda: torch.matmul(a, b))
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        flops = 2.0 * M * d * f
        print(f"| {label} | {ms:.3f} | {flops / ms / 1e9:.0f} | {flops / ms / 1e9 / 2500:.3f} |", flush=True)
        del a, b
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.library_gemm:
        library_gemm(DEFAULT_CONFIG if args.config == "all" else args.config, args.steps)
        return
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
    from synthetic.configs import CONFIG_ORDER

    for name in (CONFIG_ORDER if args.config == "all" else [args.config]):
        run_config(args, name)


if __name__ == "__main__":
    main()
