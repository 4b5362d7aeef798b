#!/usr/bin/env python3
"""Benchmark of the routed MoE layer forward (ftmoe_forward) on one MI355X.

One step = one ftmoe_forward call (router GEMM + softmax top-k, align,
gate_up GEMM + SwiGLU, down GEMM, weighted combine) over one batch of
synthetic tokens, with the inputs already resident in HBM.

Default workload: the decode configuration of the 30B-A3B-class layer
(T = 8 tokens, hidden 2048, 128 experts, top-8, intermediate 768, MXFP4
experts).  Its metric is the selected-expert weight bytes streamed per second
(each distinct selected expert's packed bytes counted once per step).  To
keep the 256 MB Infinity Cache from serving those bytes, consecutive steps
cycle through several device copies of the layer (a model's consecutive MoE
layers) and through different token batches.

The default run also measures the three prefill configurations (the
30B-A3B-class layer at T = 4096, the 512-expert NVFP4 layer with a shared
expert at T = 8192, the FP8 W8A8 layer with Zipf-skewed routing at
T = 16384) and reports them in a "prefill" object of the same JSON line:
tokens/s, step time, and the gate_up GEMM's MFMA roofline from the kernel's
own event-timed launches in the same run.

Prints one JSON line (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}
METRIC = "MoE-layer tokens/s (prefill) + decode expert-weight GB/s, % of MI355X roofline"
# Arithmetic of the expert GEMMs by weight format: MXFP4 codes meet the
# activations as a pair of E4M3 codes per element (as exact as bf16) on the
# E8M0-scaled MFMA (two MFMAs per product, so its roofline is the bf16 one);
# NVFP4 dequantises exactly to bf16; FP8 W8A8 runs E4M3 x E4M3.
# MXFP8 activations (W4A8) meet MXFP4 codes on one scaled MFMA per product,
# at the 8-bit operand rate (FP8 roofline).
DTYPE = {"mxfp4": "e2m1 x e4m3-pair mfma/fp32-acc", "nvfp4": "bf16-mfma/fp32-acc",
         "fp8": "bf16-mfma/fp32-acc", "fp8act": "fp8-e4m3-mfma/fp32-acc",
         "mxfp8act": "e2m1 x mxfp8-e4m3 mfma/fp32-acc", "bf16": "bf16-mfma/fp32-acc"}

WORKLOADS = {
    # name: (config, T, kind)
    "c1": ("c1", 8, "decode"),
    "c1-t1": ("c1", 1, "decode"),
    "c3-t1": ("c3", 1, "decode"),
    "c2": ("c2", 4096, "prefill"),
    "c3": ("c3", 8192, "prefill"),
    "c4": ("c4", 16384, "prefill"),
    "c1-w4a8": ("c1-w4a8", 8, "decode"),
    "c2-w4a8": ("c2-w4a8", 4096, "prefill"),
    "c2-bf16": ("c2-bf16", 4096, "prefill"),
}
# the prefill configurations the default line carries
PREFILL_LINE = ("c2", "c3", "c4")
# CPU baseline of a prefill configuration: the grouped oracle over a bounded
# batch (the first tokens of the workload's batch, as a batch of their own)
CPU_PREFILL_TOKENS = {"c2": 4096, "c3": 2048, "c4": 512, "c2-w4a8": 4096, "c2-bf16": 4096}
# tokens of the per-token loop on one core (each new expert it meets is
# dequantised in float64, which dominates on the larger layers)
CPU_PER_TOKEN_SAMPLE = {"c1": 8, "c2": 4, "c3": 4, "c4": 2}


def describe(cfg, T):
    s = (f"{cfg.name}: T={T}, hidden {cfg.hidden}, {cfg.num_experts} experts, top-{cfg.top_k}, "
         f"intermediate {cfg.inter}, {cfg.fmt.upper()} experts")
    if cfg.shared_inter:
        s += f", shared expert (intermediate {cfg.shared_inter})"
    if cfg.act == "fp8":
        s += ", per-tensor E4M3 activations"
    if cfg.act == "mxfp8":
        s += ", MXFP8 activations (W4A8)"
    if cfg.zipf_s:
        s += f", Zipf({cfg.zipf_s}) router bias"
    return s


def per_expert_bytes(q):
    b = q.codes[0].nbytes
    if q.block_scales is not None:
        b += q.block_scales[0].nbytes
    if q.tensor_scales is not None:
        b += q.tensor_scales[0].nbytes
    return b


def event_steps(torch, stream, n, step):
    """Durations (ms) of n steps, from stream events around each (no host
    synchronisation between steps)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def pct(a):
    return {q: round(float(np.percentile(a, v)), 5) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}


def measure(ft, torch, synth, workload, steps, warmup, path="auto", ring=None, batches=16, pool_slots=0,
            host_threads=0):
    """Times `steps` forwards of a workload; returns its results and the
    host-side inputs (for the CPU baseline)."""
    name, T, kind = WORKLOADS[workload]
    cfg = synth.CONFIGS[name]
    lay = synth.make_layer(name)
    ring = ring or (4 if kind == "decode" and not pool_slots else 1)
    dev = "cuda"
    dlays = [ft.DeviceLayer.from_host(lay, dev, path=path) for _ in range(ring)]
    pool = ft.ExpertCache.from_host(lay, pool_slots, dev, path=path) if pool_slots else None
    if pool is not None and host_threads:
        pool.set_host_compute(host_threads)
    if (kind == "prefill" or path == "prefill") and pool is None:
        # load-time step: the prefill GEMMs read their weight stages from the
        # packed tile layout (outside the timed region, like loading a model)
        for d in dlays:
            d.pack()
        torch.cuda.synchronize()
    descs = [d.desc() for d in dlays]
    nb = batches if kind == "decode" else 2
    xs_host = [synth.make_tokens(lay, T, stream=100 + b) for b in range(nb)]
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs_host]
    ws = ft.alloc_workspace(dlays[0], T)
    y = torch.empty((T, cfg.hidden), dtype=torch.int16, device=dev)
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    # Routing of every batch: the byte count of its selected experts, and
    # (decode) its routing kept for the experts-only timing.
    sel_bytes, routes = [], []
    for b in range(nb):
        ft.forward(dlays[0], xs[b], T, ws, y, ids, w, desc=descs[0])
        torch.cuda.synchronize()
        sel_bytes.append(dlays[0].selected_expert_bytes(ids.cpu().numpy()))
        if kind == "decode" and pool is None:
            sg = torch.empty((T,), dtype=torch.float32, device=dev) if cfg.shared_inter else None
            rw = torch.empty_like(w)
            ri = torch.empty_like(ids)
            ft.route(dlays[0], xs[b], T, ws, ri, rw, sg)
            routes.append((ri, rw, sg))
    torch.cuda.synchronize()

    def step(i):
        ft.forward(dlays[i % ring], xs[i % nb], T, ws, y, ids, w, stream=stream, desc=descs[i % ring])

    if pool is not None:
        del dlays, descs
        pws = pool.workspace(T)

        def step(i):  # noqa: F811
            pool.forward(xs[i % nb], T, pws, y, ids, w, stream=stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    pool_before = pool.stats() if pool is not None else None
    host_before = pool.host_stats() if pool is not None else None
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    res = {"name": name, "T": T, "kind": kind, "cfg": cfg, "lay": lay, "xs_host": xs_host, "ms": ms, "ring": ring,
           "nb": nb, "sel_bytes": sel_bytes}
    if pool is not None:
        st = pool.stats()
        d = {key: st[key] - pool_before[key] for key in st}
        res["pool"] = {"slots": pool_slots, "hit_rate": round(d["hits"] / max(1, d["hits"] + d["misses"]), 4),
                       "copied_bytes_per_step": d["bytes_copied"] // steps,
                       "passes_per_step": round(d["passes"] / steps, 3),
                       "copy_GBs": round(d["bytes_copied"] / (t1 - t0) / 1e9, 2),
                       "h2d_copy_GBs_measured": h2d_rate(torch, dev)}
        if host_threads:
            hs = pool.host_stats()
            res["pool"]["host_compute"] = {
                "threads": host_threads, "experts_per_step": round((hs["experts"] - host_before["experts"]) / steps, 3),
                "rows_per_step": round((hs["rows"] - host_before["rows"]) / steps, 3),
                "host_ms_per_step": round((hs["seconds"] - host_before["seconds"]) * 1e3 / steps, 4),
                "cost_model": {"expert_s": hs["expert_s"], "row_s": hs["row_s"]}}
    res["mean_bytes"] = float(np.mean([sel_bytes[i % nb] for i in range(steps)]))
    res["step_pct"] = pct(event_steps(torch, stream, steps, step))

    # Same steps again with per-kernel timing: events attached to each kernel's
    # launch (recorded at its start and end), or bracketing a multi-kernel step.
    ft.timing_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    kern = ft.timing_collect()
    ft.timing_enable(False)
    res["kernel_us"] = {k: 1e3 * v[0] / v[1] for k, v in kern.items()}

    if routes:
        # ftmoe_experts_forward alone (align, gate_up, down, combine) on each
        # batch's own routing: the expert-stream rate
        def xstep(i):
            ri, rw, sg = routes[i % nb]
            ft.experts_forward(dlays[i % ring], xs[i % nb], T, ri, rw, sg, ws, y, stream=stream)

        for i in range(warmup):
            xstep(i)
        res["experts_forward_ms"] = float(np.median(event_steps(torch, stream, steps, xstep)))
    return res


def decode_roofline(res):
    lay, cfg, ku = res["lay"], res["cfg"], res["kernel_us"]
    dom = max((n for n in ku if n.startswith("decode_")), key=lambda n: ku[n])
    # Algorithmic bytes of the dominant kernel: its matrix's packed bytes of
    # every distinct selected expert (and of the shared expert).
    gu_b, dn_b = per_expert_bytes(lay.gate_up), per_expert_bytes(lay.down)
    sgu_b = per_expert_bytes(lay.shared_gate_up) if cfg.shared_inter else 0
    sdn_b = per_expert_bytes(lay.shared_down) if cfg.shared_inter else 0
    mean_unique = (res["mean_bytes"] - sgu_b - sdn_b) / (gu_b + dn_b)
    unit_bytes = {"decode_gateup": gu_b * mean_unique + sgu_b, "decode_down": dn_b * mean_unique + sdn_b}[dom]
    if "pool" in res:
        # through the pool a step runs its experts in several passes, each a
        # launch over a part of them: the bytes of the average launch
        unit_bytes /= max(1.0, res["pool"]["passes_per_step"])
    achieved = unit_bytes / (ku[dom] * 1e-6) / 1e9
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": int(unit_bytes), "avg_launch_us": round(ku[dom], 3)}
    expert_us = ku.get("decode_gateup", 0.0) + ku.get("decode_down", 0.0)
    if "pool" not in res:
        # the gate_up and down kernels alone; and ftmoe_experts_forward
        roof["expert_kernels_GBs"] = round(res["mean_bytes"] / (expert_us * 1e-6) / 1e9, 1)
        if "experts_forward_ms" in res:
            roof["experts_forward_us"] = round(res["experts_forward_ms"] * 1e3, 3)
            roof["experts_forward_GBs"] = round(res["mean_bytes"] / (res["experts_forward_ms"] * 1e-3) / 1e9, 1)
    return roof


def gateup_min_bytes(res):
    """Bytes the routed gate_up GEMM must move at least: the gate_up matrices
    of the experts that received rows, each token's activation row once, and
    each (token, expert) row of h once, in the formats the kernel reads and
    writes them (split E4M3 pairs + E8M0 scales for MXFP4, E4M3 (+ E8M0) for
    FP8 and MXFP8 activations, bf16 otherwise; h of FP8 layers is written in
    bf16 and quantised after the global maximum is known)."""
    lay, cfg, T = res["lay"], res["cfg"], res["T"]
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    gu_b, dn_b = per_expert_bytes(lay.gate_up), per_expert_bytes(lay.down)
    sh_b = (per_expert_bytes(lay.shared_gate_up) + per_expert_bytes(lay.shared_down)) if cfg.shared_inter else 0
    n_experts = (res["mean_bytes"] - sh_b) / (gu_b + dn_b)
    if cfg.fmt == "mxfp4" and cfg.act == "mxfp8":
        x_row, h_row = H + H // 32, I + I // 32
    elif cfg.fmt == "mxfp4":
        x_row, h_row = 2 * H + H // 32, 2 * I + I // 32
    elif cfg.act == "fp8":
        x_row, h_row = H, 2 * I
    else:
        x_row, h_row = 2 * H, 2 * I
    return gu_b * n_experts + T * x_row + T * k * h_row


def prefill_roofline(res):
    cfg, T, ku = res["cfg"], res["T"], res["kernel_us"]
    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    flops = 2.0 * T * k * H * 2 * I
    dom = "gemm_gateup"
    achieved = flops / (ku[dom] * 1e-6) / 1e12
    peak = MFMA_PEAK_TFLOPS["fp8" if cfg.act in ("fp8", "mxfp8") else "bf16"]
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": None, "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": int(gateup_min_bytes(res)), "avg_launch_us": round(ku[dom], 3)}
    if "gemm_down" in ku:
        # both routed GEMMs together (gate_up 2/3, down 1/3 of the flops)
        g = 3.0 * flops / 2.0 / ((ku[dom] + ku["gemm_down"]) * 1e-6) / 1e12
        roof["grouped_gemms_TFLOPs"] = round(g, 1)
        roof["grouped_gemms_frac"] = round(g / peak, 4)
    return roof


def progress(msg):
    """One line on stderr per phase, so a long run is never silent."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c1", choices=sorted(WORKLOADS))
    ap.add_argument("--ring", type=int, default=None, help="device copies of the layer cycled over steps")
    ap.add_argument("--batches", type=int, default=16, help="distinct token batches cycled over steps")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave out the prefill configurations the default decode line carries")
    ap.add_argument("--prefill-steps", type=int, default=100)
    ap.add_argument("--prefill-warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="decode: oracle steps run until this much time")
    ap.add_argument("--pool-slots", type=int, default=0,
                    help="serve the routed experts from pinned host memory through an HBM pool of this many "
                         "expert slots (ftmoe_cache_*); the rate then includes the host-to-device copies")
    ap.add_argument("--host-threads", type=int, default=0,
                    help="with --pool-slots: CPU-GPU co-execution, missing experts split between this many host "
                         "threads and the pool by the calibrated cost model (ftmoe_cache_set_host_compute)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a known-size kernel for "
                         "scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; the layer forward is not sharded across "
                                   "GPUs here, so --gpus above 1 is not supported"}), flush=True)
        return 2

    import torch
    import block_scaled_fp4_router_amd as ft
    import synth

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    progress(f"measuring {args.workload}")
    res = measure(ft, torch, synth, args.workload, args.steps, args.warmup, args.path, args.ring, args.batches,
                  args.pool_slots, args.host_threads)
    cfg, T, kind = res["cfg"], res["T"], res["kind"]
    if kind == "decode":
        value, unit = res["mean_bytes"] / (res["ms"] * 1e-3) / 1e9, "GB/s"
        roof = decode_roofline(res)
    else:
        value, unit = T / (res["ms"] * 1e-3), "tokens/s"
        roof = prefill_roofline(res)
    traffic = measured_traffic(roof["kernel"], args.workload)
    if traffic is not None:
        roof["traffic"] = traffic["bytes"]
        roof["traffic_counters"] = traffic["counters"]
        roof["traffic_dram"] = traffic["dram"]
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(res["ms"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE[cfg.fmt if cfg.act == "bf16" else cfg.act + "act"],
        "data": "synthetic (seeded generator; random-init weights quantised to the named format)",
        "config": {"workload": describe(cfg, T), "kind": kind, "tokens": T, "layer_copies_cycled": res["ring"],
                   "token_batches_cycled": res["nb"], "path": args.path,
                   "selected_expert_bytes_per_step": int(res["mean_bytes"])},
        **({"expert_pool": res["pool"]} if "pool" in res else {}),
        "step_ms_percentiles": res["step_pct"],
        "roofline": roof,
        "kernel_avg_us": {k2: round(v, 3) for k2, v in sorted(res["kernel_us"].items())},
    }
    if "pool" in res:
        out["config"]["workload"] += f", routed experts in pinned host memory through a {args.pool_slots}-slot HBM pool"
    cpu_jobs = []
    if not args.no_cpu_baseline and "pool" not in res:
        cpu_jobs.append((out, res))

    if kind == "decode" and args.workload == "c1" and not args.no_prefill and not args.pool_slots:
        prefill = {}
        for wl in PREFILL_LINE:
            progress(f"measuring {wl}")
            r = measure(ft, torch, synth, wl, args.prefill_steps, args.prefill_warmup)
            pr = prefill_roofline(r)
            tr = measured_traffic(pr["kernel"], wl)
            if tr is not None:
                pr["traffic"] = tr["bytes"]
                pr["traffic_counters"] = tr["counters"]
                pr["traffic_dram"] = tr["dram"]
            entry = {"workload": describe(r["cfg"], r["T"]), "value": round(r["T"] / (r["ms"] * 1e-3), 1),
                     "unit": "tokens/s", "ms_per_step": round(r["ms"], 5), "steps": args.prefill_steps,
                     "warmup": args.prefill_warmup,
                     "dtype": DTYPE[r["cfg"].fmt if r["cfg"].act == "bf16" else r["cfg"].act + "act"],
                     "step_ms_percentiles": r["step_pct"], "roofline": pr,
                     "kernel_avg_us": {k2: round(v, 3) for k2, v in sorted(r["kernel_us"].items())}}
            prefill[wl] = entry
            if not args.no_cpu_baseline:
                cpu_jobs.append((entry, r))
            del r
            torch.cuda.empty_cache()
        out["prefill"] = prefill

    for dst, r in cpu_jobs:
        progress(f"cpu baseline {r['cfg'].name} T={r['T']}")
        dst["cpu_baseline"] = cpu_baseline(r, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


def h2d_rate(torch, dev, mib=256):
    """GB/s of one plain pinned-host -> device copy of `mib` MiB (the link's rate, for context)."""
    src = torch.empty(mib << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    return round((mib << 20) / (time.perf_counter() - t0) / 1e9, 2)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(res, seconds):
    """The oracle as it stands, on this host's cores, after the GPU timing:
    its grouped mode (one fp32 BLAS matmul per expert over the rows routed to
    it, BLAS threads = the process's affinity cores) on the workload's
    batches (decode: whole steps until `seconds` have passed; prefill: a
    bounded batch), and its literal per-token loop on one core (float64) on
    a few tokens, as microseconds per token."""
    import oracle
    from threadpoolctl import threadpool_limits
    lay, xs, kind, T = res["lay"], res["xs_host"], res["kind"], res["T"]
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    out = {"kind": "oracle", "cores": cores, "cpu_model": cpu_model()}
    with threadpool_limits(cores):
        if kind == "decode":
            done, nbytes = 0, 0.0
            t0 = time.perf_counter()
            while True:
                b = done % len(xs)
                oracle.forward_grouped(lay, xs[b], dtype=np.float32)
                nbytes += res["sel_bytes"][b]
                done += 1
                dt = time.perf_counter() - t0
                if dt >= seconds or done >= 256:
                    break
            out.update(value=round(nbytes / dt / 1e9, 4), unit="GB/s", seconds=round(dt, 2),
                       sample=f"{done} whole decode steps (T={T}) over the same token batches, grouped oracle "
                              f"(fp32 BLAS, {cores} threads)")
        else:
            n = min(T, CPU_PREFILL_TOKENS.get(res["name"], 2048))
            x = xs[0][:n]
            t0 = time.perf_counter()
            oracle.forward_grouped(lay, x, dtype=np.float32)
            dt = time.perf_counter() - t0
            out.update(value=round(n / dt, 2), unit="tokens/s", seconds=round(dt, 2),
                       sample=f"the first {n} of the {T} tokens as a batch of their own, grouped oracle "
                              f"(fp32 BLAS, {cores} threads)")
    # the literal per-token loop (float64) on one core
    with threadpool_limits(1):
        m = min(CPU_PER_TOKEN_SAMPLE.get(res["name"], 4), T)
        tok = np.arange(m)
        s_h = 1.0 if lay.cfg.act == "fp8" else None   # the h scale only sets magnitudes here
        t0 = time.perf_counter()
        oracle.forward_tokens(lay, xs[0], tok, s_h=s_h)
        dt = time.perf_counter() - t0
    out["per_token_us_one_core"] = round(dt / m * 1e6, 1)
    out["per_token_sample"] = f"{m} tokens through the per-token float64 loop on 1 core (experts dequantised once each, included)"
    return out


def measured_traffic(kernel, workload):
    """Bytes per launch of `kernel` between the L2 and memory (L2-miss bytes:
    FETCH_SIZE + WRITE_SIZE) and the bytes of its requests to the memory
    controllers (TCC_EA0_RDREQ_DRAM + WRREQ_DRAM), each scaled by a known-size
    copy, from the committed counter summary; None when there is none or the
    kernel sources changed since it was taken."""
    import re
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]+)", text, re.M)
    m_c = re.search(r"^traffic_counters:\s*(.+)$", text, re.M)
    m_d = re.search(r"^dram_bytes_per_launch:\s*(\d+)", text, re.M)
    if not m_b or not m_h or m_h.group(1) != kernel_source_sha():
        return None
    return {"bytes": int(m_b.group(1)), "counters": m_c.group(1).strip() if m_c else "FETCH_SIZE + WRITE_SIZE",
            "dram": int(m_d.group(1)) if m_d else None}


def kernel_source_sha():
    """Hash of the HIP sources the expert kernels are built from."""
    import hashlib
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_scaled_fp4_router_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(root)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            h.update(open(os.path.join(root, name), "rb").read())
    return h.hexdigest()


if __name__ == "__main__":
    sys.exit(main())
