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
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
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

    name, T, kind = WORKLOADS[args.workload]
    cfg = synth.CONFIGS[name]
    lay = synth.make_layer(name)
    ring = args.ring or (4 if kind == "decode" and not args.pool_slots else 1)
    dev = "cuda"
    dlays = [ft.DeviceLayer.from_host(lay, dev, path=args.path) for _ in range(ring)]
    pool = ft.ExpertCache.from_host(lay, args.pool_slots, dev, path=args.path) if args.pool_slots else None
    if pool is not None and args.host_threads:
        pool.set_host_compute(args.host_threads)
    if (kind == "prefill" or args.path == "prefill") and pool is None:
        # load-time step: the prefill GEMMs read their weight stages from the
        # packed tile layout (outside the timed region, like loading a model)
        for d in dlays:
            d.pack()
        torch.cuda.synchronize()
    descs = [d.desc() for d in dlays]
    nb = args.batches if kind == "decode" else 2
    xs_host = [synth.make_tokens(lay, T, stream=100 + b) for b in range(nb)]
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs_host]
    ws = ft.alloc_workspace(dlays[0], T)
    y = torch.empty((T, cfg.hidden), dtype=torch.int16, device=dev)
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Routing of every batch (for the byte count of the selected experts).
    sel_bytes = []
    for b in range(nb):
        ft.forward(dlays[0], xs[b], T, ws, y, ids, w, desc=descs[0])
        torch.cuda.synchronize()
        sel_bytes.append(dlays[0].selected_expert_bytes(ids.cpu().numpy()))

    def step(i):
        ft.forward(dlays[i % ring], xs[i % nb], T, ws, y, ids, w, stream=stream, desc=descs[i % ring])

    if pool is not None:
        del dlays, descs
        pws = pool.workspace(T)

        def step(i):  # noqa: F811
            pool.forward(xs[i % nb], T, pws, y, ids, w, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    pool_before = pool.stats() if pool is not None else None
    host_before = pool.host_stats() if pool is not None else None
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    pool_stats = None
    if pool is not None:
        st = pool.stats()
        d = {key: st[key] - pool_before[key] for key in st}
        pool_stats = {"slots": args.pool_slots, "hit_rate": round(d["hits"] / max(1, d["hits"] + d["misses"]), 4),
                      "copied_bytes_per_step": d["bytes_copied"] // args.steps,
                      "passes_per_step": round(d["passes"] / args.steps, 3),
                      "copy_GBs": round(d["bytes_copied"] / (t1 - t0) / 1e9, 2),
                      "h2d_copy_GBs_measured": h2d_rate(torch, dev)}
        if args.host_threads:
            hs = pool.host_stats()
            pool_stats["host_compute"] = {
                "threads": args.host_threads, "experts_per_step": round((hs["experts"] - host_before["experts"]) /
                                                                        args.steps, 3),
                "rows_per_step": round((hs["rows"] - host_before["rows"]) / args.steps, 3),
                "host_ms_per_step": round((hs["seconds"] - host_before["seconds"]) * 1e3 / args.steps, 4),
                "cost_model": {"expert_s": hs["expert_s"], "row_s": hs["row_s"]}}
    mean_bytes = float(np.mean([sel_bytes[i % nb] for i in range(args.steps)]))

    # Per-step durations (events on the stream around each step, no host
    # synchronisation between steps): median and spread.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in evs])
    step_pct = {q: round(float(np.percentile(per_step, v)), 5) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

    # Same steps again with per-kernel timing: events attached to each kernel's
    # launch (recorded at its start and end), or bracketing a multi-kernel step.
    ft.timing_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kern = ft.timing_collect()
    ft.timing_enable(False)
    kernel_us = {k: 1e3 * v[0] / v[1] for k, v in kern.items()}

    H, I, k = cfg.hidden, cfg.inter, cfg.top_k
    if kind == "decode":
        value = mean_bytes / (ms * 1e-3) / 1e9
        unit = "GB/s"
        dom = max((n for n in kernel_us if n.startswith("decode_")), key=lambda n: kernel_us[n])
        # Algorithmic bytes of the dominant kernel: its matrix's packed bytes of
        # every distinct selected expert (shared expert for the shared kernels).
        def per_expert(q):
            b = q.codes[0].nbytes
            if q.block_scales is not None:
                b += q.block_scales[0].nbytes
            if q.tensor_scales is not None:
                b += q.tensor_scales[0].nbytes
            return b
        gu_b, dn_b = per_expert(lay.gate_up), per_expert(lay.down)
        shared_b = per_expert(lay.shared_gate_up) + per_expert(lay.shared_down) if cfg.shared_inter else 0
        mean_unique = (mean_bytes - shared_b) / (gu_b + dn_b)
        sgu_b = per_expert(lay.shared_gate_up) if cfg.shared_inter else 0
        sdn_b = per_expert(lay.shared_down) if cfg.shared_inter else 0
        unit_bytes = {"decode_gateup": gu_b * mean_unique + sgu_b,
                      "decode_down": dn_b * mean_unique + sdn_b}[dom]
        achieved = unit_bytes / (kernel_us[dom] * 1e-6) / 1e9
        expert_us = kernel_us["decode_gateup"] + kernel_us["decode_down"]
        # the expert kernels alone (one launch each per step; a pool runs several passes)
        expert_rate = round(mean_bytes / (expert_us * 1e-6) / 1e9, 1) if pool is None else None
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": int(unit_bytes), "avg_launch_us": round(kernel_us[dom], 3),
                "expert_kernels_GBs": expert_rate}
    else:
        value = T / (ms * 1e-3)
        unit = "tokens/s"
        dom = "gemm_gateup"
        flops = 2.0 * T * k * H * 2 * I
        achieved = flops / (kernel_us[dom] * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS["fp8" if cfg.act in ("fp8", "mxfp8") else "bf16"]
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "algorithmic_flops_per_launch": flops, "avg_launch_us": round(kernel_us[dom], 3)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE[cfg.fmt if cfg.act == "bf16" else cfg.act + "act"],
        "data": "synthetic (seeded generator; random-init weights quantised to the named format)",
        "config": {"workload": describe(cfg, T), "kind": kind, "tokens": T, "layer_copies_cycled": ring,
                   "token_batches_cycled": nb, "path": args.path,
                   "selected_expert_bytes_per_step": int(mean_bytes)},
        **({"expert_pool": pool_stats} if pool_stats else {}),
        "step_ms_percentiles": step_pct,
        "roofline": roof,
        "kernel_avg_us": {k2: round(v, 3) for k2, v in sorted(kernel_us.items())},
    }

    traffic = measured_traffic(roof["kernel"], args.workload)
    if traffic is not None:
        roof["traffic"] = traffic
    if pool is not None:
        out["config"]["workload"] += f", routed experts in pinned host memory through a {args.pool_slots}-slot HBM pool"
    if not args.no_cpu_baseline and pool is None:
        out["cpu_baseline"] = cpu_baseline(lay, xs_host, kind, T, args.cpu_sample_tokens, sel_bytes,
                                           args.cpu_seconds)
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


PREFILL_SAMPLE = {"c2": 128, "c3": 64, "c4": 64, "c2-w4a8": 128, "c2-bf16": 128}


def cpu_baseline(lay, xs, kind, T, sample_tokens, sel_bytes, seconds):
    """The oracle (float64 NumPy, as it stands) on a bounded sample of the
    same workload, timed on this host's cores."""
    import oracle
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    if kind == "decode":
        # whole decode steps over the same token batches, until `seconds` have passed
        done, nbytes = 0, 0.0
        t0 = time.perf_counter()
        while True:
            b = done % len(xs)
            oracle.forward(lay, xs[b])
            nbytes += sel_bytes[b]
            done += 1
            dt = time.perf_counter() - t0
            if dt >= seconds or done >= 256:
                break
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{done} full decode steps (T={T}) of the same layer and token batches, per-token "
                          f"oracle loop", "seconds": round(dt, 2)}
    n = sample_tokens or PREFILL_SAMPLE.get(lay.cfg.name, 32)
    tok = np.arange(n)
    s_h = None
    if lay.cfg.act == "fp8":
        s_h = 1.0  # the sample measures the per-token arithmetic; the h scale only sets magnitudes
    t0 = time.perf_counter()
    oracle.forward_tokens(lay, xs[0], tok, s_h=s_h)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of the {T} tokens through the per-token oracle loop (experts dequantised once "
                      f"each, included)", "seconds": round(dt, 2)}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a known-size copy), or None when
    there is none or the kernel sources changed since it was taken."""
    import hashlib
    import re
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m_b or not m_h:
        return None
    return int(m_b.group(1)) if m_h.group(1) == kernel_source_sha() else None


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
