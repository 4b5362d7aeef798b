"""The benchmark's own arithmetic, on the CPU: the refusal of more than one
GPU, the per-expert byte counts against the formats' definitions, and the
roofline fields against values worked out by hand from their definitions
(achieved = algorithmic bytes or flops per launch / launch time; frac =
achieved / the published peak)."""
import json
import os
import subprocess
import sys

import pytest

from synth import LayerConfig, make_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def _tiny(fmt, act="bf16", shared=0):
    cfg = LayerConfig(f"tiny-{fmt}-{act}", (16,), 256, 8, 2, 128, fmt, act=act, shared_inter=shared, seed=5)
    return cfg, make_layer(cfg, cache=False)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "fp8", "bf16"])
def test_per_expert_bytes_follow_the_formats(fmt):
    # one expert's gate_up [2I][H] and down [H][I]: codes, block scales, tensor scale
    cfg, lay = _tiny(fmt)
    H, I = cfg.hidden, cfg.inter
    elem = {"mxfp4": 0.5, "nvfp4": 0.5, "fp8": 1.0, "bf16": 2.0}[fmt]
    block = {"mxfp4": 32, "nvfp4": 16}.get(fmt)   # one 1-byte scale per block
    tensor = 4 if fmt in ("nvfp4", "fp8") else 0  # one fp32 per matrix
    for q, (n, k) in ((lay.gate_up, (2 * I, H)), (lay.down, (H, I))):
        want = int(n * k * elem) + (n * (k // block) if block else 0) + tensor
        assert bench.per_expert_bytes(q) == want


def test_the_30b_class_decode_units_match_their_definition():
    # the 30B-A3B-class MXFP4 layer: gate_up 1536 x 2048 and down 2048 x 768
    gate_up = 1536 * 2048 // 2 + 1536 * 2048 // 32
    down = 2048 * 768 // 2 + 2048 * 768 // 32
    assert (gate_up, down) == (1_671_168, 835_584)


def test_decode_roofline_arithmetic():
    cfg, lay = _tiny("mxfp4")
    gu, dn = bench.per_expert_bytes(lay.gate_up), bench.per_expert_bytes(lay.down)
    res = {"lay": lay, "cfg": cfg, "kernel_us": {"decode_gateup": 2.0, "decode_down": 1.0},
           "mean_bytes": 3.0 * (gu + dn)}   # three distinct experts per step
    r = bench.decode_roofline(res)
    assert r["kernel"] == "decode_gateup" and r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["algorithmic_bytes_per_launch"] == int(3 * gu)
    achieved = 3 * gu / 2.0e-6 / 1e9
    assert r["achieved"] == pytest.approx(achieved, abs=0.051)
    assert r["peak"] == 8000.0
    assert r["frac"] == pytest.approx(achieved / 8000.0, abs=1e-4)
    assert r["expert_kernels_GBs"] == pytest.approx(3 * (gu + dn) / 3.0e-6 / 1e9, abs=0.051)


@pytest.mark.parametrize("fmt,act,peak", [("mxfp4", "bf16", 2516.6), ("mxfp4", "mxfp8", 5033.2),
                                          ("fp8", "fp8", 5033.2), ("nvfp4", "bf16", 2516.6)])
def test_prefill_roofline_arithmetic(fmt, act, peak):
    cfg, lay = _tiny(fmt, act)
    T, H, I, k = 512, cfg.hidden, cfg.inter, cfg.top_k
    gu, dn = bench.per_expert_bytes(lay.gate_up), bench.per_expert_bytes(lay.down)
    res = {"lay": lay, "cfg": cfg, "T": T, "kernel_us": {"gemm_gateup": 10.0, "gemm_down": 5.0},
           "mean_bytes": 8.0 * (gu + dn)}
    r = bench.prefill_roofline(res)
    flops = 2.0 * T * k * H * 2 * I   # gate_up: T k routed rows x 2I outputs x H
    assert r["algorithmic_flops_per_launch"] == flops
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == peak
    # (the line rounds achieved figures to one decimal)
    assert r["achieved"] == pytest.approx(flops / 10e-6 / 1e12, abs=0.051)
    assert r["frac"] == pytest.approx(flops / 10e-6 / 1e12 / peak, abs=1e-4)
    # gate_up and down together: 3/2 of gate_up's flops over both launches
    assert r["grouped_gemms_TFLOPs"] == pytest.approx(1.5 * flops / 15e-6 / 1e12, abs=0.051)
    # the strict byte count: 8 experts' gate_up matrices + T activation rows + T k rows of h
    x_row, h_row = {("mxfp4", "bf16"): (2 * H + H // 32, 2 * I + I // 32),
                    ("mxfp4", "mxfp8"): (H + H // 32, I + I // 32),
                    ("fp8", "fp8"): (H, 2 * I), ("nvfp4", "bf16"): (2 * H, 2 * I)}[(fmt, act)]
    assert r["algorithmic_bytes_per_launch"] == int(8 * gu + T * x_row + T * k * h_row)


def test_traffic_is_withheld_when_no_counter_summary_matches():
    # a kernel / workload pair without a committed counter summary reports none
    assert bench.measured_traffic("decode_gateup", "no-such-workload") is None
