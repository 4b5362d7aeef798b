"""GPU parity for every weight format / activation mode on small layers, at
token counts that take each kernel path: decode (T <= 16), prefill with
64-row blocks, and prefill with 128-row blocks whose column tiles reach past
the layer's width (idle waves).  Expected values come from the oracle."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import oracle
import synth
from gpu_util import DEV, rel_fro, run_forward, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LAYERS = {
    # name: (hidden, experts, top_k, inter, format, activations, shared_inter)
    "mx384": (384, 8, 2, 384, "mxfp4", "bf16", 0),
    "nv256": (256, 8, 2, 128, "nvfp4", "bf16", 128),
    "f8a8": (256, 8, 2, 256, "fp8", "fp8", 0),
    "f8bf": (256, 8, 2, 128, "fp8", "bf16", 0),
    "mx8a": (512, 8, 2, 384, "mxfp4", "mxfp8", 128),
    # fp32 multipliers per matrix row, or per part of the fused gate_up
    "f8row": (256, 8, 2, 256, "fp8", "fp8", 0, {"scale_mode": "row"}),
    "f8part": (256, 8, 2, 128, "fp8", "bf16", 0, {"scale_mode": "part"}),
    "nvrow": (256, 8, 2, 128, "nvfp4", "bf16", 128, {"scale_mode": "row"}),
    # BF16 experts (with a shared expert)
    "bf16w": (256, 8, 2, 256, "bf16", "bf16", 128),
    # Zipf router bias used for the selection only
    "mxsel": (384, 16, 4, 256, "mxfp4", "bf16", 0, {"zipf_s": 1.1, "zipf_ratio": 2.5, "bias_mode": "select"}),
}
TOKENS = [(5, "auto"), (16, "decode"), (70, "prefill"), (1024, "prefill")]

_cache = {}


def layer(name, packed=False):
    if packed and LAYERS[name][4] == "bf16":
        pytest.skip("BF16 experts have no packed layout")
    key = (name, packed)
    if key not in _cache:
        H, E, k, I, fmt, act, Is = LAYERS[name][:7]
        extra = LAYERS[name][7] if len(LAYERS[name]) > 7 else {}
        if (name, False) in _cache:
            lay = _cache[(name, False)][0]
        else:
            cfg = synth.LayerConfig(name, (16,), H, E, k, I, fmt, act=act, shared_inter=Is, seed=7, **extra)
            lay = synth.make_layer(cfg, cache=False)
        dlay = ft.DeviceLayer.from_host(lay, DEV)
        _cache[key] = (lay, dlay.pack() if packed else dlay)
    return _cache[key]


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("T,path", TOKENS)
@pytest.mark.timeout(600)
def test_format_parity(name, T, path):
    say(f"format parity {name} T={T} path={path}")
    lay, dlay = layer(name)
    x = synth.make_tokens(lay, T, stream=T)
    y, ids, w = run_forward(dlay, x, path)
    ref = oracle.forward(lay, x)
    assert np.array_equal(ids, ref["ids"])
    assert np.abs(w - ref["w"]).max() <= 1e-5
    err = rel_fro(y, ref["y"])
    say(f"  rel_fro={err:.3e} max_abs={np.abs(y - ref['y']).max():.3e}")
    assert np.isfinite(y).all()
    assert err <= (3e-2 if LAYERS[name][5] in ("fp8", "mxfp8") else 2e-2)


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("T,path", [(70, "prefill"), (1024, "prefill"), (16, "decode")])
@pytest.mark.timeout(600)
def test_packed_weights_give_identical_outputs(name, T, path):
    """The prefill tile layout changes only where the GEMMs read their weight
    stages from, so outputs equal the row-major ones bit for bit (decode
    ignores it)."""
    say(f"packed weights {name} T={T} path={path}")
    lay, dlay = layer(name)
    _, play = layer(name, packed=True)
    x = synth.make_tokens(lay, T, stream=T)
    y0, ids0, w0 = run_forward(dlay, x, path)
    y1, ids1, w1 = run_forward(play, x, path)
    assert np.array_equal(ids0, ids1) and np.array_equal(w0, w1)
    assert np.array_equal(y0, y1)
