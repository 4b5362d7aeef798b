"""GPU parity of the one- and two-token decode kernels: the gate_up that
splits each group of weight rows along K (dequantised formats, hidden a
multiple of 512) and the single launch of down and combine for one-token
MXFP4 steps (with a shared expert of the routed experts' width, and with
MXFP8 activations).  Expected values come from the oracle.  A token's output
must also not depend on whether it is decoded alone or beside a second token
(one launch instead of two, the same arithmetic), bit for bit, and the
one-token MXFP4 step must indeed run without a separate combine launch."""
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
    "mxsh": (512, 8, 2, 256, "mxfp4", "bf16", 256),
    "mx8sh": (512, 8, 2, 256, "mxfp4", "mxfp8", 256),
    "mxk8": (512, 16, 8, 256, "mxfp4", "bf16", 0),
    "nvw": (512, 8, 2, 256, "nvfp4", "bf16", 256),
    "f8w": (1024, 8, 2, 256, "fp8", "fp8", 0),
    "f8bw": (512, 8, 2, 256, "fp8", "bf16", 0),
    "bfw": (512, 8, 2, 256, "bf16", "bf16", 256),
}

_cache = {}


def layer(name):
    if name not in _cache:
        H, E, k, I, fmt, act, Is = LAYERS[name]
        cfg = synth.LayerConfig(name, (2,), H, E, k, I, fmt, act=act, shared_inter=Is, seed=11)
        lay = synth.make_layer(cfg, cache=False)
        _cache[name] = (lay, ft.DeviceLayer.from_host(lay, DEV))
    return _cache[name]


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("T", [1, 2])
@pytest.mark.timeout(300)
def test_small_batch_parity(name, T):
    say(f"small-batch decode parity {name} T={T}")
    lay, dlay = layer(name)
    x = synth.make_tokens(lay, T, stream=40 + T)
    y, ids, w = run_forward(dlay, x, "decode")
    ref = oracle.forward(lay, x)
    assert np.array_equal(ids, ref["ids"])
    assert np.abs(w - ref["w"]).max() <= 1e-5
    err = rel_fro(y, ref["y"])
    say(f"  rel_fro={err:.3e} max_abs={np.abs(y - ref['y']).max():.3e}")
    assert np.isfinite(y).all()
    assert err <= (3e-2 if LAYERS[name][5] in ("fp8", "mxfp8") else 2e-2)


# per-tensor FP8 activations take their scale from the whole batch, so a
# token's codes depend on its neighbour; every other mode quantises per row
@pytest.mark.parametrize("name", sorted(n for n in LAYERS if LAYERS[n][5] != "fp8"))
@pytest.mark.timeout(300)
def test_token_alone_equals_token_in_pair(name):
    say(f"one token alone vs beside a second one {name}")
    lay, dlay = layer(name)
    x = synth.make_tokens(lay, 2, stream=50)
    y2, ids2, w2 = run_forward(dlay, x, "decode")
    y1, ids1, w1 = run_forward(dlay, x[:1], "decode")
    assert np.array_equal(ids1[0], ids2[0])
    assert np.array_equal(w1[0], w2[0])
    assert np.array_equal(y1[0], y2[0])


# which launches a step makes: one-token MXFP4 steps run down and combine as
# one launch; other steps keep the separate combine
@pytest.mark.parametrize("name,T,combine", [("mxsh", 1, False), ("mx8sh", 1, False), ("mxsh", 2, True),
                                            ("nvw", 1, True)])
@pytest.mark.timeout(300)
def test_one_token_launches(name, T, combine):
    say(f"launches of a decode step {name} T={T}")
    lay, dlay = layer(name)
    x = synth.make_tokens(lay, T, stream=60)
    ft.timing_collect()
    ft.timing_enable(True)
    try:
        run_forward(dlay, x, "decode")
        torch.cuda.synchronize()
        kern = ft.timing_collect()
    finally:
        ft.timing_enable(False)
    assert "decode_down" in kern and "decode_gateup" in kern
    assert ("combine" in kern) == combine
