"""GPU parity of the NVFP4 prefill GEMMs' 64 x 128 wave tiles, whose
workgroup spans two packed 512-row weight tiles, on layers where the tile
pair is partly past the matrix: 2I = 768 (the second packed tile half
filled) and 2I = 1280 (the last pair's second tile absent, so its waves have
no columns).  Many small experts make 64-row blocks and enough tiles for the
wide layout.  Every output row is compared with the oracle's grouped mode in
float32, itself held to the float64 per-token loop on a sample; packed
weights (as the benchmark runs them) and the row-major layout both."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import oracle
import synth
from gpu_util import DEV, rel_fro, run_forward, sample_tokens, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LAYERS = {
    # name: (hidden, experts, top_k, inter, shared_inter)
    "nvw384": (512, 256, 8, 384, 0),
    "nvw640": (512, 256, 8, 640, 384),
}
T = 4096   # 128 rows per expert: 64-row blocks, 700+ of them

_cache = {}


def layer(name, packed):
    key = (name, packed)
    if key not in _cache:
        H, E, k, I, Is = LAYERS[name]
        if (name, not packed) in _cache:
            lay = _cache[(name, not packed)][0]
        else:
            cfg = synth.LayerConfig(name, (T,), H, E, k, I, "nvfp4", act="bf16", shared_inter=Is, seed=13)
            lay = synth.make_layer(cfg, cache=False)
        dlay = ft.DeviceLayer.from_host(lay, DEV)
        _cache[key] = (lay, dlay.pack() if packed else dlay)
    return _cache[key]


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.parametrize("packed", [True, False])
@pytest.mark.timeout(600)
def test_wide_nvfp4_tiles_every_row(name, packed):
    say(f"wide NVFP4 tiles {name} T={T} packed={packed}, every row")
    lay, dlay = layer(name, packed)
    x = synth.make_tokens(lay, T, stream=7)
    y, ids, w = run_forward(dlay, x, "prefill")
    g = oracle.forward_grouped(lay, x, dtype=np.float32)
    assert np.array_equal(ids, g["ids"])
    assert np.abs(w - g["w"]).max() <= 1e-5
    tok = sample_tokens(T, 24, seed=3)
    g_err = rel_fro(g["y"][tok], oracle.forward_tokens(lay, x, tok))
    say(f"  grouped float32 oracle vs per-token float64 on {len(tok)} tokens: {g_err:.2e}")
    assert g_err <= 1e-4
    assert np.isfinite(y).all()
    ref = g["y"]
    err = rel_fro(y, ref)
    rows = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    say(f"  rel_fro={err:.3e} worst row {rows.max():.3e}")
    assert err <= 2e-2
    assert rows.max() <= 4e-2


@pytest.mark.parametrize("name", sorted(LAYERS))
@pytest.mark.timeout(600)
def test_wide_nvfp4_tiles_packed_equals_row_major(name):
    """The packed layout changes only where the wide tiles read their
    weight stages from: the outputs are the same bits."""
    say(f"wide NVFP4 tiles {name}: packed == row-major")
    lay, dp = layer(name, True)
    _, dr = layer(name, False)
    x = synth.make_tokens(lay, T, stream=8)
    yp = run_forward(dp, x, "prefill")[0]
    yr = run_forward(dr, x, "prefill")[0]
    assert np.array_equal(yp, yr)
