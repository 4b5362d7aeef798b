"""GPU parity at the edges of the code tables, through the C ABI against the
oracle in float64 (expected values from the oracle only).

Crafted layers (``synth.crafted``) make every code of a format occur and
matter to the output:
- MXFP4 weight blocks under every E8M0 scale code 0..254 (bf16 activations,
  carried as split E4M3 pairs, and MXFP8 activations);
- NVFP4 blocks under every non-negative finite E4M3 block scale, the zero
  scale, the subnormals and 448 included, with a shared expert;
- FP8 weights using all 254 finite E4M3 codes (with bf16 and with per-tensor
  FP8 activations);
and hidden states with about 2^16 of dynamic range inside each 32-block run
through layers of every format.  Both expert paths (decode and prefill,
row-major and packed weights) run each case.

Bars as for the other forward tests: routing ids bit-exact, weights within
1e-5, relative Frobenius error of y within 2e-2 (3e-2 with 8-bit
activations), and every token's row within twice that."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import oracle
from gpu_util import DEV, rel_fro, run_forward, say
from synth.crafted import CRAFTED, WIDE, crafted_layer, crafted_tokens

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

_cache = {}


def layer(name, packed):
    key = (name, packed)
    if key not in _cache:
        lay = _cache.get((name, None))
        if lay is None:
            lay = crafted_layer(name)
            _cache[(name, None)] = lay
        dl = ft.DeviceLayer.from_host(lay, DEV)
        _cache[key] = dl.pack() if packed else dl
    return _cache[(name, None)], _cache[key]


def bar(lay):
    return 3e-2 if lay.cfg.act in ("fp8", "mxfp8") else 2e-2


CASES = [(n, T, path, packed) for n in sorted(CRAFTED) + sorted(WIDE)
         for (T, path, packed) in ((5, "decode", False), (16, "decode", False), (70, "prefill", False),
                                   (70, "prefill", True))]


@pytest.mark.parametrize("name,T,path,packed", CASES)
@pytest.mark.timeout(300)
def test_code_table_edges(name, T, path, packed):
    say(f"edge layer {name} T={T} path={path} packed={packed}")
    lay, dlay = layer(name, packed)
    x = crafted_tokens(lay, T, stream=T, wide=name in WIDE)
    y, ids, w = run_forward(dlay, x, path)
    ref = oracle.forward(lay, x)
    assert np.array_equal(ids, ref["ids"])
    assert np.abs(w - ref["w"]).max() <= 1e-5
    assert np.isfinite(y).all()
    err = rel_fro(y, ref["y"])
    rows = np.linalg.norm(y - ref["y"], axis=1) / np.linalg.norm(ref["y"], axis=1)
    say(f"  rel_fro={err:.3e} worst row {rows.max():.3e} (token {int(rows.argmax())}) "
        f"max_abs={np.abs(y - ref['y']).max():.3e}")
    assert err <= bar(lay)
    assert rows.max() <= 2 * bar(lay)
