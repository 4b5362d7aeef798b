"""Generator contract: determinism per seed, the top-k gap, the Zipf skew."""
import numpy as np
import pytest

import oracle
import synth
from synth import LayerConfig, make_layer, make_tokens


def test_deterministic_per_seed():
    a = make_layer("c0", cache=False)
    b = make_layer("c0", cache=False)
    assert np.array_equal(a.gate_up.codes, b.gate_up.codes)
    assert np.array_equal(a.down.block_scales, b.down.block_scales)
    assert np.array_equal(make_tokens(a, 16), make_tokens(b, 16))
    assert not np.array_equal(make_tokens(a, 16, stream=1), make_tokens(a, 16))


def test_topk_gap_holds_in_fp64():
    lay = make_layer("c0")
    x = make_tokens(lay, 16)
    lg = oracle.router_logits(lay, oracle.bf16_to_f64(x))
    top = -np.sort(-lg, axis=1)[:, :lay.top_k + 1]
    assert (top[:, :-1] - top[:, 1:]).min() >= 1e-3


def test_token_prefix_stable():
    lay = make_layer("c0")
    assert np.array_equal(make_tokens(lay, 16)[:4], make_tokens(lay, 4))


def test_zipf_bias_skews_load():
    cfg = LayerConfig("z", (4096,), 64, 16, 2, 32, "fp8", act="fp8", zipf_s=1.1, zipf_ratio=4.0, seed=7)
    lay = make_layer(cfg, cache=False)
    assert abs(lay.extra["calibration_ratio"] - 4.0) < 0.3
    x = make_tokens(lay, 4096)
    ids = oracle.select_topk(oracle.router_logits(lay, oracle.bf16_to_f64(x)), 2)
    c = np.bincount(ids.ravel(), minlength=16)
    assert 3.0 < c.max() / c.mean() < 5.0


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.00390625, 1.0078125 + 2 ** -9, -3.14159, 1 + 2 ** -8], np.float32)
    b = synth.f32_to_bf16_bits(v)
    back = synth.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0           # exact tie 1 + 2^-8 -> even (1.0)
    assert back[4] == 1.0
    assert back[2] == np.float32(1.0078125)  # a quarter ulp above rounds down


def test_crafted_layers_cover_every_code():
    """The edge-case layers hold what their names promise: every E8M0 scale
    code 0..254, every non-negative finite E4M3 block scale 0..126, and all
    254 finite E4M3 weight codes; their tokens are finite bf16 of the
    intended sizes, and the top-k gap holds."""
    from synth.crafted import crafted_layer, crafted_tokens
    mx = crafted_layer("mx_e8m0")
    assert set(np.unique(mx.gate_up.block_scales[0])) >= set(range(255))
    nv = crafted_layer("nv_e4m3")
    assert set(np.unique(nv.gate_up.block_scales)) == set(range(127))
    f8 = crafted_layer("fp8_all")
    assert set(np.unique(f8.gate_up.codes[0])) == set(range(256)) - {0x7F, 0xFF}
    for lay, wide in ((mx, False), (nv, False), (f8, False), (crafted_layer("wide_mx"), True)):
        x = crafted_tokens(lay, 9, wide=wide)
        xf = synth.bf16_bits_to_f32(x)
        assert np.isfinite(xf).all() and x.shape == (9, lay.cfg.hidden)
        nz = np.abs(xf[xf != 0])
        assert nz.min() >= 2.0 ** -126   # no bf16 subnormals
    xw = synth.bf16_bits_to_f32(crafted_tokens(crafted_layer("wide_mx"), 64, wide=True))
    blk = np.abs(xw.reshape(64, -1, 32))
    assert np.median(blk.max(axis=2) / blk.min(axis=2)) > 2.0 ** 12   # wide range inside a 32-block
