"""The host half of CPU-GPU co-execution (ftmoe_host_expert_rows): routed
SwiGLU experts computed on the host cores from host-resident matrices, for
every weight format and activation mode the co-execution supports, against
the oracle's expert (dequantised matrices, fp64) on the same rows.  No GPU:
this is product code that runs on the host.  Bar: relative Frobenius error
1e-2 (h is rounded to bf16 as on the device: measured about 2e-3; with
MXFP8 activations both sides quantise x and h the same way: about 1e-8);
a row's output does not depend on the other rows of the call (bit for
bit)."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import oracle
import synth

LAYERS = {
    # H, E, k, I, weight format, activations, extra generator options
    "mx": (256, 8, 2, 128, "mxfp4", "bf16", {}),
    "mx8a": (512, 8, 2, 384, "mxfp4", "mxfp8", {}),
    "nv": (256, 8, 2, 256, "nvfp4", "bf16", {}),
    "nvrow": (256, 8, 2, 128, "nvfp4", "bf16", {"scale_mode": "row"}),
    "f8": (256, 8, 2, 128, "fp8", "bf16", {}),
    "f8part": (384, 8, 2, 128, "fp8", "bf16", {"scale_mode": "part"}),
    "bf16": (256, 8, 2, 256, "bf16", "bf16", {}),
}


def _layer(name):
    H, E, k, I, fmt, act, extra = LAYERS[name]
    return synth.make_layer(synth.LayerConfig(name, (16,), H, E, k, I, fmt, act=act, seed=11, **extra), cache=False)


def _oracle_rows(lay, x, tok, ex):
    xf = oracle.bf16_to_f64(x)
    xq = oracle.quant_act_mxfp8(xf)[0] if lay.cfg.act == "mxfp8" else xf
    out = []
    for t, e in zip(tok, ex):
        wgu, wd = oracle.dequant(lay.gate_up, int(e)), oracle.dequant(lay.down, int(e))
        h = oracle.swiglu_expert(wgu, wd, xq[t])[0]
        if lay.cfg.act == "mxfp8":
            h = oracle.quant_act_mxfp8(h)[0]
        out.append(wd @ h)
    return np.array(out)


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_host_expert_rows_match_oracle(name):
    lay = _layer(name)
    T = 24
    x = synth.make_tokens(lay, T, stream=4)
    rng = np.random.default_rng(5)
    # ragged: one expert with many rows (groups of four and a tail), others with one or two
    ex = np.concatenate([np.full(11, 3), rng.integers(0, lay.cfg.num_experts, 26)]).astype(np.int32)
    tok = rng.integers(0, T, len(ex)).astype(np.int32)
    o = ft.host_expert_rows(lay, x, tok, ex, threads=3)
    ref = _oracle_rows(lay, x, tok, ex)
    err = np.linalg.norm(o - ref) / np.linalg.norm(ref)
    assert np.isfinite(o).all()
    assert err <= 1e-2, err
    # each row alone gives the same bits
    for r in (0, 5, 11, len(ex) - 1):
        alone = ft.host_expert_rows(lay, x, tok[r:r + 1], ex[r:r + 1], threads=1)
        assert np.array_equal(alone[0], o[r])


def test_host_expert_rows_empty_and_refusals():
    lay = _layer("mx")
    x = synth.make_tokens(lay, 4)
    assert ft.host_expert_rows(lay, x, [], [], threads=2).shape == (0, lay.cfg.hidden)
    with pytest.raises(ft.FtmoeError) as err:
        ft.host_expert_rows(lay, x, [0], [lay.cfg.num_experts], threads=1)
    assert err.value.status == ft.ERR_INVALID_ARG
    f8a8 = synth.make_layer(synth.LayerConfig("f8a8", (16,), 256, 8, 2, 128, "fp8", act="fp8", seed=11), cache=False)
    with pytest.raises(ft.FtmoeError) as err:
        ft.host_expert_rows(f8a8, synth.make_tokens(f8a8, 2), [0], [0], threads=1)
    assert err.value.status == ft.ERR_UNSUPPORTED
