"""Pins for the oracle's MoE forward.

Closed forms: E=1, k=1 is a dense SwiGLU MLP (computed here with torch's
F.linear / F.silu in float64); k=E gives the full softmax (torch.softmax).
Invariants: token permutation, weights summing to one in descending order,
counts summing to T*k.  Brute force: every expert on every token mixed by
the dense renormalised top-k mask.  A hand-worked MXFP4 example under
tests/golden fixes packing, scale, gate/up order and the combine."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from synth import LayerConfig, make_layer, make_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(fmt="mxfp4", H=64, E=4, k=2, I=64, act="bf16", shared=0, seed=11, std=None, zipf=None, scale="tensor"):
    cfg = LayerConfig("tiny", (8,), H, E, k, I, fmt, act=act, shared_inter=shared,
                      router_std=std, zipf_s=zipf, seed=seed, scale_mode=scale)
    return make_layer(cfg, cache=False)


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _torch_dense(lay, e, x, qact=False):
    """SwiGLU MLP of expert e by torch ops, float64."""
    wgu = _t(oracle.dequant(lay.gate_up, e))
    wd = _t(oracle.dequant(lay.down, e))
    I = wgu.shape[0] // 2
    a = F.linear(x, wgu)
    return F.silu(a[:, :I]) * a[:, I:], wd


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "fp8", "bf16"])
def test_single_expert_is_dense_swiglu(fmt):
    lay = tiny(fmt, E=1, k=1, H=64, I=32)
    x = make_tokens(lay, 6)
    r = oracle.forward(lay, x)
    assert np.all(r["w"] == 1.0) and np.all(r["ids"] == 0)
    xt = _t(oracle.bf16_to_f64(x))
    h, wd = _torch_dense(lay, 0, xt)
    ref = F.linear(h, wd).numpy()
    assert np.abs(r["y"] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_single_expert_fp8_activations_match_torch_quantiser():
    """E=1, k=1 with per-tensor E4M3 activations: x and h are quantised with
    torch's float8_e4m3fn conversion (scale amax/448 in fp32)."""
    lay = tiny("fp8", E=1, k=1, H=64, I=32, act="fp8")
    x = make_tokens(lay, 12)
    r = oracle.forward(lay, x)

    def q(v64):
        v = v64.to(torch.float32)
        s = v.abs().max() / 448.0
        return (v / s).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64) * s.double()

    xt = q(_t(oracle.bf16_to_f64(x)))
    h, wd = _torch_dense(lay, 0, xt)
    ref = F.linear(q(h), wd).numpy()
    assert np.abs(r["y"] - ref).max() <= 1e-12 * np.abs(ref).max()


def _torch_mxfp8(v64):
    """MXFP8 quantise-dequantise by torch ops: block exponent from
    torch.frexp, elements through torch's float8_e4m3fn conversion."""
    v = v64.to(torch.float32)
    b = v.reshape(*v.shape[:-1], -1, 32)
    amax = b.abs().amax(-1)
    _, ex = torch.frexp(amax)
    X = torch.where(amax > 0, ex.to(torch.int64) - 9, torch.full_like(ex, -127, dtype=torch.int64)).clamp(min=-127)
    p2 = torch.pow(torch.tensor(2.0, dtype=torch.float64), X.to(torch.float64))[..., None]
    q = (b.double() / p2).to(torch.float32).clamp(-448, 448).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * p2).reshape(v.shape), q.view(torch.uint8).reshape(v.shape), X


def test_single_expert_mxfp8_activations_match_torch_quantiser():
    """E=1, k=1 with MXFP8 activations (and a shared expert): x, h and the
    shared expert's h go through the torch MXFP8 quantiser above."""
    lay = tiny("mxfp4", E=1, k=1, H=64, I=64, act="mxfp8", shared=32)
    x = make_tokens(lay, 12)
    r = oracle.forward(lay, x)
    xf = _t(oracle.bf16_to_f64(x))
    xt = _torch_mxfp8(xf)[0]
    h, wd = _torch_dense(lay, 0, xt)
    ref = F.linear(_torch_mxfp8(h)[0], wd)
    wgs = _t(oracle.dequant(lay.shared_gate_up, 0))
    wds = _t(oracle.dequant(lay.shared_down, 0))
    a = F.linear(xt, wgs)
    hs = F.silu(a[:, :32]) * a[:, 32:]
    sg = torch.sigmoid(xf @ _t(lay.shared_gate_w))
    ref = ref + sg[:, None] * F.linear(_torch_mxfp8(hs)[0], wds)
    assert np.abs(r["y"] - ref.numpy()).max() <= 1e-12 * np.abs(ref.numpy()).max()


def test_mxfp8_quantiser_definition():
    """Block exponent by its defining inequality 2^(X+8) <= amax < 2^(X+9)
    (X = -127 for a zero block and below E8M0's range), element codes and
    values against torch's E4M3 conversion."""
    rng = np.random.default_rng(21)
    v = rng.standard_normal((6, 8, 32)) * np.exp2(rng.integers(-20, 20, (6, 8, 1)))
    v[0, 0] = 0.0                       # zero block
    v[0, 1] = 0.0
    v[0, 1, 5] = 2.0 ** -130            # fp32 subnormal maximum
    v[0, 2, :] = 1e-3
    v[0, 2, 7] = 2.0 ** -118            # exponent clamped at -127
    v[0, 3, :] = 0.1
    v[0, 3, 3] = 8.0                    # amax an exact power of two: X = 3 - 8
    v[0, 4, :] = 0.1
    v[0, 4, 9] = -15.5                  # X = -5 and 15.5 * 32 = 496 saturates to 448
    v = v.reshape(6, 256)
    deq, codes, sc = oracle.quant_act_mxfp8(v)
    assert sc.shape == (6, 8) and codes.shape == v.shape
    v32 = v.astype(np.float32).astype(np.float64)
    for r in range(6):
        for b in range(8):
            amax = np.abs(v32[r, 32 * b:32 * b + 32]).max()
            X = int(sc[r, b]) - 127
            if amax == 0 or amax < 2.0 ** -119:
                assert X == -127
            else:
                assert 2.0 ** (X + 8) <= amax < 2.0 ** (X + 9)
    assert int(sc[0, 3]) - 127 == 3 - 8
    tq, tc, tX = _torch_mxfp8(torch.from_numpy(v))
    assert np.array_equal(tX.numpy() + 127, sc.astype(np.int64))
    assert np.array_equal(tc.numpy(), codes)
    assert np.array_equal(tq.numpy(), deq)
    assert deq[0, 3 * 32 + 3] == 8.0 and codes[0, 3 * 32 + 3] == 0x78
    assert int(sc[0, 4]) - 127 == -5 and deq[0, 4 * 32 + 9] == -448 * 2.0 ** -5


def test_mxfp8_hand_example():
    """One block worked by hand: amax 1.9 gives X = -8 (floor(log2 1.9) = 0);
    1.9 * 256 = 486.4 saturates to 448 (value 1.75); 1.0 -> 256 = 2^8 (code
    0x78: exponent field 15, mantissa 0); 0.5 -> 128 (0x70); 0.001 * 256 =
    0.256 -> 0.25 = 2^-2 (0x28); -0.3 * 256 = -76.8 -> -80 (sign 1, exponent
    field 13, mantissa 2: 0xEA, since 72 < 76.8 and 80 - 76.8 < 76.8 - 72)."""
    v = np.zeros(32)
    v[:5] = [1.9, 1.0, 0.5, 0.001, -0.3]
    deq, codes, sc = oracle.quant_act_mxfp8(v)
    assert sc.tolist() == [127 - 8]
    assert codes[:5].tolist() == [0x7E, 0x78, 0x70, 0x28, 0xEA]
    assert np.array_equal(deq[:5], [1.75, 1.0, 0.5, 2.0 ** -10, -80 / 256])
    assert np.all(codes[5:] == 0) and np.all(deq[5:] == 0)


def test_selection_only_bias_ranks_biased_and_weights_unbiased():
    """bias_mode "select": torch.topk of x W^T + b picks the experts (the
    generator keeps a gap at the k-th place, so the order is unique) and the
    weights are torch.softmax of the selected x W^T, without b."""
    lay = tiny("mxfp4", E=16, k=3, zipf=1.1)
    lay.cfg = synth.LayerConfig(**{**lay.cfg.__dict__, "bias_mode": "select"})
    x = make_tokens(lay, 20)
    lg, ids, w = oracle.route(lay, oracle.bf16_to_f64(x))
    xt = _t(oracle.bf16_to_f64(x))
    raw = F.linear(xt, _t(lay.router_w))
    top = torch.topk(raw + _t(lay.router_b), 3, dim=1)
    assert np.array_equal(ids, top.indices.numpy())
    assert np.abs(lg - raw.numpy()).max() <= 1e-12
    ref_w = torch.softmax(torch.gather(raw, 1, top.indices), dim=1).numpy()
    assert np.abs(w - ref_w).max() <= 1e-12
    r = oracle.forward(lay, x)
    assert np.array_equal(r["ids"], ids) and np.abs(r["w"] - ref_w).max() <= 1e-12
    b = oracle.forward_all_experts_masked(lay, x)
    assert np.abs(r["y"] - b).max() <= 1e-12 * np.abs(b).max()
    # the default mode puts the bias into the weights as well
    lay.cfg = synth.LayerConfig(**{**lay.cfg.__dict__, "bias_mode": "logits"})
    _, ids0, w0 = oracle.route(lay, oracle.bf16_to_f64(x))
    assert np.array_equal(ids0, ids) and np.abs(w0 - w).max() > 1e-3


def test_k_equal_E_gives_full_softmax():
    lay = tiny(E=4, k=4)
    x = make_tokens(lay, 8)
    r = oracle.forward(lay, x)
    full = torch.softmax(_t(r["logits"]), dim=1).numpy()
    got = np.zeros_like(full)
    np.put_along_axis(got, r["ids"].astype(np.int64), r["w"], axis=1)
    assert np.abs(got - full).max() <= 1e-15


def test_router_logits_match_torch_linear_with_bias():
    lay = tiny("fp8", E=8, k=2, zipf=1.1)
    assert lay.router_b is not None and np.any(lay.router_b != 0)
    x = make_tokens(lay, 16)
    xf = oracle.bf16_to_f64(x)
    ref = F.linear(_t(xf), _t(lay.router_w), _t(lay.router_b)).numpy()
    assert np.abs(oracle.router_logits(lay, xf) - ref).max() <= 1e-13


@pytest.mark.parametrize("fmt,act,shared,scale", [("mxfp4", "bf16", 0, "tensor"), ("nvfp4", "bf16", 32, "tensor"),
                                                  ("fp8", "bf16", 0, "tensor"), ("mxfp4", "mxfp8", 32, "tensor"),
                                                  ("fp8", "bf16", 0, "row"), ("nvfp4", "bf16", 32, "part"),
                                                  ("bf16", "bf16", 32, "tensor")])
def test_brute_force_all_experts_masked(fmt, act, shared, scale):
    lay = tiny(fmt, E=8, k=3, H=64, I=32, shared=shared, act=act, scale=scale)
    x = make_tokens(lay, 16)
    r = oracle.forward(lay, x)
    b = oracle.forward_all_experts_masked(lay, x)
    assert np.abs(r["y"] - b).max() <= 1e-12 * np.abs(b).max()


@pytest.mark.parametrize("act", ["bf16", "fp8", "mxfp8"])
def test_token_permutation_is_bitwise(act):
    lay = tiny("fp8" if act == "fp8" else "mxfp4", E=8, k=2, act=act)
    x = make_tokens(lay, 16)
    perm = np.random.default_rng(0).permutation(16)
    a = oracle.forward(lay, x)
    b = oracle.forward(lay, x[perm])
    assert np.array_equal(a["ids"][perm], b["ids"])
    assert np.array_equal(a["y"][perm], b["y"])
    ca = np.bincount(a["ids"].ravel(), minlength=8)
    cb = np.bincount(b["ids"].ravel(), minlength=8)
    assert np.array_equal(ca, cb) and ca.sum() == 16 * 2


def test_weights_sum_to_one_and_descend():
    lay = make_layer("c0")
    x = make_tokens(lay, 16)
    r = oracle.forward(lay, x)
    assert np.abs(r["w"].sum(1) - 1).max() <= 1e-15
    assert np.all(r["w"][:, :-1] >= r["w"][:, 1:])
    lg = r["logits"]
    sel = np.take_along_axis(lg, r["ids"].astype(np.int64), 1)
    assert np.all(sel[:, :-1] > sel[:, 1:])


def test_topk_matches_full_sort_and_breaks_ties_low_index():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 16))
    lg[0, [3, 9, 12]] = 5.0  # three-way tie at the top
    ids = oracle.select_topk(lg, 4)
    ref = np.argsort(-lg, axis=1, kind="stable")[:, :4]
    assert np.array_equal(ids, ref)
    assert ids[0, :3].tolist() == [3, 9, 12]


@pytest.mark.parametrize("fmt,act,shared", [("mxfp4", "bf16", 0), ("nvfp4", "bf16", 32), ("fp8", "fp8", 0),
                                            ("mxfp4", "mxfp8", 32)])
def test_grouped_mode_matches_per_token_mode(fmt, act, shared):
    lay = tiny(fmt, E=8, k=2, act=act, shared=shared)
    x = make_tokens(lay, 24)
    a = oracle.forward(lay, x)
    g = oracle.forward_grouped(lay, x)
    assert np.abs(a["y"] - g["y"]).max() <= 1e-12 * np.abs(a["y"]).max()
    sub = [3, 7, 20]
    ft = oracle.forward_tokens(lay, x, sub, s_h=g.get("s_h"))
    assert np.abs(ft - a["y"][sub]).max() <= 1e-12 * np.abs(a["y"]).max()
    g2 = oracle.forward_grouped(lay, x, tokens=sub)
    assert np.abs(g2["y"] - a["y"][sub]).max() <= 1e-12 * np.abs(a["y"]).max()


def test_hand_worked_mxfp4_example():
    with open(os.path.join(GOLDEN, "tiny_mxfp4_by_hand.json")) as f:
        g = json.load(f)
    H, E, k, I = g["H"], g["E"], g["k"], g["I"]

    class L:  # duck-typed layer
        pass

    lay = L()
    lay.cfg = LayerConfig("hand", (2,), H, E, k, I, "mxfp4")
    lay.router_w = np.zeros((E, H), np.float32)
    for e, c in enumerate(g["router_w_unit_rows"]):
        lay.router_w[e, c] = 1.0
    lay.router_b = None
    lay.shared_gate_w = None

    def qw(n, kk, bytes_, scales):
        codes = np.zeros((E, n, kk // 2), np.uint8)
        sc = np.full((E, n, kk // 32), 127, np.uint8)
        for e, r, b, v in bytes_:
            codes[e, r, b] = v
        for e, r, b, v in scales:
            sc[e, r, b] = v
        return synth.QWeight("mxfp4", E, n, kk, codes, sc, None)

    lay.gate_up = qw(2 * I, H, g["gate_up_bytes"], g["gate_up_scales"])
    lay.down = qw(H, I, g["down_bytes"], g["down_scales"])
    x = np.zeros((2, H), np.float32)
    for t, row in enumerate(g["x"]):
        x[t, :len(row)] = row
    r = oracle.forward(lay, synth.f32_to_bf16_bits(x))
    assert r["ids"].tolist() == g["expected_ids"]
    want = np.zeros((2, H))
    for t, n, expr in g["expected_y"]:
        want[t, n] = eval(expr, {"exp": math.exp})
    assert np.abs(r["y"] - want).max() <= 1e-13


# ------------------------------------------------------------------ align --


def _align_brute(ids, E, BM):
    """Definition restated set-wise: expert segments in expert order, each the
    sorted list of flat rows routed to it, padded to a multiple of BM."""
    flat = ids.reshape(-1)
    out, blocks = [], []
    for e in range(E):
        rows = sorted(i for i in range(flat.size) if flat[i] == e)
        if not rows:
            continue
        nb = -(-len(rows) // BM)
        out += rows + [flat.size] * (nb * BM - len(rows))
        blocks += [e] * nb
    return out, blocks


@pytest.mark.parametrize("T,k,E,BM", [(1, 8, 128, 16), (8, 8, 128, 16), (16, 2, 8, 4),
                                      (37, 3, 5, 8), (64, 4, 16, 1), (5, 5, 5, 64), (0, 2, 4, 8)])
def test_align_definition(T, k, E, BM):
    rng = np.random.default_rng(T * 131 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    counts, offsets, sorted_ids, block_expert, npad = oracle.align(ids, E, BM)
    seg, blocks = _align_brute(ids, E, BM)
    assert npad == len(seg)
    assert sorted_ids[:npad].tolist() == seg
    assert np.all(sorted_ids[npad:] == T * k)
    assert block_expert[:npad // BM].tolist() == blocks
    assert np.all(block_expert[npad // BM:] == -1)
    assert counts.sum() == T * k
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert np.all(offsets % BM == 0) and offsets[-1] == npad
    assert len(sorted_ids) == oracle.align_max_padded(T, k, E, BM) >= npad


def test_align_hand_example():
    # tokens: t0 -> (2, 0), t1 -> (0, 1), t2 -> (2, 1); BM = 2
    ids = np.array([[2, 0], [0, 1], [2, 1]], np.int32)
    counts, offsets, sorted_ids, block_expert, npad = oracle.align(ids, 3, 2)
    assert counts.tolist() == [2, 2, 2]
    assert offsets.tolist() == [0, 2, 4, 6]
    # flat rows: 0:e2 1:e0 2:e0 3:e1 4:e2 5:e1
    assert sorted_ids[:6].tolist() == [1, 2, 3, 5, 0, 4]
    assert block_expert[:3].tolist() == [0, 1, 2]
    ids2 = np.array([[1, 0]], np.int32)
    c2, o2, s2, b2, n2 = oracle.align(ids2, 3, 4)
    assert o2.tolist() == [0, 4, 8, 8] and s2[:8].tolist() == [1, 2, 2, 2, 0, 2, 2, 2]


def test_fp8_activation_quantiser_definition():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((7, 33)) * 3
    deq, s, codes = oracle.quant_act_per_tensor(v)
    v32 = v.astype(np.float32)
    assert s == np.float32(np.abs(v32).max() / np.float32(448))
    ref = torch.from_numpy(v32 / np.float32(s)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.abs(deq).max() == 448 * s
    z, s0, _ = oracle.quant_act_per_tensor(np.zeros((2, 3)))
    assert s0 == 1.0 and np.all(z == 0)
