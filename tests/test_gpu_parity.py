"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars: routing ids, per-expert counts and the align outputs are bit-exact;
routing weights and the shared gate within 1e-5; the layer output within a
relative Frobenius error of 2e-2 (bf16 activations) or 3e-2 (FP8 per-tensor
or MXFP8 activations), max-abs error reported.  At the benchmark sizes every
output row is compared with the oracle's grouped mode (float32, itself held
to the float64 per-token loop on a sample of tokens; the FP8 layer's h scale
is a whole-batch quantity that the grouped pass supplies), with a bar on each
row as well as on the whole."""
import numpy as np
import pytest

import block_scaled_fp4_router_amd as ft
import oracle
import synth
from gpu_util import DEV, layer_pair, rel_fro, run_forward, sample_tokens, say, to_dev_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def tol_for(name):
    return 3e-2 if synth.CONFIGS[name].act in ("fp8", "mxfp8") else 2e-2


# ------------------------------------------------------------------ route --
# (c3 at 8155 and c2 at 16300 tokens: 128-token router tiles with a ragged
# last tile; for c2 and c2-w4a8 the router also writes the split or MXFP8 x)
@pytest.mark.parametrize("name,T", [("c0", 16), ("c1", 1), ("c1", 8), ("c2", 4096), ("c3", 1), ("c3", 8192),
                                    ("c4", 16384), ("c1", 17), ("c3", 33), ("c4-selbias", 1), ("c4-selbias", 8),
                                    ("c4-selbias", 16384), ("c3", 8155), ("c2", 16300), ("c2-w4a8", 16300)])
@pytest.mark.timeout(600)
def test_route_parity(name, T):
    say(f"route parity {name} T={T}")
    lay, dlay = layer_pair(name)
    x = synth.make_tokens(lay, T)
    xd = to_dev_bf16(x)
    ws = ft.alloc_workspace(dlay, T)
    k = dlay.top_k
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    sg = torch.empty((T,), dtype=torch.float32, device=DEV) if dlay.shared_inter else None
    ft.route(dlay, xd, T, ws, ids, w, sg)
    torch.cuda.synchronize()
    xf = oracle.bf16_to_f64(x)
    _, ref_ids, ref_w = oracle.route(lay, xf)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.abs(w.cpu().numpy() - ref_w).max() <= 1e-5
    if sg is not None:
        assert np.abs(sg.cpu().numpy() - oracle.shared_gate(lay, xf)).max() <= 1e-5
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=dlay.num_experts)
    assert np.array_equal(counts, np.bincount(ref_ids.ravel(), minlength=dlay.num_experts))


# ------------------------------------------------------------------ align --
def _random_ids(T, k, E, seed, skew=None):
    rng = np.random.default_rng(seed)
    if skew is None:
        return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    p = 1.0 / np.arange(1, E + 1) ** skew
    lg = np.log(p)[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-lg, axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,k,E,BM,skew", [(1, 8, 128, 16, None), (8, 8, 128, 16, None), (16, 2, 8, 16, None),
                                           (37, 3, 5, 8, None), (300, 4, 16, 1, None), (4096, 8, 128, 64, None),
                                           (16384, 8, 128, 64, 1.1), (16384, 8, 128, 128, 1.1),
                                           (8192, 10, 512, 64, None),
                                           (129, 16, 16, 64, None), (2000, 1, 1, 128, None),
                                           # more chunks per scan thread than it keeps in registers
                                           (65536, 8, 128, 128, 1.1), (3000, 16, 1024, 64, None)])
@pytest.mark.timeout(300)
def test_align_parity(T, k, E, BM, skew):
    say(f"align parity T={T} k={k} E={E} BM={BM}")
    ids = _random_ids(T, k, E, T * 7 + E, skew)
    counts, offsets, sorted_ids, bexp, npad = oracle.align(ids, E, BM)
    P = ft.align_max_padded(T, k, E, BM)
    assert P == len(sorted_ids)
    d_ids = torch.from_numpy(ids).to(DEV)
    g_counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    g_off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    g_sorted = torch.full((P,), -7, dtype=torch.int32, device=DEV)
    g_bexp = torch.full((P // BM,), -7, dtype=torch.int32, device=DEV)
    g_npad = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    nws = ft.align_workspace_size(T, k, E, BM)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=DEV)
    ft.align(d_ids, T, k, E, BM, g_counts, g_off, g_sorted, g_bexp, g_npad, ws)
    torch.cuda.synchronize()
    assert np.array_equal(g_counts.cpu().numpy(), counts)
    assert np.array_equal(g_off.cpu().numpy(), offsets)
    assert int(g_npad.item()) == npad
    assert np.array_equal(g_sorted.cpu().numpy(), sorted_ids)
    assert np.array_equal(g_bexp.cpu().numpy(), bexp)


# --------------------------------------------------------------- forward --
SMALL_CASES = [("c0", 16, "auto"), ("c0", 16, "decode"), ("c0", 16, "prefill"),
               ("c0", 5, "decode"), ("c0", 5, "prefill"), ("c0", 70, "prefill"), ("c0", 70, "decode"),
               ("c1", 1, "decode"), ("c1", 1, "prefill"), ("c1", 8, "decode"), ("c1", 8, "prefill"),
               ("c1", 17, "auto"), ("c3", 1, "decode"), ("c3", 1, "prefill"), ("c3", 8, "decode"),
               ("c3", 20, "prefill"), ("c1-w4a8", 1, "decode"), ("c1-w4a8", 8, "decode"),
               ("c1-w4a8", 8, "prefill"), ("c1-w4a8", 40, "prefill")]


@pytest.mark.parametrize("name,T,path", SMALL_CASES)
@pytest.mark.timeout(600)
def test_forward_parity_full(name, T, path):
    say(f"forward parity {name} T={T} path={path}")
    lay, dlay = layer_pair(name)
    x = synth.make_tokens(lay, T)
    y, ids, w = run_forward(dlay, x, path)
    ref = oracle.forward(lay, x)
    assert np.array_equal(ids, ref["ids"])
    assert np.abs(w - ref["w"]).max() <= 1e-5
    err = rel_fro(y, ref["y"])
    say(f"  rel_fro={err:.3e} max_abs={np.abs(y - ref['y']).max():.3e}")
    assert np.isfinite(y).all()
    assert err <= tol_for(name)


# Per-row bar at full size: every token's row of y against the grouped
# oracle, relative to that row's norm (a fault confined to some tiles shows
# up in the rows it touches even when the aggregate stays small).
ROW_BAR = 2.0


@pytest.mark.parametrize("name,T,nsample", [("c2", 4096, 48), ("c3", 8192, 40), ("c4", 16384, 24),
                                            ("c2-w4a8", 4096, 48), ("c2-bf16", 4096, 32),
                                            ("c0", 1 << 20, 32)])   # the largest batch the library takes
@pytest.mark.timeout(900)
def test_forward_parity_full_size_every_row(name, T, nsample):
    """Every output row at full size, in the launch configuration the
    benchmark times (packed weights), against the oracle's grouped mode in
    float32; that mode is itself held to the float64 per-token loop on a
    sample of tokens first."""
    say(f"forward parity full size {name} T={T}, every row, packed weights as the benchmark runs")
    lay, dlay = layer_pair(name, packed=True)
    x = synth.make_tokens(lay, T)
    y, ids, w = run_forward(dlay, x, "auto")
    g = oracle.forward_grouped(lay, x, dtype=np.float32)
    assert np.array_equal(ids, g["ids"])
    assert np.abs(w - g["w"]).max() <= 1e-5
    # the float32 grouped oracle against the float64 per-token loop
    tok = sample_tokens(T, nsample, seed=T)
    ref_tok = oracle.forward_tokens(lay, x, tok, s_h=g.get("s_h"))
    g_err = rel_fro(g["y"][tok], ref_tok)
    say(f"  grouped float32 oracle vs per-token float64 on {len(tok)} tokens: {g_err:.2e}")
    assert g_err <= 1e-4
    assert np.isfinite(y).all()
    ref = g["y"]
    err = rel_fro(y, ref)
    rows = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    worst = int(rows.argmax())
    say(f"  rel_fro={err:.3e} max_abs={np.abs(y - ref).max():.3e} worst row {rows[worst]:.3e} "
        f"(token {worst}, experts {ids[worst].tolist()})")
    assert err <= tol_for(name)
    assert rows.max() <= ROW_BAR * tol_for(name)


@pytest.mark.timeout(600)
def test_forward_is_deterministic():
    say("forward determinism c2 T=4096")
    lay, dlay = layer_pair("c2")
    x = synth.make_tokens(lay, 4096, stream=3)
    a = run_forward(dlay, x)[0]
    b = run_forward(dlay, x)[0]
    assert np.array_equal(a, b)


@pytest.mark.timeout(600)
def test_decode_and_prefill_paths_agree():
    say("decode vs prefill c1 T=8")
    lay, dlay = layer_pair("c1")
    x = synth.make_tokens(lay, 8, stream=5)
    a = run_forward(dlay, x, "decode")[0]
    b = run_forward(dlay, x, "prefill")[0]
    assert rel_fro(a, b) <= 1e-2


@pytest.mark.timeout(600)
def test_experts_forward_with_given_routing():
    """ftmoe_experts_forward on the oracle's routing equals the oracle."""
    say("experts_forward c0 T=16 with oracle routing")
    lay, dlay = layer_pair("c0")
    x = synth.make_tokens(lay, 16, stream=2)
    ref = oracle.forward(lay, x)
    T, k = 16, dlay.top_k
    ids = torch.from_numpy(ref["ids"]).to(DEV)
    w = torch.from_numpy(ref["w"].astype(np.float32)).to(DEV)
    ws = ft.alloc_workspace(dlay, T)
    y = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ft.experts_forward(dlay, to_dev_bf16(x), T, ids, w, None, ws, y)
    torch.cuda.synchronize()
    from gpu_util import bf16_dev_to_f64
    assert rel_fro(bf16_dev_to_f64(y), ref["y"]) <= 2e-2


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,T", [("c0", 300), ("c1", 200), ("c1-w4a8", 64), ("c3", 40), ("c2", 16300),
                                    ("c2-w4a8", 16300)])
def test_forward_equals_route_then_experts_forward_prefill(name, T):
    """On the prefill kernels, ftmoe_forward (whose router GEMM also writes the
    split or MXFP8 x of MXFP4 layers) equals ftmoe_route followed by
    ftmoe_experts_forward (which converts x with its own kernel) bit for
    bit: both conversions implement the same block rule.  (At 16300 tokens
    the router runs 128-token tiles, where a thread converts a whole
    32-block; at the smaller counts 64-token tiles, where two lanes share
    one.)"""
    say(f"forward == route + experts_forward, prefill kernels, {name} T={T}")
    lay, dlay = layer_pair(name)
    pl = dlay.with_path("prefill")
    x = synth.make_tokens(lay, T, stream=5)
    xd = to_dev_bf16(x)
    k = dlay.top_k
    ws = ft.alloc_workspace(pl, T)
    y1 = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ids1 = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w1 = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ft.forward(pl, xd, T, ws, y1, ids1, w1)
    ids2 = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w2 = torch.empty((T, k), dtype=torch.float32, device=DEV)
    sg = torch.empty((T,), dtype=torch.float32, device=DEV) if dlay.shared_inter else None
    ft.route(pl, xd, T, ws, ids2, w2, sg)
    y2 = torch.empty((T, dlay.hidden), dtype=torch.int16, device=DEV)
    ft.experts_forward(pl, xd, T, ids2, w2, sg, ws, y2)
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2) and torch.equal(w1, w2)
    assert torch.equal(y1, y2)


# ---------------------------------------------------------- FP8 quantiser --
@pytest.mark.timeout(300)
def test_fp8_quantiser_bit_exact():
    say("fp8 per-tensor quantiser")
    lay = synth.make_layer("c4")
    x = synth.make_tokens(lay, 2048)
    rng = np.random.default_rng(4)
    wide = synth.f32_to_bf16_bits((rng.standard_normal(40_003) * np.exp(rng.uniform(-12, 6, 40_003))).astype(np.float32))
    for arr in (x.reshape(-1), wide):
        n = arr.size
        xd = to_dev_bf16(arr)
        q = torch.empty(n, dtype=torch.uint8, device=DEV)
        s = torch.empty(1, dtype=torch.float32, device=DEV)
        ws = torch.empty(256, dtype=torch.uint8, device=DEV)
        ft.quantize_fp8_per_tensor(xd, n, q, s, ws)
        torch.cuda.synchronize()
        _, s_ref, codes = oracle.quant_act_per_tensor(oracle.bf16_to_f64(arr))
        assert float(s.item()) == s_ref
        assert np.array_equal(q.cpu().numpy(), codes)
