"""Routed MoE layer forward, written out as its plain definition.
TEST INFRASTRUCTURE ONLY (see package docstring).

Inputs are duck-typed (no import of the generator): a layer object with
``router_w [E,H] fp32``, ``router_b [E] or None``, ``gate_up`` and ``down``
stacked packed matrices (fields fmt, codes, block_scales, tensor_scales, n, k),
optional ``shared_gate_up``/``shared_down``/``shared_gate_w``, and ``cfg``
with ``top_k``, ``act`` ("bf16" | "fp8" | "mxfp8") and optionally
``bias_mode`` ("logits", the default, or "select").  Hidden states are bf16 bit
patterns (uint16).

Arithmetic is float64 throughout, except where a floating-point value decides
an integer code (the per-tensor E4M3 activation quantiser): there the scale and
the quotient are formed in fp32, the precision the GPU kernels use, so both
sides take the same decision on the same fp32 number.

The forward, for token t (FreeToken README: a Mixture-of-Experts serving
engine over MXFP4/NVFP4/FP8 experts; the layer arithmetic is the standard
routed SwiGLU MoE):
  1. l[t,e]  = x_t . W_r[e] + b[e]
  2. ids_t   = the k largest logits, descending, ties to the lower index
  3. w_t     = softmax over the k selected logits
     (selection-only bias, bias_mode "select": l = x_t . W_r[e] in 1 and 3,
      and step 2 ranks l + b instead)
  4. sg_t    = sigmoid(x_t . w_sg)                          (shared expert)
  5. x^      = x, or E4M3 per-tensor quantise-dequantise of x  (FP8 layers),
               or MXFP8 of each row of x                      (MXFP8 layers)
  6. a       = W_gu[e] x^_t ; h = silu(a[:I]) * a[I:]
  7. h^      = h, or E4M3 per-tensor over all T*k rows of h     (FP8 layers),
               or MXFP8 of each row of h                      (MXFP8 layers)
  8. y_t     = sum_j w_tj W_d[e_j] h^_tj   (ascending j)
  9. y_t    += sg_t * W_ds hs^_t,  hs_t = silu(W_gs x^_t)[:Is] * ...[Is:]
               (shared expert; hs^ = hs, or its MXFP8 form in MXFP8 layers)
"""
from __future__ import annotations

import numpy as np

from .codecs import dequant, e4m3_decode, e4m3_encode_nearest


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- routing --


def _bias_select_only(lay) -> bool:
    return getattr(lay.cfg, "bias_mode", "logits") == "select"


def router_logits(lay, xf: np.ndarray) -> np.ndarray:
    """Step 1: l = x W_r^T + b  (float64); a selection-only bias is left to
    ``selection_scores``."""
    lg = xf @ np.asarray(lay.router_w, np.float64).T
    if getattr(lay, "router_b", None) is not None and not _bias_select_only(lay):
        lg = lg + np.asarray(lay.router_b, np.float64)
    return lg


def selection_scores(lay, lg: np.ndarray) -> np.ndarray:
    """The values step 2 ranks: the logits, or logits + b when the bias takes
    part in the selection only."""
    if getattr(lay, "router_b", None) is not None and _bias_select_only(lay):
        return lg + np.asarray(lay.router_b, np.float64)
    return lg


def route(lay, xf: np.ndarray):
    """Steps 1-3: (logits, selected ids, weights)."""
    lg = router_logits(lay, xf)
    ids = select_topk(selection_scores(lay, lg), lay.cfg.top_k)
    return lg, ids, topk_softmax(lg, ids)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Step 2: per row, indices of the k largest values in descending value
    order, equal values ordered by ascending index (a full stable sort)."""
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        ids[t] = order[:k]
    return ids


def topk_softmax(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Step 3: softmax over the selected logits (renormalised weights)."""
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    return ex / ex.sum(axis=1, keepdims=True)


def shared_gate(lay, xf: np.ndarray) -> np.ndarray:
    """Step 4: sigmoid(x . w_sg)."""
    g = xf @ np.asarray(lay.shared_gate_w, np.float64)
    return 1.0 / (1.0 + np.exp(-g))


# ---------------------------------------------------------------- align ----


def align_max_padded(T: int, k: int, E: int, block_m: int) -> int:
    """Capacity of the padded, expert-sorted row list: every non-empty expert
    pads its rows up to a multiple of block_m, and at most min(E, T*k)
    experts are non-empty.  Rounded up to whole blocks."""
    p = T * k + min(E, T * k) * (block_m - 1)
    return -(-p // block_m) * block_m


def align(ids: np.ndarray, E: int, block_m: int):
    """Token-to-expert alignment (count, prefix-sum, padded scatter).

    Returns counts[E], offsets[E+1], sorted_ids[P_max], block_expert[P_max/BM],
    num_padded.  Row i = t*k + j of the flat routing table goes to expert
    ids[t, j]; within an expert rows keep ascending i; each expert's segment
    is padded with the sentinel T*k up to a multiple of block_m; experts with
    no rows get no blocks.  Entries past num_padded hold the sentinel (rows)
    and -1 (blocks)."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    n = flat.size
    counts = np.zeros(E, np.int32)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int32)
    for e in range(E):
        padded = -(-int(counts[e]) // block_m) * block_m
        offsets[e + 1] = offsets[e] + padded
    p_max = align_max_padded(T, k, E, block_m)
    sorted_ids = np.full(p_max, n, np.int32)
    block_expert = np.full(p_max // block_m, -1, np.int32)
    fill = offsets[:-1].copy()
    for i in range(n):
        e = flat[i]
        sorted_ids[fill[e]] = i
        fill[e] += 1
    for e in range(E):
        block_expert[offsets[e] // block_m: offsets[e + 1] // block_m] = e
    return counts, offsets, sorted_ids, block_expert, int(offsets[E])


# ------------------------------------------------------- activation quant --


def quant_act_per_tensor(v: np.ndarray):
    """E4M3 per-tensor quantise-dequantise: s = amax/448 (1 if amax is 0),
    code = nearest E4M3 of v/s.  Scale and quotient are fp32.  Returns
    (dequantised float64 values, s as float, codes)."""
    v32 = np.asarray(v, np.float64).astype(np.float32)
    amax = np.float32(np.abs(v32).max()) if v32.size else np.float32(0)
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    codes = e4m3_encode_nearest(v32 / s)
    return e4m3_decode(codes) * np.float64(s), float(s), codes


def quant_act_mxfp8(v: np.ndarray):
    """MXFP8 quantise-dequantise along the last axis (OCP Microscaling v1.0:
    E4M3 elements, one E8M0 scale per block of 32 consecutive elements).

    The conversion rule of the MX specification: a block's shared exponent is
    X = floor(log2(amax)) - 8, 8 being the largest exponent of E4M3, so the
    block maximum lands in [256, 512) and saturates to 448 above 448.  X is
    kept inside E8M0's range (at least -127, which is also taken for an
    all-zero block).  Each element becomes the nearest E4M3 (ties to even,
    saturating) of v / 2^X.  The block maximum and the quotient are fp32, the
    precision the GPU kernels decide in; v / 2^X is exact.

    Returns (dequantised float64 values, element codes uint8 of v's shape,
    scale codes uint8 of shape [..., n / 32] holding X + 127)."""
    v32 = np.asarray(v, np.float64).astype(np.float32)
    n = v32.shape[-1]
    assert n % 32 == 0, "MXFP8 blocks need a multiple of 32 elements"
    blk = v32.reshape(*v32.shape[:-1], n // 32, 32).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex with m in [0.5, 1)
    X = np.where(amax > 0, ex - 1 - 8, -127)
    X = np.maximum(X, -127)
    q = blk * np.ldexp(1.0, -X)[..., None]       # exact power-of-two scaling
    codes = e4m3_encode_nearest(q.astype(np.float32))
    deq = e4m3_decode(codes) * np.ldexp(1.0, X)[..., None]
    return (deq.reshape(v32.shape), codes.reshape(v32.shape),
            (X + 127).astype(np.uint8))


# ---------------------------------------------------------------- experts --


def _silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_expert(w_gu: np.ndarray, w_d: np.ndarray, xr: np.ndarray):
    """SwiGLU expert on rows xr [..., K]: gate rows [0,I), up rows [I,2I).
    Returns (h, o) with h = silu(gate) * up and o = W_d h."""
    I = w_gu.shape[0] // 2
    a = xr @ w_gu.T
    h = _silu(a[..., :I]) * a[..., I:]
    return h, h @ w_d.T


def _routing(lay, x_bits):
    xf = bf16_to_f64(x_bits)
    lg, ids, w = route(lay, xf)
    sg = shared_gate(lay, xf) if getattr(lay, "shared_gate_w", None) is not None else None
    return xf, lg, ids, w, sg


def _is_fp8_act(lay) -> bool:
    return getattr(lay.cfg, "act", "bf16") == "fp8"


def _is_mxfp8_act(lay) -> bool:
    return getattr(lay.cfg, "act", "bf16") == "mxfp8"


def _quant_x(lay, xf):
    """x^ of step 5."""
    if _is_fp8_act(lay):
        return quant_act_per_tensor(xf)[0]
    if _is_mxfp8_act(lay):
        return quant_act_mxfp8(xf)[0]
    return xf


def _quant_rows_mx(lay, h):
    """h^ of MXFP8 layers: every row of h (last axis) on its own."""
    return quant_act_mxfp8(h)[0] if _is_mxfp8_act(lay) else h


def _shared_out(lay, wgs, wds, xr):
    """Shared expert output W_ds hs^ for rows xr (step 9)."""
    hs = swiglu_expert(wgs, wds, xr)[0]
    return _quant_rows_mx(lay, hs) @ wds.T


def forward(lay, x_bits: np.ndarray) -> dict:
    """Per-token mode: the literal loop over tokens and their k experts.
    FP8-activation layers need the amax of h over every token, so this mode
    first evaluates all h, then quantises, then runs the down projections."""
    xf, lg, ids, w, sg = _routing(lay, x_bits)
    T, H = xf.shape
    k = lay.cfg.top_k
    xq = _quant_x(lay, xf)
    cache = {}

    def W(qw, e):
        key = (id(qw), e)
        if key not in cache:
            cache[key] = dequant(qw, e)
        return cache[key]

    I = lay.gate_up.n // 2
    h = np.zeros((T, k, I))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            h[t, j] = swiglu_expert(W(lay.gate_up, e), W(lay.down, e), xq[t])[0]
    if _is_fp8_act(lay):
        h = quant_act_per_tensor(h)[0].reshape(h.shape)
    h = _quant_rows_mx(lay, h)
    y = np.zeros((T, H))
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = int(ids[t, j])
            acc = acc + w[t, j] * (W(lay.down, e) @ h[t, j])
        y[t] = acc
    if sg is not None:
        wgs, wds = dequant(lay.shared_gate_up, 0), dequant(lay.shared_down, 0)
        for t in range(T):
            y[t] = y[t] + sg[t] * _shared_out(lay, wgs, wds, xq[t])
    return dict(y=y, ids=ids, w=w, logits=lg, sgate=sg)


def forward_grouped(lay, x_bits: np.ndarray, tokens=None, dtype=np.float64) -> dict:
    """Grouped mode: the same arithmetic with one matmul per expert over the
    rows routed to it.  Evaluates h for every token (the FP8 per-tensor scale
    of h needs all of them) but only returns y for ``tokens`` (all if None).
    ``dtype`` may be float32 to fit full-size layers in memory and time; the
    float64 default is the reference."""
    xf, lg, ids, w, sg = _routing(lay, x_bits)
    T, H = xf.shape
    k = lay.cfg.top_k
    E = lay.router_w.shape[0]
    fp8 = _is_fp8_act(lay)
    xq = _quant_x(lay, xf)
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    flat = ids.reshape(-1)
    I = lay.gate_up.n // 2
    h_amax = 0.0
    # Pass 1: h for the rows we need (all rows when the h scale is global).
    need = np.zeros(T, bool)
    need[sel] = True
    h_rows = {}
    for e in range(E):
        rows = np.flatnonzero(flat == e)
        if rows.size == 0:
            continue
        if not fp8:
            rows = rows[need[rows // k]]
            if rows.size == 0:
                continue
        wgu = dequant(lay.gate_up, e).astype(dtype)
        a = xq[rows // k].astype(dtype) @ wgu.T
        g, u = a[:, :I].astype(np.float64), a[:, I:].astype(np.float64)
        h = _quant_rows_mx(lay, _silu(g) * u)
        if fp8:
            h_amax = max(h_amax, float(np.abs(h.astype(np.float32)).max()))
            keep = need[rows // k]
            rows, h = rows[keep], h[keep]
        h_rows[e] = (rows, h)
    if fp8:
        amax = np.float32(h_amax)
        s_h = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    y = np.zeros((T, H))
    o = np.zeros((T * k, H))
    for e, (rows, h) in h_rows.items():
        if fp8:
            h = e4m3_decode(e4m3_encode_nearest(h.astype(np.float32) / s_h)) * np.float64(s_h)
        wd = dequant(lay.down, e).astype(dtype)
        o[rows] = (h.astype(dtype) @ wd.T).astype(np.float64)
    o = o.reshape(T, k, H)
    for j in range(k):
        y[sel] += w[sel, j:j + 1] * o[sel, j]
    if sg is not None:
        wgs = dequant(lay.shared_gate_up, 0).astype(dtype)
        wds = dequant(lay.shared_down, 0).astype(dtype)
        Is = wgs.shape[0] // 2
        a = (xq[sel].astype(dtype) @ wgs.T).astype(np.float64)
        hs = _quant_rows_mx(lay, _silu(a[:, :Is]) * a[:, Is:])
        y[sel] += sg[sel, None] * (hs.astype(dtype) @ wds.T).astype(np.float64)
    out = dict(y=y[sel], ids=ids, w=w, logits=lg, sgate=sg)
    if fp8:
        out["s_h"] = float(s_h)
    return out


def forward_tokens(lay, x_bits: np.ndarray, tokens, s_h=None) -> np.ndarray:
    """y for a sample of tokens by the per-token loop.  For FP8-activation
    layers the h scale is a whole-batch quantity: pass the oracle's own s_h
    from ``forward_grouped`` over the full batch."""
    xf, lg, ids, w, sg = _routing(lay, x_bits)
    fp8 = _is_fp8_act(lay)
    xq = _quant_x(lay, xf)
    k = lay.cfg.top_k
    out = np.zeros((len(tokens), xf.shape[1]))
    cache = {}

    def W(qw, e):
        key = (id(qw), e)
        if key not in cache:
            cache[key] = dequant(qw, e)
        return cache[key]

    for r, t in enumerate(tokens):
        acc = np.zeros(xf.shape[1])
        for j in range(k):
            e = int(ids[t, j])
            wgu, wd = W(lay.gate_up, e), W(lay.down, e)
            h = swiglu_expert(wgu, wd, xq[t])[0]
            if fp8:
                s = np.float32(s_h)
                h = e4m3_decode(e4m3_encode_nearest(h.astype(np.float32) / s)) * np.float64(s)
            h = _quant_rows_mx(lay, h)
            acc = acc + w[t, j] * (wd @ h)
        if sg is not None:
            acc = acc + sg[t] * _shared_out(lay, W(lay.shared_gate_up, 0), W(lay.shared_down, 0), xq[t])
        out[r] = acc
    return out


# ----------------------------------------------- independent formulations --


def dense_swiglu(w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, x: np.ndarray, qh=None):
    """A dense SwiGLU MLP with separate gate/up matrices:
    W_down q(silu(W_gate x) * (W_up x)), row-wise over x; q is the identity
    unless given."""
    g = x @ w_gate.T
    u = x @ w_up.T
    h = g / (1.0 + np.exp(-g)) * u
    return (h if qh is None else qh(h)) @ w_down.T


def forward_all_experts_masked(lay, x_bits: np.ndarray) -> np.ndarray:
    """Brute force for tiny layers: every expert runs on every token and the
    results are mixed by a dense [T, E] matrix that is zero except on the
    k selected experts, where it holds the renormalised weights.
    For bf16 and MXFP8 activations (whose quantisation acts on each row
    alone); not for per-tensor FP8, whose h scale spans the routed rows."""
    assert not _is_fp8_act(lay)
    xf = bf16_to_f64(x_bits)
    mx = _is_mxfp8_act(lay)
    qh = (lambda h: quant_act_mxfp8(h)[0]) if mx else None
    lg = router_logits(lay, xf)
    T, E = lg.shape
    k = lay.cfg.top_k
    order = np.argsort(-selection_scores(lay, lg), axis=1, kind="stable")
    M = np.zeros((T, E))
    for t in range(T):
        top = order[t, :k]
        p = np.exp(lg[t, top] - lg[t, top].max())
        M[t, top] = p / p.sum()
    y = np.zeros((T, xf.shape[1]))
    I = lay.gate_up.n // 2
    xin = quant_act_mxfp8(xf)[0] if mx else xf
    for e in range(E):
        wgu = dequant(lay.gate_up, e)
        y += M[:, e:e + 1] * dense_swiglu(wgu[:I], wgu[I:], dequant(lay.down, e), xin, qh)
    if getattr(lay, "shared_gate_w", None) is not None:
        wgs = dequant(lay.shared_gate_up, 0)
        Is = wgs.shape[0] // 2
        sg = 1.0 / (1.0 + np.exp(-(xf @ np.asarray(lay.shared_gate_w, np.float64))))
        y += sg[:, None] * dense_swiglu(wgs[:Is], wgs[Is:], dequant(lay.shared_down, 0), xin, qh)
    return y
