"""Crafted layers and token batches for the edges of the code tables.

Input generation only: these functions build packed codes, block scales and
bf16 hidden states directly (instead of quantising random fp32 weights), so
that every code of a format occurs and every one of them matters to the
output.  They compute no part of the layer forward.

- ``mx_e8m0``: MXFP4 gate_up whose rows carry every E8M0 scale code 0..254.
  Row r of an expert's gate_up has one non-zero 32-block, scaled by code
  c(r); the hidden state's 32-block k holds values of magnitude [1, 2) times
  2^(123 - 2k) (clipped to the bf16 normal range), and a row with code c
  reads block c // 2, so that every row's dot product is of order one
  whatever its code (rows where the clipping leaves a larger product keep
  fewer non-zero elements, each of magnitude 0.5).
- ``nv_e4m3``: NVFP4 gate_up whose 16-blocks carry every finite non-negative
  E4M3 scale code 0..126 (zero, the subnormals 1..7 and the largest, 0x7E);
  the block scale exponent depends on the column block only (its mantissa is
  random per row), and the hidden state's 16-block carries the reciprocal
  size, so that every block contributes alike.
- ``fp8_all``: FP8 gate_up using all 254 finite E4M3 codes (both zeros and
  the subnormals included): a row's codes share one exponent field (random
  sign and mantissa) and its per-row multiplier undoes that exponent, so that
  every row's output is of order one.
- ``crafted_tokens(..., wide=True)``: hidden states whose elements are
  N(0, 1) times 2^u, u uniform in [-16, 0] per element: about 2^16 of
  dynamic range inside every 32-block (run through the ``WIDE`` layers,
  which follow the generator's recipe).

Every batch is redrawn row by row until its top-k logits are at least the
layer's gap apart (as ``make_tokens`` does), so that routing has one answer.
"""
from __future__ import annotations

import math

import numpy as np

from .layers import (Layer, LayerConfig, QWeight, _gap_ok, _make_qweight, _normal, _pack_nibbles, f32_to_bf16_bits,
                     make_layer)

CRAFTED = {
    # name: (hidden, experts, top_k, inter, fmt, act, shared_inter)
    "mx_e8m0": (4096, 4, 2, 128, "mxfp4", "bf16", 0),
    "mx_e8m0_a8": (4096, 4, 2, 128, "mxfp4", "mxfp8", 0),
    "nv_e4m3": (2048, 4, 2, 256, "nvfp4", "bf16", 128),
    "fp8_all": (512, 4, 2, 256, "fp8", "bf16", 0),
    "fp8_all_a8": (512, 4, 2, 256, "fp8", "fp8", 0),
}

# layers of the generator's own recipe that the wide-range batches run through
WIDE = {
    "wide_mx": (512, 8, 2, 256, "mxfp4", "bf16", 0),
    "wide_mx_a8": (512, 8, 2, 256, "mxfp4", "mxfp8", 0),
    "wide_nv": (512, 8, 2, 256, "nvfp4", "bf16", 128),
    "wide_fp8_a8": (512, 8, 2, 256, "fp8", "fp8", 0),
}

E4M3_NAN = 0x7F


def _rng(seed, *tag):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tag])))


def _cfg(name, shape, seed):
    H, E, k, I, fmt, act, Is = shape
    return LayerConfig(name, (16,), H, E, k, I, fmt, act=act, shared_inter=Is, seed=seed)


# ------------------------------------------------------------- MXFP4 ------
def _mx_block_exponent(H):
    """Size exponent of the hidden state's 32-blocks: 123 - 2 kb, kept inside
    the bf16 normal range for magnitudes in [1, 2)."""
    kb = np.arange(H // 32)
    return np.clip(123 - 2 * kb, -126, 122)


def _mx_e8m0_gate_up(rng, E, I, H):
    n = 2 * I
    assert n >= 255 and H // 32 >= 128
    nb = H // 32
    codes = np.zeros((E, n, H // 2), np.uint8)
    scales = np.full((E, n, nb), 127, np.uint8)
    ex = _mx_block_exponent(H)
    for e in range(E):
        row_code = np.concatenate([np.arange(255), rng.integers(0, 255, n - 255)])
        rng.shuffle(row_code)
        for r in range(n):
            c = int(row_code[r])
            kb = c // 2
            p = c - 127 + int(ex[kb])   # exponent of the block's products
            el = np.zeros(H, np.uint8)
            if p <= -3:
                el[32 * kb:32 * kb + 32] = rng.integers(0, 16, 32)
            else:   # magnitude 0.5 (codes 1, 9) on 4^(1 - p) elements, at most 32
                nz = min(32, 4 ** max(0, 1 - p))
                el[32 * kb:32 * kb + nz] = 1 | (rng.integers(0, 2, nz) << 3)
            codes[e, r] = _pack_nibbles(el)
            scales[e, r, kb] = c
    return QWeight("mxfp4", E, n, H, codes, scales, None)


def _mx_router(rng, E, H):
    ex = np.repeat(_mx_block_exponent(H), 32)
    w = rng.standard_normal((E, H)).astype(np.float64) / 8.0 * np.ldexp(1.0, -ex)
    w[:, np.abs(ex) > 100] = 0.0   # keeps the router weights inside the fp32 normal range
    return w.astype(np.float32)


# ------------------------------------------------------------- NVFP4 ------
def _nv_block_codes(H):
    """E4M3 scale code of each 16-block column: 0..126, then repeating."""
    return np.arange(H // 16) % 127


def _e4m3_exponent_size(code):
    """2^(exponent field - 7), the size of an E4M3 value of that code
    (subnormals: 2^-7)."""
    e = (np.asarray(code) >> 3) & 0xF
    return np.where(e == 0, 2.0 ** -7, np.ldexp(1.0, e - 7))


def _nv_gate_up(rng, E, I, H):
    n = 2 * I
    base = _nv_block_codes(H)
    codes = rng.integers(0, 256, (E, n, H // 2), dtype=np.uint8)
    # same exponent field per column block, random mantissa per row
    sc = (base[None, None, :] & 0x78) | rng.integers(0, 8, (E, n, H // 16))
    sc = np.where(sc == E4M3_NAN, base[None, None, :], sc).astype(np.uint8)
    # every code 0..126 occurs at least once exactly
    sc[:, 0, :] = base
    ts = np.full((E,), 1.0 / 16.0, np.float32)
    return QWeight("nvfp4", E, n, H, codes, sc, ts)


def _nv_sizes(H):
    return np.repeat(_e4m3_exponent_size(_nv_block_codes(H)), 16)


# --------------------------------------------------------------- FP8 ------
def _fp8_gate_up(rng, E, I, H):
    n = 2 * I
    i = np.arange(I)
    expo = np.concatenate([i % 16, (i // 16) % 16])   # gate rows, then up rows
    mant = rng.integers(0, 8, (E, n, H))
    mant = np.where(expo[None, :, None] == 15, np.minimum(mant, 6), mant)
    sign = rng.integers(0, 2, (E, n, H))
    codes = ((sign << 7) | (expo[None, :, None] << 3) | mant).astype(np.uint8)
    # all 254 finite codes at least once: the first 16 columns of each row of
    # expert 0 walk its exponent band's codes
    for r in range(n):
        band = [(s << 7) | (expo[r] << 3) | m for s in (0, 1) for m in range(8)
                if not (expo[r] == 15 and m == 7)]
        codes[0, r, :len(band)] = band
    size = _e4m3_exponent_size(expo << 3)
    rs = np.broadcast_to((1.0 / size / 16.0).astype(np.float32), (E, n)).copy()
    return QWeight("fp8", E, n, H, codes, None, rs)


# ------------------------------------------------------------- layers -----
def crafted_layer(name: str, seed: int = 21) -> Layer:
    """One of the ``CRAFTED`` layers (gate_up crafted, down and shared
    expert by the generator's recipe) or a ``WIDE`` layer (all by the
    generator's recipe)."""
    if name in WIDE:
        return make_layer(_cfg(name, WIDE[name], seed), cache=False)
    H, E, k, I, fmt, act, Is = shape = CRAFTED[name]
    cfg = _cfg(name, shape, seed)
    rng = _rng(seed, 7)
    root = np.random.SeedSequence(seed)
    s_router, s_d, s_sgu, s_sd, s_sg = root.spawn(5)
    if fmt == "mxfp4":
        gate_up = _mx_e8m0_gate_up(rng, E, I, H)
        router_w = _mx_router(rng, E, H)
    elif fmt == "nvfp4":
        gate_up = _nv_gate_up(rng, E, I, H)
        router_w = (_normal(s_router, (E, H), 1.0 / math.sqrt(H)) * _nv_sizes(H)).astype(np.float32)
    else:
        gate_up = _fp8_gate_up(rng, E, I, H)
        router_w = _normal(s_router, (E, H), 1.0 / math.sqrt(H))
    down = _make_qweight(fmt, s_d.spawn(E), H, I, 1.0 / math.sqrt(I))
    lay = Layer(cfg, router_w, None, gate_up, down)
    if Is:
        lay.shared_gate_up = _make_qweight(fmt, s_sgu.spawn(1), 2 * Is, H, 1.0 / math.sqrt(H), gate_up=True)
        lay.shared_down = _make_qweight(fmt, s_sd.spawn(1), H, Is, 1.0 / math.sqrt(Is))
        w = _normal(s_sg, (H,), 1.0 / math.sqrt(H))
        lay.shared_gate_w = (w * _nv_sizes(H)).astype(np.float32) if fmt == "nvfp4" else w
    return lay


def _size_of_columns(lay: Layer) -> np.ndarray:
    """Per hidden column, the size the crafted layer expects of x there."""
    name, H = lay.cfg.name, lay.cfg.hidden
    if name.startswith("mx_e8m0"):
        return np.ldexp(1.0, np.repeat(_mx_block_exponent(H), 32))
    if name.startswith("nv_e4m3"):
        return 1.0 / _nv_sizes(H)
    return np.ones(H)


def _draw(rng, T, H, size, wide, unit):
    if unit:   # magnitudes in [1, 2), random signs (stays normal at the smallest sizes)
        v = rng.uniform(1.0, 1.99, (T, H)) * np.where(rng.integers(0, 2, (T, H)) == 1, -1.0, 1.0)
    else:
        v = np.clip(rng.standard_normal((T, H)), -1.99, 1.99)
    if wide:
        v = v * np.exp2(rng.uniform(-16.0, 0.0, (T, H)))
    return f32_to_bf16_bits((v * size[None, :]).astype(np.float32))


def crafted_tokens(lay: Layer, T: int, stream: int = 0, wide: bool = False, max_tries: int = 64) -> np.ndarray:
    """bf16 hidden states [T, H] (uint16 bits) for a crafted or wide layer:
    each column at the size its layer expects (1 for the generator's
    layers), times 2^u per element when ``wide``; rows redrawn until the
    top-k logits are ``gap`` apart."""
    H = lay.cfg.hidden
    rng = _rng(lay.cfg.seed, 3000 + stream)
    size = _size_of_columns(lay)
    unit = lay.cfg.name.startswith("mx_e8m0")
    x = _draw(rng, T, H, size, wide, unit)
    for _ in range(max_tries):
        bad = np.flatnonzero(~_gap_ok(x, lay, lay.cfg.gap))
        if bad.size == 0:
            return x
        x[bad] = _draw(rng, bad.size, H, size, wide, unit)
    raise RuntimeError(f"could not draw {T} tokens with a {lay.cfg.gap} top-k gap")
