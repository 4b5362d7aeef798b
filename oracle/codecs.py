"""Exact decoders of the weight/scale codes, and the E4M3 encoder the forward
applies to activations.  TEST INFRASTRUCTURE ONLY (see package docstring).

- E2M1 (OCP MX v1.0, FP4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
  bit.  Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
- E8M0 (OCP MX v1.0 scale): value 2^(c - 127); code 255 is NaN.
- E4M3FN (OCP OFP8): bias 7, subnormals m/8 * 2^-6, max 448, NaN at 0x7F and
  0xFF, no infinities.
- MXFP4: blocks of 32 elements along K share one E8M0 scale.
- NVFP4: blocks of 16 elements along K share one E4M3 scale, and the whole
  matrix has one fp32 multiplier.
- Packing: element k of a row sits in byte k/2, low nibble for even k.
- BF16 experts: one bf16 (the top 16 bits of an fp32) per element, no scale.
"""
from __future__ import annotations

import numpy as np

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15) -> float64."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 codes -> float64 (2^(c-127), NaN for 255)."""
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    v = sign * np.where(e == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


# Finite non-negative E4M3 magnitudes and their codes, in code order (which is
# also magnitude order).
_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)
_E4M3_POS_VALS = e4m3_decode(_E4M3_POS_CODES)


def e4m3_encode_nearest(v32: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code to each fp32 value: ties go to the even code,
    magnitudes beyond 448 saturate to 448 (code 0x7E), sign is kept.

    Written as a plain nearest-neighbour search over the code table: for each
    value the two neighbouring representable magnitudes are compared by
    distance (exact in float64 for fp32 inputs)."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    hi = np.searchsorted(_E4M3_POS_VALS, a, side="left")  # first table value >= a
    hi = np.clip(hi, 0, len(_E4M3_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_hi = np.abs(_E4M3_POS_VALS[hi] - a)
    d_lo = np.abs(a - _E4M3_POS_VALS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_E4M3_POS_CODES[lo] % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= 448.0, 0x7E, code)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def _unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes (low nibble = even element)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


# Value of every code, for decoding whole matrices by table lookup (the same
# values as the decoders above, looked up instead of recomputed per element).
_E2M1_TABLE = e2m1_decode(np.arange(16))
_E8M0_TABLE = e8m0_decode(np.arange(256))
_E4M3_TABLE = e4m3_decode(np.arange(256))


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[n,k] = E2M1(code[n,k]) * 2^(S[n, k//32] - 127), float64."""
    el = _E2M1_TABLE[_unpack_nibbles(codes)]
    sc = _E8M0_TABLE[np.asarray(scales, np.uint8)]
    return (el.reshape(*el.shape[:-1], -1, 32) * sc[..., None]).reshape(el.shape)


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """W[n,k] = E2M1(code[n,k]) * E4M3(S[n, k//16]) * g (g a scalar, or [N, 1]
    per row), float64."""
    el = _E2M1_TABLE[_unpack_nibbles(codes)]
    sc = _E4M3_TABLE[np.asarray(scales, np.uint8)] * np.asarray(g, np.float64)
    return (el.reshape(*el.shape[:-1], -1, 16) * sc[..., None]).reshape(el.shape)


def dequant_fp8(codes: np.ndarray, s) -> np.ndarray:
    """W[n,k] = E4M3(code[n,k]) * s (s a scalar, or [N, 1] per row), float64."""
    return _E4M3_TABLE[np.asarray(codes, np.uint8)] * np.asarray(s, np.float64)


def dequant_bf16(bits: np.ndarray) -> np.ndarray:
    """W[n,k] = the bf16 value of bits[n,k], float64 (exact: a bf16 is the
    upper half of an fp32)."""
    u = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def dequant(qw, e: int) -> np.ndarray:
    """Dequantise expert e of a stacked packed matrix (duck-typed: needs
    fmt, codes, block_scales, tensor_scales).  NVFP4 and FP8 multipliers are
    one per matrix ([E]) or one per matrix row ([E, N]: row-wise scaling,
    and per-part scaling of a fused projection as runs of equal rows)."""
    if qw.fmt == "mxfp4":
        return dequant_mxfp4(qw.codes[e], qw.block_scales[e])
    if qw.fmt == "bf16":
        return dequant_bf16(qw.codes[e])
    ts = np.asarray(qw.tensor_scales[e], np.float64)
    g = ts[:, None] if ts.ndim == 1 else ts   # a row's multiplier broadcasts along K
    if qw.fmt == "nvfp4":
        return dequant_nvfp4(qw.codes[e], qw.block_scales[e], g)
    if qw.fmt == "fp8":
        return dequant_fp8(qw.codes[e], g)
    raise ValueError(f"unknown weight format {qw.fmt!r}")
