"""Pins for the oracle's code tables and the generator's encoders.

Each decoder is compared, code by code, with (a) the bit-field definition of
its format (sign / exponent / mantissa with the format's bias) and (b) torch's
float8 dtypes, an implementation that shares nothing with this repository.
Encoders are compared with a brute-force nearest-value search and with torch's
fp32 -> float8 conversion."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import codecs


def _bitfield_minifloat(code, ebits, mbits, bias):
    """Value of a sign/exponent/mantissa code with subnormals (no inf/NaN)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = m / (1 << mbits) * 2.0 ** (1 - bias)
    else:
        v = (1 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -v if s else v


def test_e2m1_all_codes_match_bitfield():
    got = oracle.e2m1_decode(np.arange(16))
    want = [_bitfield_minifloat(c, 2, 1, 1) for c in range(16)]
    assert np.array_equal(got, np.array(want))
    assert np.array_equal(np.abs(got[:8]), [0, 0.5, 1, 1.5, 2, 3, 4, 6])
    assert np.signbit(got[8])  # code 8 is -0


def test_e8m0_all_codes_match_torch():
    got = oracle.e8m0_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    # torch widens through fp32, which cannot hold 2^-127 exactly as a normal
    # number but can as a subnormal; compare all finite codes exactly.
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_e4m3_all_codes_match_torch_and_bitfield():
    got = oracle.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    for c in range(256):
        if c & 0x7F != 0x7F:
            assert got[c] == _bitfield_minifloat(c, 4, 3, 7)
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def _all_bf16_finite_f32():
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << np.uint32(16)).view(np.float32)
    return f[np.isfinite(f)]


def test_oracle_e4m3_encoder_matches_torch_on_all_bf16():
    v = _all_bf16_finite_f32()
    v = v[np.abs(v) < 1e30]
    got = oracle.e4m3_encode_nearest(v)
    clamped = torch.from_numpy(np.clip(v, -448.0, 448.0))
    ref = clamped.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch maps -0 and +0 and tiny negatives to signed zero codes as we do.
    assert np.array_equal(got, ref)


def test_oracle_e4m3_encoder_random_fp32_matches_torch():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(200_000) * rng.choice([1e-3, 1, 100, 1000], 200_000)).astype(np.float32)
    got = oracle.e4m3_encode_nearest(v)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_oracle_e4m3_encoder_ties_go_to_even_code():
    vals = codecs._E4M3_POS_VALS
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    got = oracle.e4m3_encode_nearest(mids)
    lo = np.arange(len(mids))
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got.astype(np.int64), want)


def _brute_nearest(v, table, codes):
    """argmin |v - table|, ties to the even code; table covers magnitudes."""
    out = []
    for x in v:
        d = np.abs(np.abs(x) - table)
        best = np.flatnonzero(d == d.min())
        c = codes[best]
        c = c[c % 2 == 0][0] if len(c) > 1 else c[0]
        out.append(c | (8 if np.signbit(x) else 0))
    return np.array(out)


def test_generator_e2m1_encoder_matches_brute_force():
    table = oracle.E2M1_VALUES
    grid = np.concatenate([np.arange(-8, 8.0001, 0.03125), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 7.99, -0.0]])
    grid = grid.astype(np.float32)
    got = synth.e2m1_encode(grid)
    sat = np.clip(grid, -6, 6)
    want = _brute_nearest(sat, table, np.arange(8))
    assert np.array_equal(got.astype(np.int64), want)


def test_generator_e4m3_encoder_matches_torch():
    v = _all_bf16_finite_f32()
    v = v[np.abs(v) < 1e30]
    got = synth.e4m3_encode(v)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_mxfp4_quant_roundtrip_bound_and_scale_rule():
    """Generator packing read back by the oracle's decoder: every element is
    within half a quantum (E2M1 spacing times the block scale) or saturated,
    and the scale is 2^(floor(log2 amax) - 2)."""
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((8, 256)) * 0.05).astype(np.float32)
    codes, scales = synth.quantize_mxfp4(w)
    wq = oracle.dequant_mxfp4(codes, scales)
    amax = np.abs(w.reshape(8, 8, 32)).max(-1)
    assert np.array_equal(scales.astype(np.int64) - 127, np.floor(np.log2(amax)).astype(np.int64) - 2)
    sc = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    r = np.abs(w) / sc
    # E2M1 spacing: 0.5 below 2, 1 in [2,4), 2 in [4,6]
    half_q = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0)) * sc
    err = np.abs(wq - w)
    ok = (err <= half_q + 1e-12) | ((np.abs(wq) == 6 * sc) & (r > 6))
    assert ok.all()


def test_nvfp4_quant_roundtrip_bound():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((16, 128)) * 0.03).astype(np.float32)
    codes, sb, g = synth.quantize_nvfp4(w)
    wq = oracle.dequant_nvfp4(codes, sb, g)
    assert np.isclose(g, np.abs(w).max() / (6 * 448), rtol=1e-6)
    blk = np.repeat(oracle.e4m3_decode(sb) * g, 16, axis=1)
    r = np.abs(w) / blk
    half_q = np.where(r < 2, 0.25, np.where(r < 4, 0.5, 1.0)) * blk
    # block scale rounding can push amax/scale slightly past 6 (saturates)
    err = np.abs(wq - w)
    assert ((err <= half_q * (1 + 1e-6)) | (r > 6)).all()
    # largest E2M1 step is 2 (between 4 and 6): at most 1/6 of a block amax
    assert np.max(np.abs(wq - w)) / np.abs(w).max() <= 1 / 6 + 1e-3


def test_fp8_weight_roundtrip():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((32, 64)) * 0.02).astype(np.float32)
    codes, s = synth.quantize_fp8(w)
    wq = oracle.dequant_fp8(codes, s)
    assert np.isclose(np.abs(wq).max(), 448 * s)
    assert np.max(np.abs(wq - w) / np.maximum(np.abs(w), 2 ** -6 * s)) <= 2 ** -4 + 1e-9


def test_nibble_order_low_is_even_element():
    """Byte 0x4A holds code 0xA (= -1.0) for element 0 and 0x4 (= 2.0) for
    element 1; scale code 127 is 1.0."""
    codes = np.full((1, 16), 0x4A, np.uint8)
    scales = np.array([[127]], np.uint8)
    w = oracle.dequant_mxfp4(codes, scales)
    assert w[0, 0] == -1.0 and w[0, 1] == 2.0


class _QW:
    def __init__(self, fmt, codes, bs, ts):
        self.fmt, self.codes, self.block_scales, self.tensor_scales = fmt, codes, bs, ts


def test_row_scaled_fp8_dequant_matches_torch():
    """Row-wise FP8 multipliers: W[n,k] = E4M3(code) * g[n], decoded by torch's
    float8_e4m3fn."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (2, 12, 64), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11   # no NaN codes
    ts = (rng.random((2, 12)) * 0.01 + 1e-4).astype(np.float32)
    qw = _QW("fp8", codes, None, ts)
    for e in range(2):
        ref = torch.from_numpy(codes[e]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        ref = ref * ts[e].astype(np.float64)[:, None]
        assert np.array_equal(oracle.dequant(qw, e), ref)


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_row_scales_reduce_to_tensor_scale_and_act_per_row(fmt):
    """Equal row multipliers give exactly the per-matrix result; changing one
    row's multiplier rescales that row alone (by the same factor)."""
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((3, 10, 64)) * 0.05).astype(np.float32)
    if fmt == "fp8":
        parts = [synth.quantize_fp8(w[e]) for e in range(3)]
        codes = np.stack([c for c, _ in parts])
        bs = None
        g = np.array([s for _, s in parts], np.float32)
    else:
        parts = [synth.quantize_nvfp4(w[e]) for e in range(3)]
        codes = np.stack([c for c, _, _ in parts])
        bs = np.stack([b for _, b, _ in parts])
        g = np.array([s for _, _, s in parts], np.float32)
    tensor = _QW(fmt, codes, bs, g)
    rows = np.repeat(g[:, None], 10, axis=1)
    for e in range(3):
        assert np.array_equal(oracle.dequant(_QW(fmt, codes, bs, rows), e), oracle.dequant(tensor, e))
    rows2 = rows.copy()
    rows2[1, 4] *= 4.0
    a, b = oracle.dequant(_QW(fmt, codes, bs, rows), 1), oracle.dequant(_QW(fmt, codes, bs, rows2), 1)
    assert np.array_equal(b[4], 4.0 * a[4])
    assert np.array_equal(np.delete(b, 4, axis=0), np.delete(a, 4, axis=0))


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_generator_scale_modes(fmt):
    """Per-row and per-part scales: each row range is quantised as a matrix of
    its own, so its multiplier is its own amax rule and the round trip keeps
    the per-format bound within every range."""
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    w[4:] *= 10.0   # the up half is ten times larger: per-part scales differ
    for mode, parts in (("row", [(r, r + 1) for r in range(8)]), ("part", [(0, 4), (4, 8)])):
        assert synth.layers._row_parts(8, mode, gate_up=True) == parts
        codes, bs, rs = synth.layers.quantize_scaled_rows(fmt, w, parts)
        for a, b in parts:
            amax = np.float32(np.abs(w[a:b]).max())
            expect = amax / np.float32(448.0) if fmt == "fp8" else amax / np.float32(6 * 448)
            assert np.all(rs[a:b] == np.float32(expect))
        wq = oracle.dequant(_QW(fmt, codes[None], None if bs is None else bs[None], rs[None]), 0)
        for a, b in parts:
            rel = np.abs(wq[a:b] - w[a:b]).max() / np.abs(w[a:b]).max()
            assert rel <= (2 ** -4 if fmt == "fp8" else 1 / 6 + 1e-3)
    assert synth.layers._row_parts(8, "part", gate_up=False) == [(0, 8)]


def test_bf16_weight_decode_matches_torch_on_all_finite_patterns():
    """BF16 experts: every finite bf16 bit pattern against torch's bfloat16."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.dequant(_QW("bf16", bits.reshape(1, 1, -1), None, None), 0)[0]
    assert np.array_equal(got, ref)
