"""Seeded generator of MoE layers and token batches.

Every workload is synthetic.  The shapes and distributions follow the layer
configurations the MoE forward is measured on (tiny check layer, a
30B-A3B-class layer, a 512-expert layer with a shared expert, an FP8 layer with
Zipf-skewed routing).  The packing follows the public block-scaled formats
named on the FreeToken README ("Broad MoE & Ecosystem Support": MXFP4, NVFP4,
FP8): OCP Microscaling v1.0 for E2M1 elements with E8M0 scales per 32, NVIDIA's
NVFP4 (E2M1 per 16 with an E4M3 block scale and an fp32 tensor scale) and OCP
OFP8 E4M3 ("FN": bias 7, max 448, no infinities).

Random streams: every tensor draws from its own child of
``numpy.random.SeedSequence(seed)`` so experts can be generated in parallel
threads with results independent of scheduling.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

# --------------------------------------------------------------------------
# bf16 <-> f32 bit helpers (input preparation only)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Element encoders used to build the packed weights
# --------------------------------------------------------------------------


def e2m1_encode(a: np.ndarray) -> np.ndarray:
    """fp32 -> 4-bit E2M1 code, round to nearest with ties to the even code,
    saturating at +-6.  Magnitudes 0,.5,1,1.5,2,3,4,6 are codes 0..7; bit 3 is
    the sign (so -0 keeps its sign bit)."""
    a = np.asarray(a, dtype=np.float32)
    m = np.abs(a)
    # Midpoints between neighbouring magnitudes; at a midpoint the even code
    # wins, so the comparison is strict when the lower neighbour is even.
    c = (m > 0.25).astype(np.uint8)
    c += m >= 0.75
    c += m > 1.25
    c += m >= 1.75
    c += m > 2.5
    c += m >= 3.5
    c += m > 5.0
    return c | (np.signbit(a).astype(np.uint8) << 3)


def e4m3_encode(a: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3FN code, round to nearest even, saturating at +-448."""
    a = np.asarray(a, dtype=np.float32)
    m = np.minimum(np.abs(a).astype(np.float64), 448.0)
    # Quantum of the binade holding m: 2^(e-3) for normals (e >= -6), 2^-9 below.
    _, ex = np.frexp(m)  # m = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, e - 3)
    r = np.rint(m / q) * q  # exact: m/q has few bits, rint is ties-to-even
    r = np.minimum(r, 448.0)
    # Re-derive the code from the rounded magnitude (rounding may carry into
    # the next binade, which is still the right code).
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    normal = r >= 2.0 ** -6
    mant_n = np.where(normal, np.ldexp(r, -np.where(normal, e2, 0)) * 8 - 8, 0)
    code_n = ((e2 + 7) << 3) + mant_n.astype(np.int64)
    code_s = np.rint(r / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_n, code_s).astype(np.uint8)
    return code | (np.signbit(a).astype(np.uint8) << 7)


def _e4m3_value(code: np.ndarray) -> np.ndarray:
    """E4M3FN code -> fp32 value (used only to form NVFP4 block divisors)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.ldexp(1.0, e - 7))
    return (s * v).astype(np.float32)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K/2] bytes, element 2i in the low nibble."""
    c = codes.reshape(*codes.shape[:-1], codes.shape[-1] // 2, 2)
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


# --------------------------------------------------------------------------
# Block quantisers (one expert matrix [N, K] at a time)
# --------------------------------------------------------------------------


def quantize_mxfp4(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP4: 32-element blocks along K, scale 2^(floor(log2 amax) - 2) as an
    E8M0 code, elements E2M1 with nearest-even rounding, saturating.
    Returns (codes [N, K/2] uint8, scales [N, K/32] uint8)."""
    n, k = w.shape
    b = w.reshape(n, k // 32, 32).astype(np.float32)
    amax = np.abs(b).max(axis=2)
    _, p = np.frexp(amax)                      # amax = f * 2^p, f in [0.5, 1)
    e = np.clip(p.astype(np.int64) - 1 - 2, -127, 127)
    zero = amax == 0
    e = np.where(zero, -127, e)
    scaled = np.ldexp(b, (-e)[..., None].astype(np.int32)).astype(np.float32)
    codes = e2m1_encode(scaled)
    codes = np.where(zero[..., None], np.uint8(0), codes)
    return _pack_nibbles(codes.reshape(n, k)), (e + 127).astype(np.uint8)


def quantize_nvfp4(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray, float]:
    """NVFP4: fp32 tensor scale g = amax/(6*448); per 16-element block an E4M3
    scale of amax_b/(6 g); elements E2M1 of w/(scale_b * g).
    Returns (codes [N, K/2], block scales [N, K/16] E4M3 codes, g)."""
    n, k = w.shape
    w = w.astype(np.float32)
    amax = np.float32(np.abs(w).max())
    g = np.float32(amax / np.float32(6 * 448)) if amax > 0 else np.float32(1.0)
    b = w.reshape(n, k // 16, 16)
    amax_b = np.abs(b).max(axis=2)
    sb = e4m3_encode(amax_b / (np.float32(6.0) * g))
    denom = (_e4m3_value(sb) * g).astype(np.float32)
    safe = np.where(denom == 0, np.float32(1.0), denom)
    codes = e2m1_encode(b / safe[..., None])
    codes = np.where((denom == 0)[..., None], np.uint8(0), codes)
    return _pack_nibbles(codes.reshape(n, k)), sb, float(g)


def quantize_fp8(w: np.ndarray) -> Tuple[np.ndarray, float]:
    """FP8 E4M3 with one fp32 scale per matrix: s = amax/448."""
    w = w.astype(np.float32)
    amax = np.float32(np.abs(w).max())
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    return e4m3_encode(w / s), float(s)


def _row_parts(n: int, mode: str, gate_up: bool):
    """Row ranges that share one fp32 scale: the whole matrix ("tensor"), each
    row ("row"), or the gate and up halves of a fused gate_up ("part"; a down
    matrix is one part)."""
    if mode == "tensor":
        return [(0, n)]
    if mode == "row":
        return [(r, r + 1) for r in range(n)]
    if mode == "part":
        return [(0, n // 2), (n // 2, n)] if gate_up else [(0, n)]
    raise ValueError(f"unknown scale mode {mode!r}")


def quantize_scaled_rows(fmt: str, w: np.ndarray, parts):
    """NVFP4 or FP8 with one fp32 scale per row range of ``parts`` (each range
    quantised as its own matrix).  Returns (codes, block scales or None,
    per-row scales [N] fp32)."""
    n, k = w.shape
    rs = np.empty((n,), np.float32)
    codes = np.empty((n, k // 2 if fmt == "nvfp4" else k), np.uint8)
    bs = np.empty((n, k // 16), np.uint8) if fmt == "nvfp4" else None
    for a, b in parts:
        if fmt == "nvfp4":
            codes[a:b], bs[a:b], g = quantize_nvfp4(w[a:b])
        else:
            codes[a:b], g = quantize_fp8(w[a:b])
        rs[a:b] = g
    return codes, bs, rs


# --------------------------------------------------------------------------
# Layer description
# --------------------------------------------------------------------------


@dataclass
class QWeight:
    """Stacked packed matrices, row-major [E][N][K] with K contiguous."""
    fmt: str                      # "mxfp4" | "nvfp4" | "fp8" | "bf16"
    num_experts: int
    n: int
    k: int
    codes: np.ndarray             # fp4: [E, N, K/2] uint8; fp8: [E, N, K] uint8; bf16: [E, N, K] uint16
    block_scales: Optional[np.ndarray]   # mxfp4 [E,N,K/32] | nvfp4 [E,N,K/16] | None
    tensor_scales: Optional[np.ndarray]  # nvfp4/fp8 [E] fp32, or [E, N] (one per row) | None

    def nbytes_per_expert(self) -> int:
        b = self.codes[0].nbytes
        if self.block_scales is not None:
            b += self.block_scales[0].nbytes
        if self.tensor_scales is not None:
            b += self.tensor_scales[0].nbytes
        return b


@dataclass(frozen=True)
class LayerConfig:
    name: str
    tokens: Tuple[int, ...]
    hidden: int
    num_experts: int
    top_k: int
    inter: int
    fmt: str
    act: str = "bf16"             # "bf16" | "fp8" (per-tensor E4M3) | "mxfp8" (E4M3 + E8M0 per 32)
    shared_inter: int = 0
    router_std: Optional[float] = None   # None -> 1/sqrt(hidden)
    zipf_s: Optional[float] = None
    zipf_ratio: float = 10.0
    seed: int = 0
    gap: float = 1e-3
    bias_mode: str = "logits"     # router bias in "logits" (selection and weights) or "select" (selection only)
    scale_mode: str = "tensor"    # NVFP4/FP8 fp32 scale per matrix, "row", or "part" (gate and up halves)


CONFIGS = {
    "c0": LayerConfig("c0", (16,), 256, 8, 2, 128, "mxfp4", router_std=0.02, seed=0),
    "c1": LayerConfig("c1", (1, 8), 2048, 128, 8, 768, "mxfp4", seed=1),
    "c2": LayerConfig("c2", (4096,), 2048, 128, 8, 768, "mxfp4", seed=1),
    "c3": LayerConfig("c3", (1, 8192), 2048, 512, 10, 512, "nvfp4", shared_inter=512, seed=3),
    "c4": LayerConfig("c4", (16384,), 4096, 128, 8, 1536, "fp8", act="fp8", zipf_s=1.1, seed=4),
    # the c4 layer with its Zipf router bias taking part in the selection only
    "c4-selbias": LayerConfig("c4-selbias", (16384,), 4096, 128, 8, 1536, "fp8", act="fp8", zipf_s=1.1,
                              bias_mode="select", seed=4),
    # the c2 layer's shape with BF16 experts
    "c2-bf16": LayerConfig("c2-bf16", (4096,), 2048, 128, 8, 768, "bf16", seed=1),
    # the c1 / c2 layers (same weights) with MXFP8 activations (W4A8)
    "c1-w4a8": LayerConfig("c1-w4a8", (1, 8), 2048, 128, 8, 768, "mxfp4", act="mxfp8", seed=1),
    "c2-w4a8": LayerConfig("c2-w4a8", (4096,), 2048, 128, 8, 768, "mxfp4", act="mxfp8", seed=1),
}


@dataclass
class Layer:
    cfg: LayerConfig
    router_w: np.ndarray                  # [E, H] fp32
    router_b: Optional[np.ndarray]        # [E] fp32 or None
    gate_up: QWeight                      # N = 2I (gate rows then up rows), K = H
    down: QWeight                         # N = H, K = I
    shared_gate_up: Optional[QWeight] = None
    shared_down: Optional[QWeight] = None
    shared_gate_w: Optional[np.ndarray] = None   # [H] fp32
    zipf_alpha: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def hidden(self): return self.cfg.hidden

    @property
    def num_experts(self): return self.cfg.num_experts

    @property
    def top_k(self): return self.cfg.top_k

    @property
    def inter(self): return self.cfg.inter


def _workers() -> int:
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return max(1, min(16, n))


def _normal(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(ss))
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _make_qweight(fmt: str, ss_list, n: int, k: int, std: float, scale_mode: str = "tensor",
                  gate_up: bool = False) -> QWeight:
    e = len(ss_list)
    if scale_mode != "tensor":
        if fmt in ("mxfp4", "bf16"):
            raise ValueError(f"{fmt} has no fp32 scale to split by rows")
        parts = _row_parts(n, scale_mode, gate_up)
        codes = np.empty((e, n, k // 2 if fmt == "nvfp4" else k), np.uint8)
        bs = np.empty((e, n, k // 16), np.uint8) if fmt == "nvfp4" else None
        ts = np.empty((e, n), np.float32)

        def one_rows(i):
            w = _normal(ss_list[i], (n, k), std)
            c, b, r = quantize_scaled_rows(fmt, w, parts)
            codes[i], ts[i] = c, r
            if bs is not None:
                bs[i] = b

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one_rows, range(e)))
        return QWeight(fmt, e, n, k, codes, bs, ts)
    if fmt in ("mxfp4", "nvfp4"):
        codes = np.empty((e, n, k // 2), np.uint8)
        bs = np.empty((e, n, k // (32 if fmt == "mxfp4" else 16)), np.uint8)
    elif fmt == "fp8":
        codes = np.empty((e, n, k), np.uint8)
        bs = None
    elif fmt == "bf16":
        codes = np.empty((e, n, k), np.uint16)
        bs = None
    else:
        raise ValueError(f"unknown weight format {fmt!r}")
    ts = None if fmt in ("mxfp4", "bf16") else np.empty((e,), np.float32)

    def one(i):
        w = _normal(ss_list[i], (n, k), std)
        if fmt == "bf16":
            codes[i] = f32_to_bf16_bits(w)
        elif fmt == "mxfp4":
            codes[i], bs[i] = quantize_mxfp4(w)
        elif fmt == "nvfp4":
            codes[i], bs[i], ts[i] = quantize_nvfp4(w)
        else:
            codes[i], ts[i] = quantize_fp8(w)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(e)))
    return QWeight(fmt, e, n, k, codes, bs, ts)


def _topk_ids_fast(logits: np.ndarray, k: int) -> np.ndarray:
    return np.argpartition(-logits, k - 1, axis=1)[:, :k]


def _zipf_bias(alpha: float, s: float, ranks: np.ndarray) -> np.ndarray:
    return (-s * alpha * np.log(ranks.astype(np.float64))).astype(np.float32)


_LAYER_CACHE: dict = {}


def make_layer(cfg, cache: bool = True) -> Layer:
    """Build (or fetch from the in-process cache) the layer for a config."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    # the arrays do not depend on the activation mode, the bias mode or the name
    key = (cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter, cfg.fmt, cfg.scale_mode,
           cfg.shared_inter, cfg.router_std, cfg.zipf_s, cfg.zipf_ratio, cfg.seed)
    if cache and key in _LAYER_CACHE:
        lay = _LAYER_CACHE[key]
        if lay.cfg != cfg:
            lay = Layer(**{**lay.__dict__, "cfg": cfg})
        return lay
    H, E, k, I = cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter
    root = np.random.SeedSequence(cfg.seed)
    (s_router, s_bias, s_sg, s_gu, s_d, s_sgu, s_sd, s_cal) = root.spawn(8)
    std_r = cfg.router_std if cfg.router_std is not None else 1.0 / math.sqrt(H)
    router_w = _normal(s_router, (E, H), std_r)
    gate_up = _make_qweight(cfg.fmt, s_gu.spawn(E), 2 * I, H, 1.0 / math.sqrt(H), cfg.scale_mode, gate_up=True)
    down = _make_qweight(cfg.fmt, s_d.spawn(E), H, I, 1.0 / math.sqrt(I), cfg.scale_mode)
    lay = Layer(cfg, router_w, None, gate_up, down)
    if cfg.shared_inter:
        Is = cfg.shared_inter
        lay.shared_gate_up = _make_qweight(cfg.fmt, s_sgu.spawn(1), 2 * Is, H, 1.0 / math.sqrt(H), cfg.scale_mode,
                                           gate_up=True)
        lay.shared_down = _make_qweight(cfg.fmt, s_sd.spawn(1), H, Is, 1.0 / math.sqrt(Is), cfg.scale_mode)
        lay.shared_gate_w = _normal(s_sg, (H,), 1.0 / math.sqrt(H))
    if cfg.zipf_s is not None:
        # Router bias alpha * log(Zipf(s) probability) over a seeded rank
        # permutation; alpha is set by bisection on a calibration batch so
        # that the busiest expert receives zipf_ratio times the mean load.
        rng = np.random.Generator(np.random.PCG64(s_bias))
        ranks = rng.permutation(E) + 1
        T_cal = 16384
        xc = bf16_bits_to_f32(f32_to_bf16_bits(_normal(s_cal, (T_cal, H), 1.0)))
        base = xc.astype(np.float64) @ router_w.astype(np.float64).T
        mean = T_cal * k / E

        def ratio(a):
            ids = _topk_ids_fast(base + _zipf_bias(a, cfg.zipf_s, ranks), k)
            return np.bincount(ids.ravel(), minlength=E).max() / mean

        lo, hi = 0.0, 4.0
        for _ in range(40):
            mid = 0.5 * (lo + hi)
            if ratio(mid) < cfg.zipf_ratio:
                lo = mid
            else:
                hi = mid
        lay.zipf_alpha = 0.5 * (lo + hi)
        lay.router_b = _zipf_bias(lay.zipf_alpha, cfg.zipf_s, ranks)
        lay.extra["zipf_ranks"] = ranks
        lay.extra["calibration_ratio"] = ratio(lay.zipf_alpha)
    if cache:
        _LAYER_CACHE[key] = lay
    return lay


def _gap_ok(x_bits: np.ndarray, lay: Layer, gap: float) -> np.ndarray:
    """True per token when the top-(k+1) fp64 logits are pairwise >= gap apart
    (the k-th/k+1-th boundary fixes the chosen set, the rest fix its order)."""
    E, k = lay.num_experts, lay.top_k
    lg = bf16_bits_to_f32(x_bits).astype(np.float64) @ lay.router_w.astype(np.float64).T
    if lay.router_b is not None:
        lg = lg + lay.router_b.astype(np.float64)
    m = min(k + 1, E)
    top = -np.sort(-lg, axis=1)[:, :m]
    if m < 2:
        return np.ones(lg.shape[0], bool)
    return (top[:, :-1] - top[:, 1:]).min(axis=1) >= gap


def make_tokens(lay: Layer, T: int, stream: int = 0, max_tries: int = 64) -> np.ndarray:
    """bf16 N(0,1) hidden states [T, H] (uint16 bits).  A row whose top-k
    logits fall within ``cfg.gap`` of each other is redrawn (next draws of
    the same stream), so routing has exactly one correct answer."""
    H = lay.hidden
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([lay.cfg.seed, 1000 + stream])))
    x = f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    if T == 0:
        return x
    for _ in range(max_tries):
        ok = _gap_ok(x, lay, lay.cfg.gap)
        bad = np.flatnonzero(~ok)
        if bad.size == 0:
            return x
        x[bad] = f32_to_bf16_bits(rng.standard_normal((bad.size, H), dtype=np.float32))
    raise RuntimeError(f"could not draw {T} tokens with a {lay.cfg.gap} top-k gap")
