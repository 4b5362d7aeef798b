// Decode experts: few tokens per expert, so the work is streaming the
// selected experts' packed weights from HBM once.
//
// Each wave owns 16 weight rows of one expert and runs 16x16 MFMA tiles whose
// 16 "columns" are those rows and whose 16 "rows" are the (up to 16) tokens
// routed to the expert; absent tokens are zero lanes.  Lane l reads the
// 16-byte slice [32g, 32g+32) (g = l/16) of every 128-element K chunk of
// weight row l%16: one MXFP4 block and its one E8M0 scale, or two NVFP4
// blocks.  Weights are dequantised in registers (gfx950 scaled FP4->bf16
// conversion) and consumed by v_mfma_f32_16x16x32_bf16, so the K reduction
// happens in the matrix core, not in cross-lane shuffles.  FP8 weights with
// FP8 activations go straight to v_mfma_scale_f32_16x16x128_f8f6f4.
//
// The weight loads of NB consecutive chunks are issued together before any
// is consumed, so each wave keeps NB*16 bytes per lane in flight.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kDecWaves = 2;   // waves per workgroup (one expert, adjacent row groups)

struct SlotInfo {
  int count;           // valid token slots (a prefix of the 16)
  int e;               // expert index (0 for the shared expert)
};

// Token of slot r of block b, and whether it is valid; slot list is a prefix.
__device__ __forceinline__ bool slot_token(const Rows& rows, int b, int r, int* flat, int* tok) {
  const int p = b * kDecodeBM + r;
  if (rows.sorted_ids) {
    const int f = rows.sorted_ids[p];
    *flat = f;
    *tok = f / rows.top_k;
    return f < rows.n_flat;
  }
  *flat = p;
  *tok = p;
  return p < rows.n_flat;
}

__device__ __forceinline__ SlotInfo block_info(const Rows& rows, int b) {
  SlotInfo s;
  s.e = rows.sorted_ids ? rows.block_expert[b] : 0;
  int cnt = 0;
  for (int r = 0; r < kDecodeBM; ++r) {
    int f, t;
    if (slot_token(rows, b, r, &f, &t)) cnt = r + 1;
  }
  s.count = cnt;
  return s;
}

// Number of bytes of one 32-element slice of a weight row for each format.
template <int WFMT> struct Fmt;
template <> struct Fmt<kMXFP4> { static constexpr int slice = 16; };
template <> struct Fmt<kNVFP4> { static constexpr int slice = 16; };
template <> struct Fmt<kFP8> { static constexpr int slice = 32; };

// Per-lane weight slice of one 128-element chunk.
struct WSlice {
  uint4 c0, c1;      // codes: fp4 uses c0 only
  uint32_t sc;       // block scale byte(s)
};

template <int WFMT>
__device__ __forceinline__ WSlice load_wslice(const QW& w, size_t row, int K, int kb) {
  WSlice s;
  if constexpr (WFMT == kFP8) {
    const uint4* p = reinterpret_cast<const uint4*>(w.codes + row * K + kb);
    s.c0 = load_nt(p);
    s.c1 = load_nt(p + 1);
    s.sc = 0;
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(w.codes + row * (K / 2) + kb / 2);
    s.c0 = load_nt(p);
    s.c1 = make_uint4(0, 0, 0, 0);
    if constexpr (WFMT == kMXFP4)
      s.sc = w.scales[row * (K / 32) + kb / 32];
    else
      s.sc = *reinterpret_cast<const uint16_t*>(w.scales + row * (K / 16) + kb / 16);
  }
  return s;
}

// bf16 operand (8 values) for MFMA step `st` (0..3) of a weight slice.
template <int WFMT>
__device__ __forceinline__ bf16x8 wslice_bf16(const WSlice& s, int st) {
  uint32_t o[4];
  if constexpr (WFMT == kMXFP4) {
    const uint32_t word = st == 0 ? s.c0.x : st == 1 ? s.c0.y : st == 2 ? s.c0.z : s.c0.w;
    fp4x8_to_bf16(word, e8m0_as_scale(s.sc), o);
  } else if constexpr (WFMT == kNVFP4) {
    const uint32_t word = st == 0 ? s.c0.x : st == 1 ? s.c0.y : st == 2 ? s.c0.z : s.c0.w;
    const float f = e4m3_to_f32((s.sc >> (st < 2 ? 0 : 8)) & 0xFF);
    fp4x8_to_bf16_mul(word, f, o);
  } else {
    const uint4 c = st < 2 ? s.c0 : s.c1;
    const uint32_t w0 = (st & 1) ? c.z : c.x, w1 = (st & 1) ? c.w : c.y;
    f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
    f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
    f32x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
    f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
    o[0] = pack_bf16x2(a[0], a[1]);
    o[1] = pack_bf16x2(b[0], b[1]);
    o[2] = pack_bf16x2(c2[0], c2[1]);
    o[3] = pack_bf16x2(d[0], d[1]);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// FP8 operand (32 bytes) of bf16 values v (32 of them) divided by s.
__device__ __forceinline__ i32x8 quant_row32(const uint16_t* p, float s) {
  i32x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[q];
    const uint32_t lo = f32x2_to_e4m3x2(bf16_to_f32(v.x & 0xFFFF) / s, bf16_to_f32(v.x >> 16) / s);
    const uint32_t hi = f32x2_to_e4m3x2(bf16_to_f32(v.y & 0xFFFF) / s, bf16_to_f32(v.y >> 16) / s);
    const uint32_t lo2 = f32x2_to_e4m3x2(bf16_to_f32(v.z & 0xFFFF) / s, bf16_to_f32(v.z >> 16) / s);
    const uint32_t hi2 = f32x2_to_e4m3x2(bf16_to_f32(v.w & 0xFFFF) / s, bf16_to_f32(v.w >> 16) / s);
    r[2 * q] = static_cast<int>(lo | (hi << 16));
    r[2 * q + 1] = static_cast<int>(lo2 | (hi2 << 16));
  }
  return r;
}

__device__ __forceinline__ float scale_from_amax(const uint32_t* bits) {
  const float a = __uint_as_float(*bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// Accumulate one wave's 16x16 tile over K.  arow(kb) gives the A operand
// source for this lane's token slot (nullptr when the slot is empty).
template <int WFMT, bool FP8ACT, int NB, class ALoad>
__device__ __forceinline__ f32x4 decode_tile(const QW& w, size_t wrow, int K, int g, ALoad aload) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kc0 = 0; kc0 < K; kc0 += NB * 128) {
    WSlice ws[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kb = kc0 + u * 128 + g * 32;
      if (kb < K) ws[u] = load_wslice<WFMT>(w, wrow, K, kb);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int kb = kc0 + u * 128 + g * 32;
      if (kc0 + u * 128 >= K) break;
      if constexpr (WFMT == kFP8 && FP8ACT) {
        const i32x8 a = aload.fp8(kb);
        const i32x8 b = {static_cast<int>(ws[u].c0.x), static_cast<int>(ws[u].c0.y),
                         static_cast<int>(ws[u].c0.z), static_cast<int>(ws[u].c0.w),
                         static_cast<int>(ws[u].c1.x), static_cast<int>(ws[u].c1.y),
                         static_cast<int>(ws[u].c1.z), static_cast<int>(ws[u].c1.w)};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8 a = aload.bf16(kb + st * 8);
          const bf16x8 b = wslice_bf16<WFMT>(ws[u], st);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
      }
    }
  }
  return acc;
}

// A operand from a bf16 row (x or h) or a pre-quantised FP8 row.
struct ALoadBf16Row {
  const uint16_t* row;  // nullptr -> zeros
  __device__ bf16x8 bf16(int kb) const {
    if (!row) return bf16x8{};
    return load_bf16x8(row + kb);
  }
  __device__ i32x8 fp8(int) const { return i32x8{}; }
};
struct ALoadFp8Row {
  const uint8_t* row;
  __device__ bf16x8 bf16(int) const { return bf16x8{}; }
  __device__ i32x8 fp8(int kb) const {
    if (!row) return i32x8{};
    const uint4 a = reinterpret_cast<const uint4*>(row + kb)[0];
    const uint4 b = reinterpret_cast<const uint4*>(row + kb)[1];
    return i32x8{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w),
                 static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
  }
};
struct ALoadQuantRow {  // bf16 row quantised to E4M3 with scale s on load
  const uint16_t* row;
  float s;
  __device__ bf16x8 bf16(int) const { return bf16x8{}; }
  __device__ i32x8 fp8(int kb) const {
    if (!row) return i32x8{};
    return quant_row32(row + kb, s);
  }
};

// ------------------------------------------------------------- gate_up ----
template <int WFMT, bool FP8ACT>
__global__ __launch_bounds__(64 * kDecWaves) void decode_gateup_kernel(QW w, Rows rows, const uint16_t* __restrict__ x,
                                                                       const uint8_t* __restrict__ xq,
                                                                       const uint32_t* __restrict__ amax_x, int H, int I,
                                                                       uint16_t* __restrict__ h,
                                                                       uint32_t* __restrict__ amax_h) {
  const int b = blockIdx.y;
  const SlotInfo si = block_info(rows, b);
  if (si.e < 0 || si.count == 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int i0 = (blockIdx.x * kDecWaves + wave) * 8;
  if (i0 >= I) return;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(si.e) * (2 * I) + (j < 8 ? i0 + j : I + i0 + (j - 8));
  int flat, tok;
  const bool have = j < si.count && slot_token(rows, b, j, &flat, &tok);
  f32x4 acc;
  if constexpr (FP8ACT) {
    ALoadFp8Row al{have ? xq + static_cast<size_t>(tok) * H : nullptr};
    acc = decode_tile<WFMT, FP8ACT, 4>(w, wrow, H, g, al);
  } else {
    ALoadBf16Row al{have ? x + static_cast<size_t>(tok) * H : nullptr};
    acc = decode_tile<WFMT, FP8ACT, (WFMT == kFP8 ? 4 : 8)>(w, wrow, H, g, al);
  }
  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[si.e];
  if constexpr (FP8ACT) f *= scale_from_amax(amax_x);
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float up = __shfl_xor(acc[r], 8, kWave);
    const int slot = 4 * g + r;
    if (j < 8 && slot < si.count) {
      const float v = swiglu(acc[r] * f, up * f);
      h[static_cast<size_t>(b * kDecodeBM + slot) * I + i0 + j] = f32_to_bf16(v);
      m = __builtin_fmaxf(m, __builtin_fabsf(v));
    }
  }
  if constexpr (FP8ACT) {
    m = wave_max(m);
    if (lane == 0) atomicMax(amax_h, __float_as_uint(m));
  }
}

// ---------------------------------------------------------------- down ----
template <int WFMT, bool FP8ACT>
__global__ __launch_bounds__(64 * kDecWaves) void decode_down_kernel(QW w, Rows rows, const uint16_t* __restrict__ h,
                                                                     const uint32_t* __restrict__ amax_h, int H, int I,
                                                                     uint16_t* __restrict__ o) {
  const int b = blockIdx.y;
  const SlotInfo si = block_info(rows, b);
  if (si.e < 0 || si.count == 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int n0 = (blockIdx.x * kDecWaves + wave) * 16;
  if (n0 >= H) return;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(si.e) * H + n0 + j;
  const bool have = j < si.count;
  const uint16_t* hrow = have ? h + static_cast<size_t>(b * kDecodeBM + j) * I : nullptr;
  f32x4 acc;
  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[si.e];
  if constexpr (FP8ACT) {
    const float sh = scale_from_amax(amax_h);
    f *= sh;
    ALoadQuantRow al{hrow, sh};
    acc = decode_tile<WFMT, FP8ACT, 4>(w, wrow, I, g, al);
  } else {
    ALoadBf16Row al{hrow};
    acc = decode_tile<WFMT, FP8ACT, (WFMT == kFP8 ? 4 : 8)>(w, wrow, I, g, al);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = 4 * g + r;
    int flat, tok;
    if (slot < si.count && slot_token(rows, b, slot, &flat, &tok))
      o[static_cast<size_t>(flat) * H + n0 + j] = f32_to_bf16(acc[r] * f);
  }
}

template <int WFMT, bool FP8ACT>
static hipError_t dispatch_decode(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                                  const uint32_t* amax_x, int H, int I, uint16_t* h, uint32_t* amax_h,
                                  hipStream_t s) {
  dim3 grid((I / 8 + kDecWaves - 1) / kDecWaves, rows.num_blocks);
  decode_gateup_kernel<WFMT, FP8ACT><<<grid, 64 * kDecWaves, 0, s>>>(w, rows, x, xq, amax_x, H, I, h, amax_h);
  return hipGetLastError();
}

template <int WFMT, bool FP8ACT>
static hipError_t dispatch_decode_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h,
                                       int H, int I, uint16_t* o, hipStream_t s) {
  dim3 grid((H / 16 + kDecWaves - 1) / kDecWaves, rows.num_blocks);
  decode_down_kernel<WFMT, FP8ACT><<<grid, 64 * kDecWaves, 0, s>>>(w, rows, h, amax_h, H, I, o);
  return hipGetLastError();
}

hipError_t launch_decode_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                                const uint32_t* amax_x, int H, int inter, uint16_t* h, uint32_t* amax_h,
                                int /*max_tokens_per_block*/, hipStream_t s) {
  const bool fp8act = xq != nullptr;
  switch (w.fmt) {
    case kMXFP4: return dispatch_decode<kMXFP4, false>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    case kNVFP4: return dispatch_decode<kNVFP4, false>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    case kFP8:
      return fp8act ? dispatch_decode<kFP8, true>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s)
                    : dispatch_decode<kFP8, false>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h, int H,
                              int inter, uint16_t* o, hipStream_t s) {
  const bool fp8act = amax_h != nullptr;
  switch (w.fmt) {
    case kMXFP4: return dispatch_decode_down<kMXFP4, false>(w, rows, h, amax_h, H, inter, o, s);
    case kNVFP4: return dispatch_decode_down<kNVFP4, false>(w, rows, h, amax_h, H, inter, o, s);
    case kFP8:
      return fp8act ? dispatch_decode_down<kFP8, true>(w, rows, h, amax_h, H, inter, o, s)
                    : dispatch_decode_down<kFP8, false>(w, rows, h, amax_h, H, inter, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ftmoe
