// Decode experts: few tokens per expert, so the work is streaming each
// selected expert's packed weights from HBM exactly once.
//
// Work unit: (block b, row group).  A block is one selected expert with its
// (up to 16) routed rows -- or, after the routed blocks, 16 tokens of the
// shared expert.  Each wave owns 16 weight rows and runs 16x16 MFMA tiles
// whose 16 columns are those rows and whose 16 rows are the block's token
// slots (absent slots are zero).  Lane l reads the 16-byte slice [32g, 32g+32)
// (g = l/16) of every 128-element K chunk of weight row l%16 -- one MXFP4
// block with its one E8M0 scale, or two NVFP4 blocks -- and all of a row's
// chunks are requested before any is used, so a wave has its whole share in
// flight at once.  Weights are dequantised in registers (gfx950 scaled
// FP4->bf16 conversion) into v_mfma_f32_16x16x32_bf16; FP8 weights with FP8
// activations go straight to v_mfma_scale_f32_16x16x128_f8f6f4.  The token
// rows are staged in LDS while the weight loads are in flight.
//
// gate_up writes h = silu(gate) * up; down writes fp32 outputs per routed
// row, and the combine sums each token's rows in ascending slot order j, then
// adds the gated shared expert.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kDownWaves = 4;   // waves per down workgroup: a 64-column tile of y
constexpr int kDownTileN = 16 * kDownWaves;

int decode_down_tiles(int H) { return (H + kDownTileN - 1) / kDownTileN; }

// Per-lane weight slice of one 128-element K chunk.
struct WSlice {
  uint4 c0, c1;      // codes: FP4 uses c0 only
  uint32_t sc;       // block scale byte(s)
};

template <int WFMT>
__device__ __forceinline__ WSlice load_wslice(const QW& w, size_t row, int K, int kb) {
  WSlice s;
  if constexpr (WFMT == kFP8) {
    const uint8_t* p = w.codes + row * K + kb;
    s.c0 = load_nt(p);
    s.c1 = load_nt(p + 16);
    s.sc = 0;
  } else {
    s.c0 = load_nt(w.codes + row * (K / 2) + kb / 2);
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
    fp4x8_to_bf16_mul(word, e4m3_to_f32((s.sc >> (st < 2 ? 0 : 8)) & 0xFF), o);
  } else {
    const uint4 c = st < 2 ? s.c0 : s.c1;
    const uint32_t w0 = (st & 1) ? c.z : c.x, w1 = (st & 1) ? c.w : c.y;
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
    const f32x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
    o[0] = pack_bf16x2(a[0], a[1]);
    o[1] = pack_bf16x2(b[0], b[1]);
    o[2] = pack_bf16x2(c2[0], c2[1]);
    o[3] = pack_bf16x2(d[0], d[1]);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ i32x8 wslice_i32x8(const WSlice& s) {
  return i32x8{static_cast<int>(s.c0.x), static_cast<int>(s.c0.y), static_cast<int>(s.c0.z),
               static_cast<int>(s.c0.w), static_cast<int>(s.c1.x), static_cast<int>(s.c1.y),
               static_cast<int>(s.c1.z), static_cast<int>(s.c1.w)};
}

__device__ __forceinline__ float scale_from_amax(const uint32_t* bits) {
  const float a = __uint_as_float(*bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// Token slots of block b: LDS tok[16] (token index, or -1) and the count of
// valid slots (a prefix).  Also returns flat row ids for routed blocks.
struct SlotTable {
  int tok[kDecodeBM];
  int flat[kDecodeBM];
  int count;
};

__device__ __forceinline__ void fill_slots(const DecodeArgs& a, int b, bool shared, SlotTable* st) {
  if (threadIdx.x < kWave) {
    const int r = lane_id();
    bool valid = false;
    int tok = -1, flat = -1;
    if (r < kDecodeBM) {
      if (shared) {
        tok = (b - a.nb_routed) * kDecodeBM + r;
        flat = tok;
        valid = tok < a.T;
      } else {
        flat = a.sorted_ids[b * kDecodeBM + r];
        valid = flat < a.T * a.k;
        tok = flat / a.k;
      }
    }
    const unsigned long long m = __ballot(valid);
    if (r < kDecodeBM) {
      st->tok[r] = valid ? tok : -1;
      st->flat[r] = valid ? flat : -1;
    }
    if (r == 0) st->count = __popcll(m);
  }
}

// A operand: 8 bf16 (or 32 FP8 bytes) of slot row j at element kb from LDS.
__device__ __forceinline__ bf16x8 lds_row_bf16(const uint8_t* xs, int pitch, int j, int count, int kb) {
  if (j >= count) return bf16x8{};
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xs + j * pitch + kb * 2));
}
__device__ __forceinline__ i32x8 lds_row_fp8(const uint8_t* xs, int pitch, int j, int count, int kb) {
  if (j >= count) return i32x8{};
  const uint4 p = *reinterpret_cast<const uint4*>(xs + j * pitch + kb);
  const uint4 q = *reinterpret_cast<const uint4*>(xs + j * pitch + kb + 16);
  return i32x8{static_cast<int>(p.x), static_cast<int>(p.y), static_cast<int>(p.z), static_cast<int>(p.w),
               static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w)};
}

// MFMA work of one batch of NB chunks held in registers.
template <int WFMT, bool FP8ACT, int NB>
__device__ __forceinline__ void mma_batch(const WSlice* ws, int kc0, int K, int g, const uint8_t* xs, int pitch,
                                          int j, int count, f32x4& acc) {
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    if (kc0 + u * 128 >= K) break;
    const int kb = kc0 + u * 128 + g * 32;
    if constexpr (FP8ACT) {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(lds_row_fp8(xs, pitch, j, count, kb),
                                                             wslice_i32x8(ws[u]), acc, 0, 0, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row_bf16(xs, pitch, j, count, kb + st * 8),
                                                      wslice_bf16<WFMT>(ws[u], st), acc, 0, 0, 0);
    }
  }
}

// ------------------------------------------------------------- gate_up ----
// WPB waves per workgroup, each on 8 adjacent intermediate indices (their 8
// gate rows and 8 up rows); the workgroup shares one LDS copy of its tokens.
template <int WFMT, bool FP8ACT, int NB, int WPB>
__global__ __launch_bounds__(64 * WPB) void decode_gateup_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ SlotTable slots;
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const QW& w = shared ? a.sgu : a.gu;
  const int I = shared ? a.Is : a.I;
  const int H = a.H;
  const int e = shared ? 0 : a.block_expert[b];
  if (e < 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int i0 = (blockIdx.x * WPB + wave) * 8;
  const bool active = i0 < I;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * (2 * I) + (j < 8 ? i0 + j : I + i0 + (j - 8));
  const int pitch = (FP8ACT ? H : 2 * H) + 16;

  WSlice ws[NB];
  if (active) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (u * 128 < H) ws[u] = load_wslice<WFMT>(w, wrow, H, u * 128 + g * 32);
  }
  fill_slots(a, b, shared, &slots);
  __syncthreads();
  const int count = slots.count;
  // Stage the block's token rows (x, or its FP8 codes) in LDS.
  {
    const int row_vec = (FP8ACT ? H : 2 * H) / 16;
    for (int i = threadIdx.x; i < count * row_vec; i += blockDim.x) {
      const int r = i / row_vec, c = i % row_vec;
      const size_t t = static_cast<size_t>(slots.tok[r]);
      const uint4 v = FP8ACT ? reinterpret_cast<const uint4*>(a.xq + t * H)[c]
                             : reinterpret_cast<const uint4*>(a.x + t * H)[c];
      *reinterpret_cast<uint4*>(xs + r * pitch + c * 16) = v;
    }
  }
  __syncthreads();
  if constexpr (!FP8ACT) {
    if (!active) return;
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    mma_batch<WFMT, FP8ACT, NB>(ws, 0, H, g, xs, pitch, j, count, acc);
    for (int kc0 = NB * 128; kc0 < H; kc0 += NB * 128) {
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (kc0 + u * 128 < H) ws[u] = load_wslice<WFMT>(w, wrow, H, kc0 + u * 128 + g * 32);
      mma_batch<WFMT, FP8ACT, NB>(ws, kc0, H, g, xs, pitch, j, count, acc);
    }
  }

  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[e];
  if constexpr (FP8ACT) f *= scale_from_amax(a.amax_x);
  uint16_t* h = shared ? a.hs : a.h;
  const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float up = __shfl_xor(acc[r], 8, kWave);
    const int slot = 4 * g + r;
    if (active && j < 8 && slot < count) {
      const float v = swiglu(acc[r] * f, up * f);
      h[static_cast<size_t>(p0 + slot) * I + i0 + j] = f32_to_bf16(v);
      m = __builtin_fmaxf(m, __builtin_fabsf(v));
    }
  }
  if constexpr (FP8ACT) {
    __shared__ float red[16];
    wg_amax_to_slots(m, a.amax_slots, red);
  }
}

// ----------------------------------------------------- down + combine ----
template <int WFMT, bool FP8ACT, int NB>
__global__ __launch_bounds__(64 * kDownWaves) void decode_down_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t hsm[];
  __shared__ SlotTable slots;
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const QW& w = shared ? a.sdn : a.dn;
  const int K = shared ? a.Is : a.I;
  const int H = a.H;
  const int e = shared ? 0 : a.block_expert[b];
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int tile = blockIdx.x;
  const int n0 = tile * kDownTileN + wave * 16;
  const int j = lane & 15, g = lane >> 4;

  if (e < 0) return;
  {
    const size_t wrow = static_cast<size_t>(e) * H + n0 + j;
    const int kmax = a.Is > a.I ? a.Is : a.I;
    const int pitch = (FP8ACT ? kmax : 2 * kmax) + 16;
    WSlice ws[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (u * 128 < K) ws[u] = load_wslice<WFMT>(w, wrow, K, u * 128 + g * 32);
    fill_slots(a, b, shared, &slots);
    __syncthreads();
    const int count = slots.count;
    float sh = 1.0f;
    if constexpr (FP8ACT) sh = scale_from_amax(a.amax_h);
    // Stage the block's h rows (quantised to E4M3 with the h scale for FP8).
    {
      const uint16_t* hsrc = shared ? a.hs : a.h;
      const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
      const int row_vec = K / 8;  // 8 bf16 per 16-byte load
      for (int i = threadIdx.x; i < count * row_vec; i += blockDim.x) {
        const int r = i / row_vec, c = i % row_vec;
        const uint4 v = reinterpret_cast<const uint4*>(hsrc + static_cast<size_t>(p0 + r) * K)[c];
        if constexpr (FP8ACT) {
          const uint32_t lo = f32x2_to_e4m3x2(bf16_to_f32(v.x & 0xFFFF) / sh, bf16_to_f32(v.x >> 16) / sh);
          const uint32_t hi = f32x2_to_e4m3x2(bf16_to_f32(v.y & 0xFFFF) / sh, bf16_to_f32(v.y >> 16) / sh);
          const uint32_t lo2 = f32x2_to_e4m3x2(bf16_to_f32(v.z & 0xFFFF) / sh, bf16_to_f32(v.z >> 16) / sh);
          const uint32_t hi2 = f32x2_to_e4m3x2(bf16_to_f32(v.w & 0xFFFF) / sh, bf16_to_f32(v.w >> 16) / sh);
          *reinterpret_cast<uint2*>(hsm + r * pitch + c * 8) = make_uint2(lo | (hi << 16), lo2 | (hi2 << 16));
        } else {
          *reinterpret_cast<uint4*>(hsm + r * pitch + c * 16) = v;
        }
      }
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mma_batch<WFMT, FP8ACT, NB>(ws, 0, K, g, hsm, pitch, j, count, acc);
    for (int kc0 = NB * 128; kc0 < K; kc0 += NB * 128) {
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (kc0 + u * 128 < K) ws[u] = load_wslice<WFMT>(w, wrow, K, kc0 + u * 128 + g * 32);
      mma_batch<WFMT, FP8ACT, NB>(ws, kc0, K, g, hsm, pitch, j, count, acc);
    }
    float f = 1.0f;
    if constexpr (WFMT != kMXFP4) f = w.tscale[e];
    if constexpr (FP8ACT) f *= sh;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int slot = 4 * g + r;
      if (slot < count) {
        if (shared)
          a.s32[static_cast<size_t>(slots.tok[slot]) * H + n0 + j] = acc[r] * f;
        else
          a.o32[static_cast<size_t>(slots.flat[slot]) * H + n0 + j] = acc[r] * f;
      }
    }
  }

}

// y[t] = sum_j w[t,j] o[t*k+j] (ascending j) + sg[t] s[t], from the fp32
// partial outputs; one thread per 4 columns.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int per_row = a.H / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.T * per_row) return;
  const int t = idx / per_row, c = (idx % per_row) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int jj = 0; jj < a.k; ++jj) {
    const size_t r = static_cast<size_t>(t) * a.k + jj;
    const float wj = a.w[r];
    const float4 v = *reinterpret_cast<const float4*>(a.o32 + r * a.H + c);
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (a.sg) {
    const float g = a.sg[t];
    const float4 v = *reinterpret_cast<const float4*>(a.s32 + static_cast<size_t>(t) * a.H + c);
    acc.x = fmaf(g, v.x, acc.x);
    acc.y = fmaf(g, v.y, acc.y);
    acc.z = fmaf(g, v.z, acc.z);
    acc.w = fmaf(g, v.w, acc.w);
  }
  *reinterpret_cast<uint2*>(a.y + static_cast<size_t>(t) * a.H + c) =
      make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

// Kernels that may need more than 64 KB of dynamic LDS opt in once.
template <class Kern>
static hipError_t allow_lds(Kern kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  if (bytes > 150 * 1024) return hipErrorInvalidValue;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

template <int WFMT, bool FP8ACT, int WPB>
static hipError_t run_decode_gateup_w(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = WFMT == kFP8 ? 8 : 16;
  const int imax = a.Is > a.I ? a.Is : a.I;
  const int rows = a.T < kDecodeBM ? a.T : kDecodeBM;
  const size_t lds = static_cast<size_t>(rows) * ((FP8ACT ? a.H : 2 * a.H) + 16);
  dim3 grid((imax / 8 + WPB - 1) / WPB, a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_gateup_kernel<WFMT, FP8ACT, NB, WPB>, lds);
  if (e != hipSuccess) return e;
  decode_gateup_kernel<WFMT, FP8ACT, NB, WPB><<<grid, 64 * WPB, lds, s>>>(a);
  return hipGetLastError();
}

// One-token batches touch few experts: single-wave workgroups spread them over
// every CU.  Larger batches share each LDS token copy among 8 waves.
template <int WFMT, bool FP8ACT>
static hipError_t run_decode_gateup(const DecodeArgs& a, hipStream_t s) {
  if (a.T <= 2) return run_decode_gateup_w<WFMT, FP8ACT, 1>(a, s);
  return run_decode_gateup_w<WFMT, FP8ACT, 8>(a, s);
}

template <int WFMT, bool FP8ACT>
static hipError_t run_decode_down(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = WFMT == kFP8 ? 4 : 8;
  const int kmax = a.Is > a.I ? a.Is : a.I;
  const int rows = a.T < kDecodeBM ? a.T : kDecodeBM;
  const size_t lds = static_cast<size_t>(rows) * ((FP8ACT ? kmax : 2 * kmax) + 16);
  dim3 grid(decode_down_tiles(a.H), a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_down_kernel<WFMT, FP8ACT, NB>, lds);
  if (e != hipSuccess) return e;
  decode_down_kernel<WFMT, FP8ACT, NB><<<grid, 64 * kDownWaves, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_gateup(const DecodeArgs& a, hipStream_t s) {
  const bool fp8act = a.xq != nullptr;
  switch (a.gu.fmt) {
    case kMXFP4: return run_decode_gateup<kMXFP4, false>(a, s);
    case kNVFP4: return run_decode_gateup<kNVFP4, false>(a, s);
    case kFP8: return fp8act ? run_decode_gateup<kFP8, true>(a, s) : run_decode_gateup<kFP8, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s) {
  const int n = a.T * (a.H / 4);
  decode_combine_kernel<<<(n + 255) / 256, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s) {
  const bool fp8act = a.amax_h != nullptr;
  switch (a.dn.fmt) {
    case kMXFP4: return run_decode_down<kMXFP4, false>(a, s);
    case kNVFP4: return run_decode_down<kNVFP4, false>(a, s);
    case kFP8: return fp8act ? run_decode_down<kFP8, true>(a, s) : run_decode_down<kFP8, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ftmoe
