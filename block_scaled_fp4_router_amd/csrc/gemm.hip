// Prefill experts: grouped GEMMs over the expert-sorted row blocks.
//
// gate_up: for each block of BM=64 rows of one expert and each tile of 64
// intermediate columns, the workgroup multiplies the gathered activation rows
// by 64 gate rows and the 64 matching up rows of the expert's gate_up matrix
// and writes h = silu(gate) * up (bf16) -- the SwiGLU never leaves registers.
// down: the same blocks times 128 rows of the expert's down matrix, written
// to the flat (token, slot) rows of o.
//
// Operands are staged through LDS in K slices.  FP4 weights are dequantised
// to bf16 on the way into LDS (MXFP4 with the hardware E8M0-scaled convert,
// NVFP4 as E2M1 x E4M3 which is exact in bf16) and feed
// v_mfma_f32_32x32x16_bf16.  FP8 weights with FP8 activations are staged as
// bytes and feed v_mfma_scale_f32_32x32x64_f8f6f4 (unit scales); the tensor
// and activation scales are applied in the epilogue.  The next K slice is
// loaded into registers while the current one is multiplied.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kBM = kPrefillBM;   // 64 rows per block
constexpr int kGateN = 64;        // gate columns per gate_up tile (+64 up)
constexpr int kDownN = 128;       // output columns per down tile

// Row gather for block b, row r (0..BM-1): token index and validity.
__device__ __forceinline__ bool row_token(const Rows& rows, int p, int* tok, int* flat) {
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

__device__ __forceinline__ int block_expert_of(const Rows& rows, int b) {
  return rows.sorted_ids ? rows.block_expert[b] : 0;
}

// ------------------------------------------------------------ B staging ---
// 128 weight rows x one K slice, 256 threads, thread t owns row t/2 and half
// t%2 of the slice.  Registers hold the raw bytes until the LDS store.
template <int WFMT, bool FP8ACT>
struct BStage {
  static constexpr int kBK = FP8ACT ? 128 : 64;            // K elements per slice
  static constexpr int kBytesPerThread = (WFMT == kFP8) ? (kBK / 2) : 16;
  uint4 c[kBytesPerThread / 16];
  uint32_t sc;

  __device__ void load(const QW& w, size_t row, int K, int k0, int half) {
    const int kb = k0 + half * (kBK / 2);
    if constexpr (WFMT == kFP8) {
      const uint4* p = reinterpret_cast<const uint4*>(w.codes + row * K + kb);
#pragma unroll
      for (int i = 0; i < kBytesPerThread / 16; ++i) c[i] = load_nt(p + i);
      sc = 0;
    } else {
      c[0] = load_nt(reinterpret_cast<const uint4*>(w.codes + row * (K / 2) + kb / 2));
      if constexpr (WFMT == kMXFP4)
        sc = w.scales[row * (K / 32) + kb / 32];
      else
        sc = *reinterpret_cast<const uint16_t*>(w.scales + row * (K / 16) + kb / 16);
    }
  }

  // Writes this thread's part of the slice to LDS row `dst` (bf16 elements or
  // FP8 bytes), starting at the thread's half.
  __device__ void store(uint8_t* dst_row, int half) const {
    if constexpr (FP8ACT) {
      uint4* d = reinterpret_cast<uint4*>(dst_row + half * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = c[i];
    } else if constexpr (WFMT == kFP8) {
      uint4* d = reinterpret_cast<uint4*>(dst_row + half * 64);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t words[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(words[q], 1.0f, false);
          f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(words[q], 1.0f, true);
          o[2 * q] = pack_bf16x2(lo[0], lo[1]);
          o[2 * q + 1] = pack_bf16x2(hi[0], hi[1]);
        }
        d[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
        d[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
      }
    } else {
      uint4* d = reinterpret_cast<uint4*>(dst_row + half * 64);
      const uint32_t words[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
        if constexpr (WFMT == kMXFP4) {
          fp4x8_to_bf16(words[q], e8m0_as_scale(sc), o);
        } else {
          fp4x8_to_bf16_mul(words[q], e4m3_to_f32((sc >> (q < 2 ? 0 : 8)) & 0xFF), o);
        }
        d[q] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

// LDS row pitch in bytes (slice bytes + 16 to spread banks).
template <bool FP8ACT> struct Pitch { static constexpr int kBytes = (FP8ACT ? 128 : 128) + 16; };

// --------------------------------------------------------- MFMA helpers ---
__device__ __forceinline__ bf16x8 lds_bf16x8(const uint8_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ i32x8 lds_i32x8(const uint8_t* p) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const uint4 b = reinterpret_cast<const uint4*>(p)[1];
  return i32x8{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w),
               static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
}

// acc[c] += A(rows arow0..+32) * B(rows brow[c]..+32)^T over one LDS slice.
template <bool FP8ACT, int NC>
__device__ __forceinline__ void mma_slice(const uint8_t* As, const uint8_t* Bs, int arow0, const int brow[NC],
                                          f32x16 acc[NC], int lane) {
  constexpr int P = Pitch<FP8ACT>::kBytes;
  const int r = lane & 31, g = lane >> 5;
  if constexpr (FP8ACT) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i32x8 a = lds_i32x8(As + (arow0 + r) * P + ks * 64 + g * 32);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const i32x8 b = lds_i32x8(Bs + (brow[c] + r) * P + ks * 64 + g * 32);
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = lds_bf16x8(As + (arow0 + r) * P + (ks * 16 + g * 8) * 2);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 b = lds_bf16x8(Bs + (brow[c] + r) * P + (ks * 16 + g * 8) * 2);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ float scale_from_amax_bits(const uint32_t* bits) {
  const float a = __uint_as_float(*bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// ------------------------------------------------------------- gate_up ----
template <int WFMT, bool FP8ACT>
__global__ __launch_bounds__(256) void gemm_gateup_kernel(QW w, Rows rows, const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ xq,
                                                          const uint32_t* __restrict__ amax_x, int H, int I,
                                                          uint16_t* __restrict__ h, uint32_t* __restrict__ amax_h) {
  constexpr int P = Pitch<FP8ACT>::kBytes;
  constexpr int BK = BStage<WFMT, FP8ACT>::kBK;
  __shared__ __attribute__((aligned(16))) uint8_t As[kBM * P];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2 * kGateN * P];

  const int b = blockIdx.y;
  const int e = block_expert_of(rows, b);
  if (e < 0) return;
  const int n0 = blockIdx.x * kGateN;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // A staging: row tid/4, part tid%4 (32 bytes of the 128-byte slice row).
  const int a_row = tid >> 2, a_part = tid & 3;
  int tok, flat;
  const bool a_valid = row_token(rows, b * kBM + a_row, &tok, &flat);
  // B staging: tile row tid/2 (gate rows 0..63, up rows 64..127), half tid%2.
  const int b_row = tid >> 1, b_half = tid & 1;
  const size_t wrow = static_cast<size_t>(e) * (2 * I) + (b_row < kGateN ? n0 + b_row : I + n0 + (b_row - kGateN));

  uint4 areg[2];
  BStage<WFMT, FP8ACT> breg;
  auto load_a = [&](int k0) {
    if (!a_valid) {
      areg[0] = areg[1] = make_uint4(0, 0, 0, 0);
      return;
    }
    const uint4* p;
    if constexpr (FP8ACT)
      p = reinterpret_cast<const uint4*>(xq + static_cast<size_t>(tok) * H + k0 + a_part * 32);
    else
      p = reinterpret_cast<const uint4*>(x + static_cast<size_t>(tok) * H + k0 + a_part * 16);
    areg[0] = p[0];
    areg[1] = p[1];
  };

  f32x16 acc[2] = {};
  const int brow[2] = {wn * 32, kGateN + wn * 32};
  load_a(0);
  breg.load(w, wrow, H, 0, b_half);
  for (int k0 = 0; k0 < H; k0 += BK) {
    uint4* ad = reinterpret_cast<uint4*>(As + a_row * P + a_part * 32);
    ad[0] = areg[0];
    ad[1] = areg[1];
    breg.store(Bs + b_row * P, b_half);
    __syncthreads();
    if (k0 + BK < H) {
      load_a(k0 + BK);
      breg.load(w, wrow, H, k0 + BK, b_half);
    }
    mma_slice<FP8ACT, 2>(As, Bs, wm * 32, brow, acc, lane);
    __syncthreads();
  }

  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[e];
  if constexpr (FP8ACT) f *= scale_from_amax_bits(amax_x);
  const int j = lane & 31, g = lane >> 5;
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * g + (r & 3);
    const int p = b * kBM + wm * 32 + i;
    const float v = swiglu(acc[0][r] * f, acc[1][r] * f);
    m = __builtin_fmaxf(m, __builtin_fabsf(v));
    h[static_cast<size_t>(p) * I + n0 + wn * 32 + j] = f32_to_bf16(v);
  }
  if constexpr (FP8ACT) {
    __shared__ float red[16];
    wg_amax_to_slots(m, amax_h, red);
  }
}

// ---------------------------------------------------------------- down ----
template <int WFMT, bool FP8ACT>
__global__ __launch_bounds__(256) void gemm_down_kernel(QW w, Rows rows, const uint16_t* __restrict__ h,
                                                        const uint32_t* __restrict__ amax_h, int H, int I,
                                                        uint16_t* __restrict__ o) {
  constexpr int P = Pitch<FP8ACT>::kBytes;
  constexpr int BK = BStage<WFMT, FP8ACT>::kBK;
  __shared__ __attribute__((aligned(16))) uint8_t As[kBM * P];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[kDownN * P];

  const int b = blockIdx.y;
  const int e = block_expert_of(rows, b);
  if (e < 0) return;
  const int n0 = blockIdx.x * kDownN;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  float sh = 1.0f;
  if constexpr (FP8ACT) sh = scale_from_amax_bits(amax_h);

  const int a_row = tid >> 2, a_part = tid & 3;
  const uint16_t* arow = h + static_cast<size_t>(b * kBM + a_row) * I;
  const int b_row = tid >> 1, b_half = tid & 1;
  const size_t wrow = static_cast<size_t>(e) * H + n0 + b_row;

  uint4 areg[4];
  BStage<WFMT, FP8ACT> breg;
  auto load_a = [&](int k0) {
    if constexpr (FP8ACT) {
      const uint4* p = reinterpret_cast<const uint4*>(arow + k0 + a_part * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) areg[i] = p[i];
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(arow + k0 + a_part * 16);
      areg[0] = p[0];
      areg[1] = p[1];
    }
  };
  auto store_a = [&]() {
    uint4* ad = reinterpret_cast<uint4*>(As + a_row * P + a_part * 32);
    if constexpr (FP8ACT) {
      uint32_t q[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f32x2_to_e4m3x2(bf16_to_f32(areg[i].x & 0xFFFF) / sh, bf16_to_f32(areg[i].x >> 16) / sh);
        const uint32_t hi = f32x2_to_e4m3x2(bf16_to_f32(areg[i].y & 0xFFFF) / sh, bf16_to_f32(areg[i].y >> 16) / sh);
        const uint32_t lo2 = f32x2_to_e4m3x2(bf16_to_f32(areg[i].z & 0xFFFF) / sh, bf16_to_f32(areg[i].z >> 16) / sh);
        const uint32_t hi2 = f32x2_to_e4m3x2(bf16_to_f32(areg[i].w & 0xFFFF) / sh, bf16_to_f32(areg[i].w >> 16) / sh);
        q[2 * i] = lo | (hi << 16);
        q[2 * i + 1] = lo2 | (hi2 << 16);
      }
      ad[0] = make_uint4(q[0], q[1], q[2], q[3]);
      ad[1] = make_uint4(q[4], q[5], q[6], q[7]);
    } else {
      ad[0] = areg[0];
      ad[1] = areg[1];
    }
  };

  f32x16 acc[2] = {};
  const int brow[2] = {wn * 64, wn * 64 + 32};
  load_a(0);
  breg.load(w, wrow, I, 0, b_half);
  for (int k0 = 0; k0 < I; k0 += BK) {
    store_a();
    breg.store(Bs + b_row * P, b_half);
    __syncthreads();
    if (k0 + BK < I) {
      load_a(k0 + BK);
      breg.load(w, wrow, I, k0 + BK, b_half);
    }
    mma_slice<FP8ACT, 2>(As, Bs, wm * 32, brow, acc, lane);
    __syncthreads();
  }

  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[e];
  if constexpr (FP8ACT) f *= sh;
  const int j = lane & 31, g = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 8 * (r >> 2) + 4 * g + (r & 3);
    int tok, flat;
    if (!row_token(rows, b * kBM + wm * 32 + i, &tok, &flat)) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      o[static_cast<size_t>(flat) * H + n0 + brow[c] + j] = f32_to_bf16(acc[c][r] * f);
  }
}

template <int WFMT, bool FP8ACT>
static hipError_t run_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                             const uint32_t* amax_x, int H, int I, uint16_t* h, uint32_t* amax_h, hipStream_t s) {
  dim3 grid(I / kGateN, rows.num_blocks);
  gemm_gateup_kernel<WFMT, FP8ACT><<<grid, 256, 0, s>>>(w, rows, x, xq, amax_x, H, I, h, amax_h);
  return hipGetLastError();
}

template <int WFMT, bool FP8ACT>
static hipError_t run_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h, int H, int I,
                           uint16_t* o, hipStream_t s) {
  dim3 grid(H / kDownN, rows.num_blocks);
  gemm_down_kernel<WFMT, FP8ACT><<<grid, 256, 0, s>>>(w, rows, h, amax_h, H, I, o);
  return hipGetLastError();
}

hipError_t launch_gemm_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                              const uint32_t* amax_x, int H, int inter, uint16_t* h, uint32_t* amax_h,
                              hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_gateup<kMXFP4, false>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    case kNVFP4: return run_gateup<kNVFP4, false>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    case kFP8:
      return xq ? run_gateup<kFP8, true>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s)
                : run_gateup<kFP8, false>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h, int H,
                            int inter, uint16_t* o, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_down<kMXFP4, false>(w, rows, h, amax_h, H, inter, o, s);
    case kNVFP4: return run_down<kNVFP4, false>(w, rows, h, amax_h, H, inter, o, s);
    case kFP8:
      return amax_h ? run_down<kFP8, true>(w, rows, h, amax_h, H, inter, o, s)
                    : run_down<kFP8, false>(w, rows, h, amax_h, H, inter, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ftmoe
