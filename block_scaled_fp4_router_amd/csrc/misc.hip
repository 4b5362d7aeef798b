// Per-tensor E4M3 activation quantisation and the weighted combine.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
  zero_u32_kernel<<<1, 64, 0, s>>>(p, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ amax(|x|) ---
// Non-negative floats order like their bit patterns, so the running maximum
// is an unsigned atomicMax on the bits.
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                        uint32_t* amax_bits) {
  const int64_t n8 = n / 8;
  float m = 0.f;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n8;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_to_f32(w[j] & 0xFFFF)));
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_to_f32(w[j] >> 16)));
    }
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += blockDim.x)
      m = __builtin_fmaxf(m, __builtin_fabsf(bf16_to_f32(x[i])));
  __shared__ float red[16];
  m = wave_max_fast(m);
  if (lane_id() == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = 0.f;
    for (int i = 0; i < static_cast<int>(blockDim.x >> 6); ++i) r = __builtin_fmaxf(r, red[i]);
    atomicMax(amax_bits, __float_as_uint(r));
  }
}

// Folds the kAmaxSlots partial maxima into one word.
__global__ void amax_fold_kernel(const uint32_t* __restrict__ slots, uint32_t* __restrict__ out) {
  const int l = lane_id();
  uint32_t v = l < kAmaxSlots ? slots[l * kAmaxStride] : 0u;
  const float m = wave_max_fast(__uint_as_float(v));
  if (l == 0) *out = __float_as_uint(m);
}

hipError_t launch_amax_fold(const uint32_t* slots, uint32_t* out, hipStream_t s) {
  return launch(amax_fold_kernel, dim3(1), dim3(64), 0, s, slots, out);
}

// s = amax / 448 (1 when amax is 0), the dequantisation scale.
__device__ __forceinline__ float fp8_scale_from_amax(uint32_t bits) {
  const float a = __uint_as_float(bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// NT: the source is read with the non-temporal hint (large sources, read
// once: the bf16 h of the FP8 layers).
template <bool NT>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                        const uint32_t* __restrict__ amax_bits,
                                                        uint8_t* __restrict__ q, float* scale_out) {
  const float s = fp8_scale_from_amax(*amax_bits);
  const int64_t n8 = n / 8;
  const int64_t i0 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i0 == 0 && scale_out) *scale_out = s;
  for (int64_t i = i0; i < n8; i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    uint4 v;
    if constexpr (NT) {
      const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + i);
      v = make_uint4(u.x, u.y, u.z, u.w);
    } else {
      v = reinterpret_cast<const uint4*>(x)[i];
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t lo = f32x2_to_e4m3x2(bf16_to_f32(w[2 * j] & 0xFFFF) / s, bf16_to_f32(w[2 * j] >> 16) / s);
      const uint32_t hi = f32x2_to_e4m3x2(bf16_to_f32(w[2 * j + 1] & 0xFFFF) / s, bf16_to_f32(w[2 * j + 1] >> 16) / s);
      out[j] = lo | (hi << 16);
    }
    reinterpret_cast<uint2*>(q)[i] = make_uint2(out[0], out[1]);
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += blockDim.x)
      q[i] = static_cast<uint8_t>(f32x2_to_e4m3x2(bf16_to_f32(x[i]) / s, 0.f) & 0xFF);
}

static int elementwise_grid(int64_t n8, int64_t cap = 4096) {
  int64_t g = (n8 + 255) / 256;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, uint32_t* amax_bits, hipStream_t s) {
  return launch(amax_bf16_kernel, dim3(elementwise_grid(n / 8, 512)), dim3(256), 0, s, x, n, amax_bits);
}

// Sources larger than this are read with the non-temporal hint (measured
// faster once they exceed the Infinity Cache, slightly slower below it).
constexpr int64_t kStreamNtBytes = int64_t{192} << 20;

hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, const uint32_t* amax_bits, uint8_t* q,
                            float* scale_out, hipStream_t s) {
  const dim3 grid(elementwise_grid(n / 8));
  if (n * static_cast<int64_t>(sizeof(uint16_t)) > kStreamNtBytes)
    return launch(quant_fp8_kernel<true>, grid, dim3(256), 0, s, x, n, amax_bits, q, scale_out);
  return launch(quant_fp8_kernel<false>, grid, dim3(256), 0, s, x, n, amax_bits, q, scale_out);
}

// -------------------------------------------------------------- combine ---
// One thread per 8 outputs: y[t, n:n+8] = sum_j w[t,j] o[t*k+j, n:n+8]
// (+ sg[t] * sh[t, n:n+8]), fp32 sums in ascending j, bf16 nearest-even.
// Every row's load is issued before the sums (MAXK >= k rows, unrolled), so
// the k loads of a thread are in flight together.  NT: the expert outputs
// are read with the non-temporal hint (each is read once; measured 20%
// faster when they exceed the Infinity Cache, slightly slower below it).
template <int MAXK, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o,
                                                      const float* __restrict__ w, int T, int k, int H,
                                                      const float* __restrict__ sg,
                                                      const uint16_t* __restrict__ sh,
                                                      uint16_t* __restrict__ y) {
  const int per_row = H / 8;
  const int64_t idx = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (idx >= static_cast<int64_t>(T) * per_row) return;
  const int t = static_cast<int>(idx / per_row);
  const int c = static_cast<int>(idx % per_row) * 8;
  uint4 v[MAXK];
  float wj[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j < k) {
      wj[j] = w[static_cast<size_t>(t) * k + j];
      const uint16_t* src = o + (static_cast<size_t>(t) * k + j) * H + c;
      if constexpr (NT) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        v[j] = make_uint4(q.x, q.y, q.z, q.w);
      } else {
        v[j] = *reinterpret_cast<const uint4*>(src);
      }
    }
  }
  float acc[8] = {};
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j < k) {
      const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj[j], bf16_to_f32(u[i] & 0xFFFF), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj[j], bf16_to_f32(u[i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  if (sg) {
    const float g = sg[t];
    const uint4 q = *reinterpret_cast<const uint4*>(sh + static_cast<size_t>(t) * H + c);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(g, bf16_to_f32(u[i] & 0xFFFF), acc[2 * i]);
      acc[2 * i + 1] = fmaf(g, bf16_to_f32(u[i] >> 16), acc[2 * i + 1]);
    }
  }
  uint4 r;
  r.x = pack_bf16x2(acc[0], acc[1]);
  r.y = pack_bf16x2(acc[2], acc[3]);
  r.z = pack_bf16x2(acc[4], acc[5]);
  r.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(y + static_cast<size_t>(t) * H + c) = r;
}

hipError_t launch_combine(const uint16_t* o, const float* w, int T, int k, int H, const float* sg,
                          const uint16_t* sh, uint16_t* y, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(T) * (H / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  const bool nt = static_cast<int64_t>(T) * k * H * static_cast<int64_t>(sizeof(uint16_t)) > kStreamNtBytes;
  if (k <= 8)
    return nt ? launch(combine_kernel<8, true>, grid, dim3(256), 0, s, o, w, T, k, H, sg, sh, y)
              : launch(combine_kernel<8, false>, grid, dim3(256), 0, s, o, w, T, k, H, sg, sh, y);
  return nt ? launch(combine_kernel<16, true>, grid, dim3(256), 0, s, o, w, T, k, H, sg, sh, y)
            : launch(combine_kernel<16, false>, grid, dim3(256), 0, s, o, w, T, k, H, sg, sh, y);
}

// ------------------------------------------------- expert-slot pool fill ---
// Work units of kFillUnit bytes of one array of one expert; 256 threads move
// a unit as 16-byte words (4 in flight per thread) when the array's
// per-expert size and both bases allow it, else as 4-byte words.
constexpr uint32_t kFillUnit = 64u << 10;

__global__ __launch_bounds__(256) void expert_fill_kernel(FillArgs a) {
  uint32_t units[kFillArrays], per_expert = 0;
#pragma unroll
  for (int j = 0; j < kFillArrays; ++j) {
    units[j] = (a.bytes[j] + kFillUnit - 1) / kFillUnit;
    per_expert += units[j];
  }
  const uint32_t total = per_expert * static_cast<uint32_t>(a.n);
  for (uint32_t u = blockIdx.x; u < total; u += gridDim.x) {
    const int m = static_cast<int>(u / per_expert);
    uint32_t r = u % per_expert;
    int j = 0;
    while (r >= units[j]) r -= units[j++];
    const size_t b = a.bytes[j];
    const uint8_t* src = a.src[j] + static_cast<size_t>(a.e[m]) * b;
    uint8_t* dst = a.dst[j] + static_cast<size_t>(a.s[m]) * b;
    const uint32_t lo = r * kFillUnit, hi = min(static_cast<uint32_t>(b), lo + kFillUnit);
    const bool vec = (b % 16 == 0) && ((reinterpret_cast<uintptr_t>(a.src[j]) | reinterpret_cast<uintptr_t>(a.dst[j])) % 16 == 0);
    if (vec) {
      const uint4* s4 = reinterpret_cast<const uint4*>(src + lo);
      uint4* d4 = reinterpret_cast<uint4*>(dst + lo);
      const uint32_t n4 = (hi - lo) / 16;
      for (uint32_t i = threadIdx.x; i < n4; i += 4 * 256) {
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (i + q * 256 < n4) v[q] = s4[i + q * 256];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (i + q * 256 < n4) d4[i + q * 256] = v[q];
      }
    } else {
      const uint32_t* s1 = reinterpret_cast<const uint32_t*>(src + lo);
      uint32_t* d1 = reinterpret_cast<uint32_t*>(dst + lo);
      for (uint32_t i = threadIdx.x; i < (hi - lo) / 4; i += 256) d1[i] = s1[i];
    }
  }
}

hipError_t launch_expert_fill(const FillArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  // 64 workgroups keep enough reads in flight to fill the link and leave the
  // other compute units to the kernels of the pass that overlaps the fill.
  expert_fill_kernel<<<64, 256, 0, s>>>(a);
  return hipGetLastError();
}

// --------------------------------------------------- host rows scatter ---
__global__ __launch_bounds__(256) void host_rows_scatter_kernel(const float* __restrict__ rows,
                                                                const int32_t* __restrict__ flat, int H,
                                                                float* o32, uint16_t* o16) {
  const int r = blockIdx.x;
  const size_t f = static_cast<size_t>(flat[r]);
  const float4* src = reinterpret_cast<const float4*>(rows + static_cast<size_t>(r) * H);
  for (int c = threadIdx.x; c < H / 4; c += 256) {
    const float4 v = src[c];
    if (o32) {
      reinterpret_cast<float4*>(o32 + f * H)[c] = v;
    } else {
      reinterpret_cast<uint2*>(o16 + f * H)[c] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
  }
}

hipError_t launch_host_rows_scatter(const float* rows, const int32_t* flat, int n, int H, float* o32, uint16_t* o16,
                                    hipStream_t s) {
  if (n <= 0) return hipSuccess;
  host_rows_scatter_kernel<<<n, 256, 0, s>>>(rows, flat, H, o32, o16);
  return hipGetLastError();
}

}  // namespace ftmoe
