// Router: logits l[t,e] = x_t . W_r[e] (fp32 accumulation of exact bf16 x
// and fp32 W_r), then per-token softmax top-k with renormalised weights and
// the shared expert's sigmoid gate.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

// ---------------------------------------------------------------- GEMV ----
// Few tokens: one wave per router row (row E is the shared-gate vector).
// Each lane walks H in float4 steps and keeps one partial per token.
constexpr int kGemvMaxT = 16;

template <int TMAX>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                          const float* __restrict__ router_w, int E,
                                                          const float* __restrict__ shared_gate_w,
                                                          float* __restrict__ logits) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = E + (shared_gate_w ? 1 : 0);
  if (row >= rows) return;
  const float* wrow = row < E ? router_w + static_cast<size_t>(row) * H : shared_gate_w;
  const int lane = lane_id();
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.f;
  for (int h = lane * 4; h < H; h += kWave * 4) {
    const float4 w = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + static_cast<size_t>(t) * H + h);
        acc[t] = fmaf(bf16_to_f32(xv.x & 0xFFFF), w.x, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv.x >> 16), w.y, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv.y & 0xFFFF), w.z, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv.y >> 16), w.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) logits[static_cast<size_t>(t) * (E + 1) + row] = v;
    }
  }
}

// ---------------------------------------------------------------- GEMM ----
// Many tokens: 64 tokens x 64 router rows per workgroup, fp32 FMA, operands
// staged through LDS in K slices of 32.  Each thread owns a 4x4 micro-tile.
constexpr int kRT = 64, kRE = 64, kRK = 32;

__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                          const float* __restrict__ router_w, int E,
                                                          const float* __restrict__ shared_gate_w,
                                                          float* __restrict__ logits) {
  __shared__ float xs[kRK][kRT + 4];
  __shared__ float wsh[kRK][kRE + 4];
  const int rows = E + (shared_gate_w ? 1 : 0);
  const int t0 = blockIdx.x * kRT, e0 = blockIdx.y * kRE;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // tx -> experts, ty -> tokens
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += kRK) {
    // x tile: 64 tokens x 32 k = 2048 bf16; each thread 8 consecutive k.
    {
      const int r = tid >> 2, c = (tid & 3) * 8;
      const int t = t0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < T) v = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + k0 + c);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xs[c + 2 * i][r] = bf16_to_f32(w4[i] & 0xFFFF);
        xs[c + 2 * i + 1][r] = bf16_to_f32(w4[i] >> 16);
      }
    }
    // W tile: 64 rows x 32 k fp32; each thread 8 consecutive k.
    {
      const int r = tid >> 2, c = (tid & 3) * 8;
      const int e = e0 + r;
      float4 a = make_float4(0, 0, 0, 0), b = a;
      if (e < rows) {
        const float* wrow = e < E ? router_w + static_cast<size_t>(e) * H : shared_gate_w;
        a = *reinterpret_cast<const float4*>(wrow + k0 + c);
        b = *reinterpret_cast<const float4*>(wrow + k0 + c + 4);
      }
      wsh[c + 0][r] = a.x; wsh[c + 1][r] = a.y; wsh[c + 2][r] = a.z; wsh[c + 3][r] = a.w;
      wsh[c + 4][r] = b.x; wsh[c + 5][r] = b.y; wsh[c + 6][r] = b.z; wsh[c + 7][r] = b.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kRK; ++kk) {
      float xa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wb[j] = wsh[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < rows) logits[static_cast<size_t>(t) * (E + 1) + e] = acc[i][j];
    }
  }
}

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* router_w, int E,
                                const float* shared_gate_w, float* logits, hipStream_t s) {
  const int rows = E + (shared_gate_w ? 1 : 0);
  if (T <= kGemvMaxT) {
    dim3 grid((rows + 3) / 4);
    if (T <= 1)
      router_gemv_kernel<1><<<grid, 256, 0, s>>>(x, T, H, router_w, E, shared_gate_w, logits);
    else if (T <= 4)
      router_gemv_kernel<4><<<grid, 256, 0, s>>>(x, T, H, router_w, E, shared_gate_w, logits);
    else
      router_gemv_kernel<kGemvMaxT><<<grid, 256, 0, s>>>(x, T, H, router_w, E, shared_gate_w, logits);
  } else {
    dim3 grid((T + kRT - 1) / kRT, (rows + kRE - 1) / kRE);
    router_gemm_kernel<<<grid, 256, 0, s>>>(x, T, H, router_w, E, shared_gate_w, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k ---
// One wave per token.  Lane l holds logits l, l+64, ...; k rounds of a wave
// argmax (larger value wins, equal values go to the lower index) remove the
// winner each round.  Weights: softmax over the k selected logits.
constexpr int kTopkMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   const float* __restrict__ bias, int has_shared,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   float* __restrict__ sgate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const float* row = logits + static_cast<size_t>(t) * (E + 1);
  float v[kTopkMaxPerLane];
#pragma unroll
  for (int i = 0; i < kTopkMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = -__builtin_inff();
    if (e < E) v[i] = row[e] + (bias ? bias[e] : 0.f);
  }
  float sel_v = 0.f;   // lane j < k keeps the j-th selected logit
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    // local best
    float bv = -__builtin_inff();
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kTopkMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (e < E && better(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
    }
    // wave argmax
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == j) { sel_v = bv; sel_i = bi; }
    if ((bi & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < kTopkMaxPerLane; ++i)
        if (lane + i * kWave == bi) v[i] = -__builtin_inff();
    }
  }
  const float m = __shfl(sel_v, 0, kWave);
  const float ex = lane < k ? expf(sel_v - m) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = sel_i;
    w[static_cast<size_t>(t) * k + lane] = ex / sum;
  }
  if (has_shared && lane == 0) {
    const float g = row[E];
    sgate[t] = 1.0f / (1.0f + expf(-g));
  }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, const float* bias, bool has_shared,
                       int32_t* ids, float* w, float* sgate, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  topk_kernel<<<grid, 256, 0, s>>>(logits, T, E, k, bias, has_shared ? 1 : 0, ids, w, sgate);
  return hipGetLastError();
}

}  // namespace ftmoe
