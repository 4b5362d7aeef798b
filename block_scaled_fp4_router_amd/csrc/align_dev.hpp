// Device helpers of the token-to-expert alignment, shared by the align
// kernels and the fused decode router.
#pragma once

#include "common.hpp"

namespace ftmoe {

constexpr int kAlignMaxE = 1024;

// Exclusive scan of `v` over a 1024-thread block (thread e holds v for expert e).
__device__ inline int block_exclusive_scan_1024(int v, int* tmp /* 32 ints */) {
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int s = lane < 16 ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o, kWave);
      if (lane >= o) s += y;
    }
    if (lane < 16) tmp[16 + lane] = s;
  }
  __syncthreads();
  const int base = wv > 0 ? tmp[16 + wv - 1] : 0;
  return base + x - v;
}

// Writes offsets, counts, num_padded, block ids and sentinels given counts in
// `cnt` (thread e handles expert e; blockDim = 1024, E <= 1024).  With
// `sentinels` false the caller has already filled sorted_ids with n.
__device__ inline void finish_layout(int e, int E, int c, int BM, int n, int P, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_ids, int32_t* block_expert,
                              int32_t* num_padded, int* tmp, int* off_out, int* total_out, bool sentinels = true) {
  const int padded = e < E ? (c + BM - 1) / BM * BM : 0;
  const int off = block_exclusive_scan_1024(padded, tmp);
  const int total = tmp[16 + 15];
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    if (sentinels)
      for (int p = off + c; p < off + padded; ++p) sorted_ids[p] = n;
    for (int b = off / BM; b < (off + padded) / BM; ++b) block_expert[b] = e;
  }
  if (e == 0) {
    offsets[E] = total;
    num_padded[0] = total;
  }
  if (sentinels)
    for (int p = total + threadIdx.x; p < P; p += blockDim.x) sorted_ids[p] = n;
  for (int b = total / BM + threadIdx.x; b < P / BM; b += blockDim.x) block_expert[b] = -1;
  *off_out = off;
  *total_out = total;
}

}  // namespace ftmoe
