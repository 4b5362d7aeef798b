// Token-to-expert alignment: count, prefix-sum, padded stable scatter.
//
// Flat row i = t*k + j of the routing table goes to expert ids[i] (entries
// outside [0, E) are ignored rather than trusted as addresses).  Each
// expert's rows are listed in ascending i, padded with the sentinel n = T*k
// up to a multiple of BM; block b of BM rows belongs to block_expert[b].
// The order is fixed by the definition (stable counting sort), so the result
// does not depend on thread timing.
//
// Small tables (n <= kAlignSmallN) use one workgroup.  Larger ones use three
// kernels: per-chunk histograms, one scan over (chunk, expert), and a
// per-chunk stable scatter where a wave ranks equal experts with lane reads.
#include <algorithm>

#include "align_dev.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kAlignSmallN = 1024;
constexpr int kAlignChunk = 1024;

static inline int max_padded(int T, int k, int E, int BM) {
  const long long n = static_cast<long long>(T) * k;
  const long long p = n + std::min<long long>(E, n) * (BM - 1);
  return static_cast<int>((p + BM - 1) / BM * BM);
}

// ---------------------------------------------------------- small table ---
__global__ __launch_bounds__(1024) void align_small_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                           int BM, int P, int32_t* counts,
                                                           int32_t* offsets, int32_t* sorted_ids,
                                                           int32_t* block_expert, int32_t* num_padded,
                                                           uint32_t* zero_words, int n_zero) {
  __shared__ int cnt[kAlignMaxE];
  __shared__ int ids_s[kAlignSmallN];
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  for (int i = e; i < n_zero; i += blockDim.x) zero_words[i] = 0u;
  cnt[e] = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ids_s[i] = ids[i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (static_cast<unsigned>(ids_s[i]) < static_cast<unsigned>(E)) atomicAdd(&cnt[ids_s[i]], 1);
  __syncthreads();
  const int c = e < E ? cnt[e] : 0;
  int off, total;
  finish_layout(e, E, c, BM, n, P, counts, offsets, sorted_ids, block_expert, num_padded, tmp, &off, &total);
  if (e < E && c > 0) {
    int pos = off;
    for (int i = 0; i < n; ++i)
      if (ids_s[i] == e) sorted_ids[pos++] = i;
  }
}

// ---------------------------------------------------------- large table ---
__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                         int32_t* __restrict__ hist,
                                                         uint32_t* zero_words, int n_zero) {
  __shared__ int cnt[kAlignMaxE];
  const int c = blockIdx.x;
  if (c == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero_words[i] = 0u;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int i0 = c * kAlignChunk, i1 = min(n, i0 + kAlignChunk);
  for (int i = i0 + threadIdx.x; i < i1; i += blockDim.x) {
    const int id = ids[i];
    if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) atomicAdd(&cnt[id], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[static_cast<size_t>(c) * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void align_scan_kernel(int n, int E, int BM, int P, int nchunks,
                                                          int32_t* __restrict__ hist, int32_t* counts,
                                                          int32_t* offsets, int32_t* sorted_ids,
                                                          int32_t* block_expert, int32_t* num_padded) {
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      int32_t* h = hist + static_cast<size_t>(c) * E + e;
      const int v = *h;
      *h = run;  // rows of expert e in earlier chunks
      run += v;
    }
  }
  int off, total;
  finish_layout(e, E, run, BM, n, P, counts, offsets, sorted_ids, block_expert, num_padded, tmp, &off, &total);
  if (e < E)
    for (int c = 0; c < nchunks; ++c) hist[static_cast<size_t>(c) * E + e] += off;
}

// One wave per chunk: rows are taken 64 at a time in index order; a row's
// slot is its expert's running position plus the number of earlier lanes in
// the same group with the same expert.
__global__ __launch_bounds__(64) void align_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                           const int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ sorted_ids) {
  __shared__ int run[kAlignMaxE];
  const int c = blockIdx.x;
  const int lane = lane_id();
  for (int e = lane; e < E; e += kWave) run[e] = hist[static_cast<size_t>(c) * E + e];
  __syncthreads();
  const int i0 = c * kAlignChunk, i1 = min(n, i0 + kAlignChunk);
  for (int g = i0; g < i1; g += kWave) {
    const int i = g + lane;
    int id = i < i1 ? ids[i] : -1;
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(E)) id = -1;  // ignored, as in the count
    const bool valid = id >= 0;
    int rank = 0, after = 0;
#pragma unroll 8
    for (int j = 0; j < kWave; ++j) {
      const int vj = __shfl(id, j, kWave);
      if (vj == id) {
        rank += j < lane ? 1 : 0;
        after += j > lane ? 1 : 0;
      }
    }
    int pos = 0;
    if (valid) pos = run[id] + rank;
    __syncthreads();
    if (valid) {
      sorted_ids[pos] = i;
      if (after == 0) run[id] = pos + 1;
    }
    __syncthreads();
  }
}

size_t align_scratch_bytes(int T, int k, int E, int BM) {
  (void)BM;
  const long long n = static_cast<long long>(T) * k;
  if (n <= kAlignSmallN) return 0;
  const long long nchunks = (n + kAlignChunk - 1) / kAlignChunk;
  return static_cast<size_t>(nchunks * E * 4);
}

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int BM, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* num_padded, void* scratch, uint32_t* zero_words, int n_zero,
                        hipStream_t s) {
  const int n = T * k;
  const int P = max_padded(T, k, E, BM);
  if (n <= kAlignSmallN) {
    align_small_kernel<<<1, 1024, 0, s>>>(ids, n, E, BM, P, counts, offsets, sorted_ids, block_expert,
                                          num_padded, zero_words, n_zero);
    return hipGetLastError();
  }
  const int nchunks = (n + kAlignChunk - 1) / kAlignChunk;
  int32_t* hist = static_cast<int32_t*>(scratch);
  align_hist_kernel<<<nchunks, 256, 0, s>>>(ids, n, E, hist, zero_words, n_zero);
  align_scan_kernel<<<1, 1024, 0, s>>>(n, E, BM, P, nchunks, hist, counts, offsets, sorted_ids,
                                       block_expert, num_padded);
  align_scatter_kernel<<<nchunks, 64, 0, s>>>(ids, n, E, hist, sorted_ids);
  return hipGetLastError();
}

}  // namespace ftmoe
