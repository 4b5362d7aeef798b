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
// per-chunk stable scatter where waves rank equal experts with ballots.
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
  __shared__ __attribute__((aligned(16))) int ids_s[kAlignSmallN];
  __shared__ int tmp[32];
  const int e = threadIdx.x;
  for (int i = e; i < n_zero; i += blockDim.x) zero_words[i] = 0u;
  // every sorted slot starts as the sentinel (coalesced); the routed rows'
  // slots are overwritten at the end, after several barriers
  for (int i = e; i < P; i += blockDim.x) sorted_ids[i] = n;
  cnt[e] = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ids_s[i] = ids[i];
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    if (static_cast<unsigned>(ids_s[i]) < static_cast<unsigned>(E)) atomicAdd(&cnt[ids_s[i]], 1);
  __syncthreads();
  const int c = e < E ? cnt[e] : 0;
  int off, total;
  finish_layout(e, E, c, BM, n, P, counts, offsets, sorted_ids, block_expert, num_padded, tmp, &off, &total, false);
  if (e < E) cnt[e] = off;   // the counts are no longer needed: reuse as segment starts
  __syncthreads();
  // row i goes after the earlier rows of its expert (stable counting sort);
  // ignored ids (outside [0, E)) are neither counted nor placed
  if (threadIdx.x < n) {
    const int i = threadIdx.x;
    const int id = ids_s[i];
    if (static_cast<unsigned>(id) < static_cast<unsigned>(E)) {
      int rank = 0;
      for (int j0 = 0; j0 < i; j0 += 4) {
        const int4 v = *reinterpret_cast<const int4*>(&ids_s[j0]);
        rank += (v.x == id) + (j0 + 1 < i && v.y == id) + (j0 + 2 < i && v.z == id) + (j0 + 3 < i && v.w == id);
      }
      sorted_ids[cnt[id] + rank] = i;
    }
  }
}

// ---------------------------------------------------------- large table ---
// Per-chunk histograms; the workgroups also fill sorted_ids [0, P) with the
// sentinel n (the scatter overwrites the routed rows' entries), so that the
// one-workgroup scan writes no padding.
__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                         int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids,
                                                         int P, uint32_t* zero_words, int n_zero) {
  __shared__ int cnt[kAlignMaxE];
  const int c = blockIdx.x;
  if (c == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero_words[i] = 0u;
  for (int i = c * blockDim.x + threadIdx.x; i < P; i += gridDim.x * blockDim.x) sorted_ids[i] = n;
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

// Exclusive prefix of the per-chunk histograms over chunks, per expert, plus
// the layout.  The 1024 threads are split into parts = 1024 / E groups of E
// (one thread per expert and part); each part owns a contiguous range of
// chunks.  A thread loads up to kScanCache of its histogram entries at once
// and keeps them in registers for the second pass, so the histogram is read
// once, with all loads in flight together.
constexpr int kScanCache = 40;

__global__ __launch_bounds__(1024) void align_scan_kernel(int n, int E, int BM, int P, int nchunks,
                                                          int32_t* __restrict__ hist, int32_t* counts,
                                                          int32_t* offsets, int32_t* sorted_ids,
                                                          int32_t* block_expert, int32_t* num_padded) {
  __shared__ int tmp[32];
  __shared__ int part_base[1024];
  __shared__ int exp_off[kAlignMaxE];
  const int tid = threadIdx.x;
  const int parts = E < 1024 ? 1024 / E : 1;
  const int e = tid % E, p = tid / E;
  const bool worker = p < parts;
  const int per = (nchunks + parts - 1) / parts;
  const int c0 = min(nchunks, p * per), c1 = min(nchunks, c0 + per);
  const int ncached = min(c1 - c0, kScanCache);
  // 1. each part's sum
  int v[kScanCache];
  int sum = 0;
  if (worker) {
#pragma unroll
    for (int u = 0; u < kScanCache; ++u) v[u] = u < ncached ? hist[static_cast<size_t>(c0 + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kScanCache; ++u) sum += v[u];
    for (int c = c0 + kScanCache; c < c1; ++c) sum += hist[static_cast<size_t>(c) * E + e];
    part_base[tid] = sum;
  }
  __syncthreads();
  // 2. per expert: exclusive prefix over its parts, total
  int total_e = 0;
  if (tid < E) {
    for (int q = 0; q < parts; ++q) {
      const int x = part_base[q * E + tid];
      part_base[q * E + tid] = total_e;
      total_e += x;
    }
  }
  __syncthreads();
  // 3. layout (thread e = expert e)
  int off, total;
  finish_layout(tid, E, tid < E ? total_e : 0, BM, n, P, counts, offsets, sorted_ids, block_expert, num_padded,
                tmp, &off, &total, false);
  if (tid < E) exp_off[tid] = off;
  __syncthreads();
  // 4. every (chunk, expert) entry becomes the expert's first slot for that chunk
  if (worker) {
    int base = exp_off[e] + part_base[tid];
#pragma unroll
    for (int u = 0; u < kScanCache; ++u) {
      if (u < ncached) {
        hist[static_cast<size_t>(c0 + u) * E + e] = base;
        base += v[u];
      }
    }
    for (int c = c0 + kScanCache; c < c1; ++c) {
      const int x = hist[static_cast<size_t>(c) * E + e];
      hist[static_cast<size_t>(c) * E + e] = base;
      base += x;
    }
  }
}

// Four waves per chunk.  The chunk's rows are taken 256 at a time in index
// order, wave w on rows [64 w, 64 w + 64) of each group.  Within a wave the
// lanes with the same expert are found with one ballot per bit of the id;
// the last lane of each such group records the wave's count of that expert,
// so a row's slot is its expert's running position, plus the rows of that
// expert in the earlier waves of the group, plus the earlier lanes of its
// own group.  The records are cleared by the lanes that wrote them.
constexpr int kScatterWaves = 4;

__global__ __launch_bounds__(64 * kScatterWaves) void align_scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                                           int E, const int32_t* __restrict__ hist,
                                                                           int32_t* __restrict__ sorted_ids) {
  __shared__ int run[kAlignMaxE];
  __shared__ int wcnt[kScatterWaves][kAlignMaxE];
  const int c = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    run[e] = hist[static_cast<size_t>(c) * E + e];
#pragma unroll
    for (int w = 0; w < kScatterWaves; ++w) wcnt[w][e] = 0;
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = (uint64_t{1} << lane) - 1;
  __syncthreads();
  const int i0 = c * kAlignChunk, i1 = min(n, i0 + kAlignChunk);
  for (int g = i0; g < i1; g += 64 * kScatterWaves) {
    const int i = g + 64 * wave + lane;
    int id = i < i1 ? ids[i] : -1;
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(E)) id = -1;  // ignored, as in the count
    const bool valid = id >= 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (id >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    const bool last = valid && (peers >> lane) == 1;
    if (last) wcnt[wave][id] = __popcll(peers);
    __syncthreads();
    int before = 0, group = 0;
    if (valid) {
#pragma unroll
      for (int w = 0; w < kScatterWaves; ++w) {
        const int x = wcnt[w][id];
        before += w < wave ? x : 0;
        group += x;
      }
      sorted_ids[run[id] + before + rank] = i;
    }
    __syncthreads();
    // the last wave holding the expert advances its running position; each
    // record is cleared by the lane that wrote it
    if (last) {
      bool later = false;
#pragma unroll
      for (int w = 0; w < kScatterWaves; ++w) later |= w > wave && wcnt[w][id] != 0;
      if (!later) run[id] += group;
    }
    __syncthreads();
    if (last) wcnt[wave][id] = 0;
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
  align_hist_kernel<<<nchunks, 256, 0, s>>>(ids, n, E, hist, sorted_ids, P, zero_words, n_zero);
  align_scan_kernel<<<1, 1024, 0, s>>>(n, E, BM, P, nchunks, hist, counts, offsets, sorted_ids,
                                       block_expert, num_padded);
  align_scatter_kernel<<<nchunks, 64 * kScatterWaves, 0, s>>>(ids, n, E, hist, sorted_ids);
  return hipGetLastError();
}

}  // namespace ftmoe
