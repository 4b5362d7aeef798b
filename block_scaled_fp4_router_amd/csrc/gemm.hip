// Prefill experts: grouped GEMMs over the expert-sorted row blocks.
//
// A workgroup is 8 waves over one (row block, column tile): BM token rows of
// one expert (BM = 128 or 64) times a tile of the expert's weight rows.  Each
// wave owns a 64 x 64 output tile (2 x 2 MFMA tiles of 32 x 32); the waves are
// laid out BM/64 along rows and 8 / (BM/64) along columns.
//   gate_up: a wave's two column tiles are 32 gate rows and the 32 matching up
//            rows, so h = silu(gate) * up is formed in registers;
//   down:    a wave's two column tiles are 64 consecutive output columns.
//
// K advances in stages of 64.  Activation rows (gathered through the sorted
// row ids) are staged through LDS, double-buffered, with their 16-byte
// vectors XOR-swizzled by row so that the 8 lanes of a ds_read_b128 phase hit
// 8 different bank groups.  Weights never touch LDS: each wave loads its own
// column tiles straight into registers one stage ahead and dequantises them
// right before the MFMA (MXFP4 with the E8M0-scaled hardware convert, NVFP4
// as E2M1 x E4M3, exact in bf16), feeding v_mfma_f32_32x32x16_bf16.  FP8
// weights with FP8 activations feed v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// scales and need no conversion at all; tensor and activation scales are
// applied in the epilogue.
//
// Within a stage, lane group g (lane / 32) of the bf16 MFMA takes K elements
// [32g + 8t, 32g + 8t + 8) at MFMA step t: both operands use this assignment,
// so a lane's weight bytes for the stage are one contiguous 16-byte run (one
// FP4 block scale per MXFP4 lane, two for NVFP4).
//
// Workgroups are numbered so that each XCD (workgroup w runs on XCD w % 8)
// receives a contiguous range of (block, tile) pairs: the column tiles of a
// row block, and the row blocks of one expert, then share that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kStageK = 64;

template <int BM>
struct TileShape {
  static constexpr int kWM = BM / 64;              // waves along rows
  static constexpr int kWN = kGemmWaves / kWM;     // waves along columns
  static constexpr int kBN = 64 * kWN;             // weight rows per workgroup
};

int gemm_block_m(int T, int k, int E) {
  // Small experts (few rows each) waste less padding with 64-row blocks.
  return static_cast<long long>(T) * k >= 192LL * E ? 128 : 64;
}

// ------------------------------------------------------------ helpers -----
__device__ __forceinline__ int logical_tile(int w, int total) {
  const int per = (total + 7) >> 3;
  return (w & 7) * per + (w >> 3);
}

// Position of vector q in an LDS row of V 16-byte vectors (V = 8 or 4).
template <int V>
__device__ __forceinline__ int swz(int r, int q) {
  if constexpr (V == 8)
    return q ^ (r & 7);
  else
    return q ^ ((r >> 1) & 3);
}

// Valid rows of block b: routed blocks end where their expert's segment does.
__device__ __forceinline__ int block_rows(const Rows& rows, int b, int e, int BM) {
  if (!rows.sorted_ids) {
    const int n = rows.n_flat - b * BM;
    return n < BM ? n : BM;
  }
  const int n = rows.offsets[e] + rows.counts[e] - b * BM;
  return n < BM ? n : BM;
}

__device__ __forceinline__ float amax_scale(const uint32_t* bits) {
  const float a = __uint_as_float(*bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// ------------------------------------------------------- weight slices ----
// One lane's part of one 32-row column tile for one stage.
template <int WFMT, bool FP8ACT>
struct BSlice {
  uint4 c0, c1;   // FP4: c0 only (32 nibbles); FP8: 32 bytes
  uint32_t sc;    // MXFP4: E8M0 byte; NVFP4: two E4M3 bytes
};

template <int WFMT, bool FP8ACT>
__device__ __forceinline__ void load_bslice(BSlice<WFMT, FP8ACT>& s, const QW& w, size_t row, int K, int k0, int g) {
  if constexpr (WFMT == kFP8) {
    const uint8_t* p = w.codes + row * K + k0;
    if constexpr (FP8ACT) {
      // hardware 8-bit operand layout: bytes [16g, 16g+16) and [32+16g, ...)
      s.c0 = load_nt(p + 16 * g);
      s.c1 = load_nt(p + 32 + 16 * g);
    } else {
      s.c0 = load_nt(p + 32 * g);
      s.c1 = load_nt(p + 32 * g + 16);
    }
    s.sc = 0;
  } else {
    s.c0 = load_nt(w.codes + row * (K / 2) + k0 / 2 + 16 * g);
    if constexpr (WFMT == kMXFP4)
      s.sc = w.scales[row * (K / 32) + k0 / 32 + g];
    else
      s.sc = *reinterpret_cast<const uint16_t*>(w.scales + row * (K / 16) + k0 / 16 + 2 * g);
  }
}

// bf16 operand of MFMA step t (elements [32g + 8t, +8) of the stage).
template <int WFMT, bool FP8ACT>
__device__ __forceinline__ bf16x8 bslice_bf16(const BSlice<WFMT, FP8ACT>& s, int t) {
  uint32_t o[4];
  if constexpr (WFMT == kFP8) {
    const uint4 c = t < 2 ? s.c0 : s.c1;
    const uint32_t w0 = (t & 1) ? c.z : c.x, w1 = (t & 1) ? c.w : c.y;
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
    const f32x2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
    o[0] = pack_bf16x2(a[0], a[1]);
    o[1] = pack_bf16x2(b[0], b[1]);
    o[2] = pack_bf16x2(c2[0], c2[1]);
    o[3] = pack_bf16x2(d[0], d[1]);
  } else {
    const uint32_t word = t == 0 ? s.c0.x : t == 1 ? s.c0.y : t == 2 ? s.c0.z : s.c0.w;
    if constexpr (WFMT == kMXFP4)
      fp4x8_to_bf16(word, e8m0_as_scale(s.sc), o);
    else
      fp4x8_to_bf16_mul(word, e4m3_to_f32((s.sc >> (t < 2 ? 0 : 8)) & 0xFF), o);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ i32x8 u4x2(const uint4& p, const uint4& q) {
  return i32x8{static_cast<int>(p.x), static_cast<int>(p.y), static_cast<int>(p.z), static_cast<int>(p.w),
               static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w)};
}

// ---------------------------------------------------- activation staging --
// LDS stage: BM rows of one K stage, V vectors of 16 bytes per row (bf16: 8,
// FP8: 4).  Thread tid stages vectors tid, tid + 512, ... of the row-major
// sequence; a thread's rows are fixed for the whole K loop.
template <int BM, bool FP8ROWS>
struct AStage {
  static constexpr int V = FP8ROWS ? 4 : 8;
  static constexpr int kVecs = BM * V;
  static constexpr int kPer = (kVecs + kGemmThreads - 1) / kGemmThreads;
  static constexpr int kBytes = BM * V * 16;
};

// bf16 source rows (gate_up from x, down from h) or FP8 rows (gate_up from x_q).
template <int BM, bool FP8ROWS, bool QUANT>
struct ALoader {
  using S = AStage<BM, FP8ROWS>;
  const uint8_t* src[S::kPer];   // row start + this thread's vector (advances per stage)
  int dst[S::kPer];              // LDS byte offset within a stage buffer (-1: none)
  uint4 v[S::kPer][QUANT ? 2 : 1];

  __device__ __forceinline__ void issue() {
#pragma unroll
    for (int j = 0; j < S::kPer; ++j) {
      if (dst[j] < 0) continue;
      const uint4* p = reinterpret_cast<const uint4*>(src[j]);
      v[j][0] = p[0];
      if constexpr (QUANT) v[j][1] = p[1];
      src[j] += QUANT ? 2 * kStageK : (FP8ROWS ? kStageK : 2 * kStageK);
    }
  }

  __device__ __forceinline__ void store(uint8_t* buf, float sh) const {
#pragma unroll
    for (int j = 0; j < S::kPer; ++j) {
      if (dst[j] < 0) continue;
      uint4 o = v[j][0];
      if constexpr (QUANT) {
        const uint32_t w[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w,
                               v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = f32x2_to_e4m3x2(bf16_to_f32(w[2 * i] & 0xFFFF) / sh, bf16_to_f32(w[2 * i] >> 16) / sh);
          const uint32_t hi =
              f32x2_to_e4m3x2(bf16_to_f32(w[2 * i + 1] & 0xFFFF) / sh, bf16_to_f32(w[2 * i + 1] >> 16) / sh);
          q[i] = lo | (hi << 16);
        }
        o = make_uint4(q[0], q[1], q[2], q[3]);
      }
      *reinterpret_cast<uint4*>(buf + dst[j]) = o;
    }
  }
};

// Sets up the loader for rows whose start addresses row_ptr(r) gives (bytes
// per element: 2 for bf16 sources, 1 for FP8 sources).
template <int BM, bool FP8ROWS, bool QUANT, class RowPtr>
__device__ __forceinline__ void aloader_init(ALoader<BM, FP8ROWS, QUANT>& L, RowPtr row_ptr) {
  using S = AStage<BM, FP8ROWS>;
#pragma unroll
  for (int j = 0; j < S::kPer; ++j) {
    const int i = threadIdx.x + j * kGemmThreads;
    if (i >= S::kVecs) {
      L.dst[j] = -1;
      L.src[j] = nullptr;
      continue;
    }
    const int r = i / S::V, q = i % S::V;
    L.dst[j] = r * (S::V * 16) + 16 * swz<S::V>(r, q);
    // source bytes of vector q of the stage: FP8 rows 16 per vector; bf16
    // rows 16 per vector, or 32 when two bf16 vectors quantise into one
    L.src[j] = static_cast<const uint8_t*>(row_ptr(r)) + q * (QUANT ? 32 : 16);
  }
}

// ------------------------------------------------------------- compute ----
// One stage of a wave's 64 x 64 tile: acc[m][c] over rows 32m.. of the wave,
// column tile c.  rows_ok[m]: M-tile m holds at least one valid row.
template <int WFMT, bool FP8ACT, int V>
__device__ __forceinline__ void mma_stage(const uint8_t* As, int arow0, const BSlice<WFMT, FP8ACT> (&bs)[2],
                                          const bool (&rows_ok)[2], f32x16 (&acc)[2][2], int lane) {
  const int i = lane & 31, g = lane >> 5;
  if constexpr (FP8ACT) {
    const i32x8 b0 = u4x2(bs[0].c0, bs[0].c1), b1 = u4x2(bs[1].c0, bs[1].c1);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (!rows_ok[m]) continue;
      const int r = arow0 + 32 * m + i;
      const uint8_t* row = As + r * (V * 16);
      const i32x8 a = u4x2(*reinterpret_cast<const uint4*>(row + 16 * swz<V>(r, g)),
                           *reinterpret_cast<const uint4*>(row + 16 * swz<V>(r, 2 + g)));
      acc[m][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b0, acc[m][0], 0, 0, 0, 127, 0, 127);
      acc[m][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b1, acc[m][1], 0, 0, 0, 127, 0, 127);
    }
  } else {
    // all A fragments of the stage first, so the LDS reads overlap
    bf16x8 a[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = arow0 + 32 * m + i;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        a[m][t] = __builtin_bit_cast(bf16x8,
                                     *reinterpret_cast<const uint4*>(As + r * (V * 16) + 16 * swz<V>(r, 4 * g + t)));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 b0 = bslice_bf16(bs[0], t), b1 = bslice_bf16(bs[1], t);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (!rows_ok[m]) continue;
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m][t], b0, acc[m][0], 0, 0, 0);
        acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m][t], b1, acc[m][1], 0, 0, 0);
      }
    }
  }
}

// The K loop shared by both GEMMs: activations staged double-buffered in LDS,
// weights one stage ahead in registers.
template <int WFMT, bool FP8ACT, int BM, bool FP8ROWS, bool QUANT>
__device__ __forceinline__ void k_loop(ALoader<BM, FP8ROWS, QUANT>& L, uint8_t* As0, uint8_t* As1, const QW& w,
                                       const size_t (&wrow)[2], int K, int arow0, const bool (&rows_ok)[2],
                                       float sh, f32x16 (&acc)[2][2], int lane) {
  constexpr int V = AStage<BM, FP8ROWS>::V;
  const int g = lane >> 5;
  const int ns = K / kStageK;
  BSlice<WFMT, FP8ACT> b0[2], b1[2];
  L.issue();
#pragma unroll
  for (int c = 0; c < 2; ++c) load_bslice(b0[c], w, wrow[c], K, 0, g);
  L.store(As0, sh);
  if (ns > 1) {
    L.issue();
#pragma unroll
    for (int c = 0; c < 2; ++c) load_bslice(b1[c], w, wrow[c], K, kStageK, g);
  }
  __syncthreads();
  for (int s = 0; s < ns; s += 2) {
    // stage s from As0 / b0
    mma_stage<WFMT, FP8ACT, V>(As0, arow0, b0, rows_ok, acc, lane);
    if (s + 1 < ns) L.store(As1, sh);
    if (s + 2 < ns) {
      L.issue();
#pragma unroll
      for (int c = 0; c < 2; ++c) load_bslice(b0[c], w, wrow[c], K, (s + 2) * kStageK, g);
    }
    __syncthreads();
    if (s + 1 >= ns) break;
    // stage s + 1 from As1 / b1
    mma_stage<WFMT, FP8ACT, V>(As1, arow0, b1, rows_ok, acc, lane);
    if (s + 2 < ns) L.store(As0, sh);
    if (s + 3 < ns) {
      L.issue();
#pragma unroll
      for (int c = 0; c < 2; ++c) load_bslice(b1[c], w, wrow[c], K, (s + 3) * kStageK, g);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- gate_up ----
template <int WFMT, bool FP8ACT, int BM>
__global__ __launch_bounds__(kGemmThreads) void gemm_gateup_kernel(QW w, Rows rows, const uint16_t* __restrict__ x,
                                                                   const uint8_t* __restrict__ xq,
                                                                   const uint32_t* __restrict__ amax_x, int H, int I,
                                                                   uint16_t* __restrict__ h,
                                                                   uint32_t* __restrict__ amax_h) {
  using TS = TileShape<BM>;
  constexpr int kStageBytes = AStage<BM, FP8ACT>::kBytes;
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * kStageBytes];
  __shared__ float red[kGemmWaves];

  const int ntile = (I + TS::kBN / 2 - 1) / (TS::kBN / 2);
  const int t = logical_tile(blockIdx.x, rows.num_blocks * ntile);
  if (t >= rows.num_blocks * ntile) return;
  const int b = t / ntile, nt = t % ntile;
  const int e = rows.sorted_ids ? rows.block_expert[b] : 0;
  if (e < 0) return;
  const int nvalid = block_rows(rows, b, e, BM);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int wm = wave % TS::kWM, wn = wave / TS::kWM;
  const int arow0 = wm * 64;
  const int n0 = nt * (TS::kBN / 2) + wn * 32;   // this wave's first gate column
  const bool wact = n0 < I;                      // a last tile may reach past I
  const bool rows_ok[2] = {wact && arow0 < nvalid, wact && arow0 + 32 < nvalid};
  const int j = lane & 31, g = lane >> 5;
  const int nw0 = wact ? n0 : 0;                 // idle waves stream a valid row, unused
  const size_t wrow[2] = {static_cast<size_t>(e) * (2 * I) + nw0 + j, static_cast<size_t>(e) * (2 * I) + I + nw0 + j};

  ALoader<BM, FP8ACT, false> L;
  aloader_init(L, [&](int r) -> const void* {
    const int p = b * BM + r;
    int tok = 0;
    if (rows.sorted_ids) {
      const int f = rows.sorted_ids[p];
      tok = f < rows.n_flat ? f / rows.top_k : 0;
    } else {
      tok = p < rows.n_flat ? p : 0;
    }
    if constexpr (FP8ACT)
      return xq + static_cast<size_t>(tok) * H;
    else
      return x + static_cast<size_t>(tok) * H;
  });

  f32x16 acc[2][2] = {};
  k_loop<WFMT, FP8ACT, BM, FP8ACT, false>(L, As, As + kStageBytes, w, wrow, H, arow0, rows_ok, 1.0f, acc, lane);

  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[e];
  if constexpr (FP8ACT) f *= amax_scale(amax_x);
  float mx = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = arow0 + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
      if (!wact || i >= nvalid) continue;
      const float v = swiglu(acc[m][0][r] * f, acc[m][1][r] * f);
      mx = __builtin_fmaxf(mx, __builtin_fabsf(v));
      h[static_cast<size_t>(b * BM + i) * I + n0 + j] = f32_to_bf16(v);
    }
  }
  if constexpr (FP8ACT) wg_amax_to_slots(mx, amax_h, red);
}

// ---------------------------------------------------------------- down ----
template <int WFMT, bool FP8ACT, int BM>
__global__ __launch_bounds__(kGemmThreads) void gemm_down_kernel(QW w, Rows rows, const uint16_t* __restrict__ h,
                                                                 const uint32_t* __restrict__ amax_h, int H, int I,
                                                                 uint16_t* __restrict__ o) {
  using TS = TileShape<BM>;
  constexpr int kStageBytes = AStage<BM, FP8ACT>::kBytes;
  __shared__ __attribute__((aligned(16))) uint8_t As[2 * kStageBytes];
  __shared__ int flat_of[BM];

  const int ntile = (H + TS::kBN - 1) / TS::kBN;
  const int t = logical_tile(blockIdx.x, rows.num_blocks * ntile);
  if (t >= rows.num_blocks * ntile) return;
  const int b = t / ntile, nt = t % ntile;
  const int e = rows.sorted_ids ? rows.block_expert[b] : 0;
  if (e < 0) return;
  const int nvalid = block_rows(rows, b, e, BM);
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int wm = wave % TS::kWM, wn = wave / TS::kWM;
  const int arow0 = wm * 64;
  const int n0 = nt * TS::kBN + wn * 64;
  const bool wact = n0 < H;   // a last tile may reach past H
  const bool rows_ok[2] = {wact && arow0 < nvalid, wact && arow0 + 32 < nvalid};
  const int j = lane & 31, g = lane >> 5;
  const int nw0 = wact ? n0 : 0;
  const size_t wrow[2] = {static_cast<size_t>(e) * H + nw0 + j, static_cast<size_t>(e) * H + nw0 + 32 + j};
  if (threadIdx.x < BM) {
    const int p = b * BM + threadIdx.x;
    flat_of[threadIdx.x] = rows.sorted_ids ? rows.sorted_ids[p] : p;
  }
  float sh = 1.0f;
  if constexpr (FP8ACT) sh = amax_scale(amax_h);

  ALoader<BM, FP8ACT, FP8ACT> L;
  aloader_init(L, [&](int r) -> const void* { return h + static_cast<size_t>(b * BM + r) * I; });

  f32x16 acc[2][2] = {};
  k_loop<WFMT, FP8ACT, BM, FP8ACT, FP8ACT>(L, As, As + kStageBytes, w, wrow, I, arow0, rows_ok, sh, acc, lane);

  float f = 1.0f;
  if constexpr (WFMT != kMXFP4) f = w.tscale[e];
  if constexpr (FP8ACT) f *= sh;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = arow0 + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
      if (!wact || i >= nvalid) continue;
      const size_t fr = static_cast<size_t>(flat_of[i]);
#pragma unroll
      for (int c = 0; c < 2; ++c) o[fr * H + n0 + 32 * c + j] = f32_to_bf16(acc[m][c][r] * f);
    }
  }
}

// ------------------------------------------------------------ launches ----
template <int WFMT, bool FP8ACT, int BM>
static hipError_t run_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                             const uint32_t* amax_x, int H, int I, uint16_t* h, uint32_t* amax_h, hipStream_t s) {
  const int ntile = (I + TileShape<BM>::kBN / 2 - 1) / (TileShape<BM>::kBN / 2);
  const int total = rows.num_blocks * ntile;
  if (total == 0) return hipSuccess;
  gemm_gateup_kernel<WFMT, FP8ACT, BM>
      <<<8 * ((total + 7) / 8), kGemmThreads, 0, s>>>(w, rows, x, xq, amax_x, H, I, h, amax_h);
  return hipGetLastError();
}

template <int WFMT, bool FP8ACT, int BM>
static hipError_t run_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h, int H, int I,
                           uint16_t* o, hipStream_t s) {
  const int ntile = (H + TileShape<BM>::kBN - 1) / TileShape<BM>::kBN;
  const int total = rows.num_blocks * ntile;
  if (total == 0) return hipSuccess;
  gemm_down_kernel<WFMT, FP8ACT, BM><<<8 * ((total + 7) / 8), kGemmThreads, 0, s>>>(w, rows, h, amax_h, H, I, o);
  return hipGetLastError();
}

template <int BM>
static hipError_t gateup_bm(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                            const uint32_t* amax_x, int H, int inter, uint16_t* h, uint32_t* amax_h, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_gateup<kMXFP4, false, BM>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    case kNVFP4: return run_gateup<kNVFP4, false, BM>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    case kFP8:
      return xq ? run_gateup<kFP8, true, BM>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s)
                : run_gateup<kFP8, false, BM>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BM>
static hipError_t down_bm(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h, int H, int inter,
                          uint16_t* o, hipStream_t s) {
  switch (w.fmt) {
    case kMXFP4: return run_down<kMXFP4, false, BM>(w, rows, h, amax_h, H, inter, o, s);
    case kNVFP4: return run_down<kNVFP4, false, BM>(w, rows, h, amax_h, H, inter, o, s);
    case kFP8:
      return amax_h ? run_down<kFP8, true, BM>(w, rows, h, amax_h, H, inter, o, s)
                    : run_down<kFP8, false, BM>(w, rows, h, amax_h, H, inter, o, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                              const uint32_t* amax_x, int H, int inter, uint16_t* h, uint32_t* amax_h,
                              hipStream_t s) {
  if (rows.block_m == 128) return gateup_bm<128>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
  if (rows.block_m == 64) return gateup_bm<64>(w, rows, x, xq, amax_x, H, inter, h, amax_h, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h, int H,
                            int inter, uint16_t* o, hipStream_t s) {
  if (rows.block_m == 128) return down_bm<128>(w, rows, h, amax_h, H, inter, o, s);
  if (rows.block_m == 64) return down_bm<64>(w, rows, h, amax_h, H, inter, o, s);
  return hipErrorInvalidValue;
}

}  // namespace ftmoe
