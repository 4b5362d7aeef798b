// Decode experts: few tokens per expert, so the work is streaming each
// selected expert's packed weights from HBM exactly once.
//
// Work unit: (block b, group of 16 weight rows per wave).  A block is one
// selected expert with its (up to 16) routed rows -- or, after the routed
// blocks, 16 tokens of the shared expert.  Each wave runs 16x16 MFMA tiles
// whose 16 columns are its weight rows and whose 16 rows are token slots
// (absent slots are zero).
//
// Prologue: every wave reads its lanes' slot-table entries, issues its whole
// weight stream into registers, and then copies the token rows of the
// block's valid slots HBM/L2 -> LDS by LDS DMA (global_load_lds_dwordx4: no
// registers, so nothing to spill) while the weights are in flight; one
// barrier later the MFMA work runs out of registers and LDS.  Rows in LDS are
// stored with their 16-byte vectors XOR-swizzled by (row & 7), so the eight
// lanes of a ds_read_b128 phase that read one K offset of eight different
// rows hit eight different bank groups.
//
// MXFP4 weights go to v_mfma_scale_f32_16x16x128_f8f6f4 as raw E2M1 codes
// with their E8M0 block scales, against activations carried as split E4M3
// pairs (common.hpp), or in the MXFP8 activation mode as single E4M3 codes
// under E8M0 block scales (one MFMA per chunk instead of two); no weight is
// dequantised.  The gate_up workgroup covers one 32-block of h per token
// slot, so it writes h directly in the form the down kernel consumes.
//
// NVFP4 (E4M3 block scales, not expressible as E8M0) and FP8 weights with
// bf16 activations are dequantised to bf16 in registers for
// v_mfma_f32_16x16x32_bf16; FP8 weights with FP8 activations use the f8f6f4
// MFMA with unit scales.
//
// Operand layout of the scaled 16x16x128 MFMA (checked on gfx950): lane
// (n, g) of a 4-bit operand holds elements [32g, 32g+32) of the 128-wide K
// window and its scale applies to exactly that block; lane (i, g) of an 8-bit
// operand holds [16g, 16g+16) in bytes 0-15 and [64+16g, 64+16g+16) in bytes
// 16-31, and the scale register of lane (i, g) is the one of K block g.  With
// unit scales (FP8 x FP8) any consistent K assignment of the two operands is
// valid, so that path keeps 32 contiguous elements per lane.
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kGateWaves = 4;   // MXFP4 gate_up workgroup: 4 x 8 intermediate indices = one 32-block of h
constexpr int kDownWaves = 4;   // waves per down workgroup: a 64-column tile of the output
constexpr int kDownTileN = 16 * kDownWaves;

int decode_down_tiles(int H) { return (H + kDownTileN - 1) / kDownTileN; }

__host__ __device__ constexpr int decode_rows(int T) { return T < kDecodeBM ? T : kDecodeBM; }

using lds_void = __attribute__((address_space(3))) void;

// ------------------------------------------------------------ staging -----
// (row, vector) of sequence element i: floor(i / per_row) through fp32 is
// exact here (i < 2^20, per_row <= 2^10: the product's error stays below
// 2^-3 / per_row, inside the 0.5 / per_row margin to the next integer).
__device__ __forceinline__ void split_index(int i, int per_row, float inv, int& r, int& q) {
  r = static_cast<int>((static_cast<float>(i) + 0.5f) * inv);
  q = i - r * per_row;
}

// Position of vector q of LDS row r (rows of a multiple of 8 vectors).
__device__ __forceinline__ int swz(int r, int q) { return q ^ (r & 7); }

__device__ __forceinline__ i32x8 u4x2(const uint4& p, const uint4& q) {
  return i32x8{static_cast<int>(p.x), static_cast<int>(p.y), static_cast<int>(p.z), static_cast<int>(p.w),
               static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w)};
}

__device__ __forceinline__ uint4 lds16(const uint8_t* row, int r, int q) {
  return *reinterpret_cast<const uint4*>(row + 16 * swz(r, q));
}

// DMA of nvec 16-byte vectors into LDS: vector v lands at lds + 16 v and is
// read from src(v).  Wave w issues the 1 KB chunks w, w + waves, ...; every
// lane of the wave evaluates src (it may shuffle), only lanes v < nvec load.
// Completion is awaited by the caller's __syncthreads (its release fence
// waits for every outstanding vector memory operation).
template <class Src>
__device__ __forceinline__ void dma_stage(uint8_t* lds, int nvec, Src src) {
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = lane_id();
  for (int c = wave; c * 64 < nvec; c += nw) {
    const int v = c * 64 + lane;
    const void* p = src(v < nvec ? v : nvec - 1);
    if (v < nvec) __builtin_amdgcn_global_load_lds(p, (lds_void*)(lds + c * 1024), 16, 0, 0);
  }
}

// DMA of `rows` rows of `rowvec` vectors each, swizzled; row_src(r) is the
// global address of row r.
template <class RowSrc>
__device__ __forceinline__ void dma_rows(uint8_t* lds, int rows, int rowvec, RowSrc row_src) {
  const float inv = 1.0f / static_cast<float>(rowvec);
  dma_stage(lds, rows * rowvec, [&](int v) -> const void* {
    int r, s;
    split_index(v, rowvec, inv, r, s);
    return static_cast<const uint8_t*>(row_src(r)) + 16 * swz(r, s);
  });
}

// DMA of split rows: hi [rows][K], lo [rows][K] (swizzled; absent when lo is
// NULL) and the scale rows [rows][spitch] (plain), consecutive in LDS.  Row r
// of the source is row src_row(r) of hi / lo ([.][K]) and of sc ([.][spitch]).
template <class SrcRow>
__device__ __forceinline__ void dma_split_rows(uint8_t* lds, int rows, int K, int spitch, const uint8_t* hi,
                                               const uint8_t* lo, const uint8_t* sc, SrcRow src_row) {
  const int hv = K / 16, sv = spitch / 16, nh = rows * hv, ncode = lo ? 2 * nh : nh;
  const float inv_h = 1.0f / static_cast<float>(hv), inv_s = 1.0f / static_cast<float>(sv);
  dma_stage(lds, ncode + rows * sv, [&](int v) -> const void* {
    const bool is_sc = v >= ncode, is_lo = !is_sc && v >= nh;
    int r, s;
    split_index(is_sc ? v - ncode : is_lo ? v - nh : v, is_sc ? sv : hv, is_sc ? inv_s : inv_h, r, s);
    // src_row may be a cross-lane shuffle: every lane evaluates it, outside
    // any branch on the lane's region
    const size_t row = static_cast<size_t>(src_row(r));
    if (is_sc) return sc + row * spitch + 16 * s;
    return (is_lo ? lo : hi) + row * K + 16 * swz(r, s);
  });
}

// ------------------------------------------------------------ blocks ------
// A block's LDS holds the rows of its valid slots (at most min(T, 16)): the
// slot table is read first, and only those rows are fetched.

// This lane's token slot (lane & 15) of block b: token row, flat row, valid.
struct LaneSlot {
  int tok, flat;
  bool valid;
};

// The slot table entry is fetched first and decoded only after the weight
// loads are issued, so that its latency overlaps theirs (a use before them
// would make the wave wait for it alone).
__device__ __forceinline__ int slot_fetch(const DecodeArgs& a, int b, bool shared) {
  return shared ? 0 : a.sorted_ids[b * kDecodeBM + (lane_id() & 15)];
}

__device__ __forceinline__ LaneSlot slot_decode(const DecodeArgs& a, bool shared, int p0, int raw) {
  const int j = lane_id() & 15;
  LaneSlot s;
  if (shared) {
    s.flat = p0 + j;
    s.tok = s.flat;
    s.valid = s.flat < a.T;
  } else {
    s.flat = raw;
    s.valid = s.flat < a.T * a.k;
    s.tok = s.valid ? s.flat / a.k : 0;
  }
  return s;
}

// ======================================================== MXFP4 kernels ====
// Activation rows in LDS: hi / lo codes [rows][K] (swizzled), scales
// [rows][spitch]; with MXFP8 activations (A8) only one code plane.
struct MxRows {
  const uint8_t* hi;
  const uint8_t* lo;
  const uint8_t* sc;
  int K, spitch;
};

template <bool A8>
__device__ __forceinline__ MxRows mx_rows(const uint8_t* base, int K, int spitch, int rows) {
  constexpr int kPlanes = A8 ? 1 : 2;
  return MxRows{base, base + rows * K, base + kPlanes * rows * K, K, spitch};
}

template <bool A8>
__host__ __device__ constexpr size_t mx_rows_bytes(int K, int spitch, int rows) {
  return static_cast<size_t>(rows) * ((A8 ? 1 : 2) * K + spitch);
}

// Weight stream of NB chunks of one row: lane group g holds K block 4u + g
// of chunk u (16 code bytes at 64u + 16g: each load instruction reads 64
// contiguous bytes of each of the wave's 16 rows) and its E8M0 scale: with
// PACK (nch a multiple of 4) the row's 16 scale bytes of 4 chunks come as one
// 16-byte load, else one byte per chunk.
template <int NB, bool PACK>
struct MxW {
  uint4 c[NB];
  uint32_t s[NB];
};

template <int NB, bool PACK>
__device__ __forceinline__ void mx_wload(MxW<NB, PACK>& w, const uint8_t* codes, const uint8_t* scales, int u0,
                                         int nch, int g) {
  // Chunks past the row end reload its last chunk (unused): every call issues
  // the same loads, so the compiler's wait counts stay exact.
#pragma unroll
  for (int u = 0; u < NB; ++u) w.c[u] = load16(codes + 64 * min(u0 + u, nch - 1) + 16 * g);
  if constexpr (PACK) {
#pragma unroll
    for (int m = 0; m < NB / 4; ++m) {
      const uint4 v = *reinterpret_cast<const uint4*>(scales + 4 * min(u0 + 4 * m, nch - 4));
      w.s[4 * m] = v.x;
      w.s[4 * m + 1] = v.y;
      w.s[4 * m + 2] = v.z;
      w.s[4 * m + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int u = 0; u < NB; ++u) w.s[u] = scales[4 * min(u0 + u, nch - 1) + g];
  }
}

template <int NB, bool PACK>
__device__ __forceinline__ int mx_wscale(const MxW<NB, PACK>& w, int u, int g) {
  if constexpr (PACK)
    return static_cast<int>((w.s[u] >> (8 * g)) & 0xFF);
  else
    return static_cast<int>(w.s[u]);
}

// MFMA chunk u (K [128u, 128u + 128)): A from LDS row r (zero unless
// `valid`), hi then lo with the scale lowered by 2^4; with A8 the single
// MXFP8 codes.
template <bool A8>
__device__ __forceinline__ void mx_mma(const MxRows& m, int r, bool valid, int u, int g, const uint4& wc, int sb,
                                       f32x4& acc) {
  i32x8 ah = {}, al = {};
  int sa = 0;
  if (valid) {
    const int q0 = 8 * u + g, q1 = q0 + 4;
    const uint8_t* rh = m.hi + r * m.K;
    ah = u4x2(lds16(rh, r, q0), lds16(rh, r, q1));
    if constexpr (!A8) {
      const uint8_t* rl = m.lo + r * m.K;
      al = u4x2(lds16(rl, r, q0), lds16(rl, r, q1));
    }
    sa = m.sc[r * m.spitch + 4 * u + g];
  }
  const i32x8 b = {static_cast<int>(wc.x), static_cast<int>(wc.y), static_cast<int>(wc.z), static_cast<int>(wc.w),
                   0, 0, 0, 0};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, b, acc, 0, 4, 0, sa, 0, sb);
  if constexpr (!A8) {
    const int sa_lo = sa >= 4 ? sa - 4 : 0;
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, b, acc, 0, 4, 0, sa_lo, 0, sb);
  }
}

// Streams one weight row (nch chunks) against LDS rows; the first NB chunks
// are already loaded.
template <int NB, bool PACK, bool A8>
__device__ __forceinline__ void mx_row_dot(MxW<NB, PACK>& wt, const uint8_t* codes, const uint8_t* scales,
                                           const MxRows& m, int r, bool valid, int nch, int g, f32x4& acc) {
#pragma unroll
  for (int u = 0; u < NB; ++u)
    if (u < nch) mx_mma<A8>(m, r, valid, u, g, wt.c[u], mx_wscale(wt, u, g), acc);
  for (int u0 = NB; u0 < nch; u0 += NB) {
    mx_wload(wt, codes, scales, u0, nch, g);
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (u0 + u < nch) mx_mma<A8>(m, r, valid, u0 + u, g, wt.c[u], mx_wscale(wt, u, g), acc);
  }
}

// Split h rows of a block: routed rows [nb_routed * 16][I] first, then the
// shared expert's [nb_shared * 16][Is]; scale rows share one pitch.
struct HSplit {
  uint8_t* hi;
  uint8_t* lo;
  uint8_t* sc;
  int K;
};

__device__ __forceinline__ HSplit h_split_rows(const DecodeArgs& a, bool shared, int row0) {
  const size_t routed = static_cast<size_t>(a.nb_routed) * kDecodeBM;
  const size_t off = shared ? routed * a.I + static_cast<size_t>(row0) * a.Is : static_cast<size_t>(row0) * a.I;
  const size_t srow = shared ? routed + row0 : row0;
  return HSplit{a.hhi + off, a.hlo ? a.hlo + off : nullptr, a.hsc + srow * a.hsc_pitch, shared ? a.Is : a.I};
}

// gate_up: 4 waves, each on 8 intermediate indices (8 gate + 8 up rows); the
// token rows arrive already split (xhi / xlo / xsc), or as MXFP8 (A8).
template <int NB, bool PACK, bool A8>
__global__ __launch_bounds__(64 * kGateWaves) void decode_gateup_mx_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float red[kGateWaves][kDecodeBM];
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const int I = shared ? a.Is : a.I;
  const int c0 = blockIdx.x * 8 * kGateWaves;
  if (c0 >= I) return;
  const int ex = shared ? 0 : a.block_expert[b];
  if (ex < 0) return;
  const QW& w = shared ? a.sgu : a.gu;
  const int e = expert_slot(w, ex);   // slot of its matrices
  if (e < 0) return;                  // served by another pass
  const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
  const int H = a.H, nch = H / 128;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int i0 = c0 + wave * 8;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * (2 * I) + (j < 8 ? i0 + j : I + i0 + (j - 8));

  // 1. the block's slot entries, then the weight stream
  const int raw = slot_fetch(a, b, shared);
  const uint8_t* codes = w.codes + wrow * (H / 2);
  const uint8_t* scales = w.scales + wrow * (H / 32);
  MxW<NB, PACK> wt;
  mx_wload(wt, codes, scales, 0, nch, g);
  __builtin_amdgcn_sched_barrier(0);
  const LaneSlot ls = slot_decode(a, shared, p0, raw);
  // 2. the split token rows of the valid slots -> LDS rows 0 .. count - 1
  const int count = __popcll(__ballot(ls.valid && lane < kDecodeBM));
  const MxRows m = mx_rows<A8>(smem, H, a.xsc_pitch, count);
  dma_split_rows(smem, count, H, a.xsc_pitch, a.xhi, A8 ? nullptr : a.xlo, a.xsc,
                 [&](int r) { return __shfl(ls.tok, r, kWave); });
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mx_row_dot<NB, PACK, A8>(wt, codes, scales, m, j, j < count, nch, g, acc);

  // 3. h = SwiGLU(gate, up) (rounded to bf16 for the split form), then
  //    quantised per 32-block: lanes j < 8 hold column i0 + j of slots
  //    4g + r; the 32-block of a slot spans the 4 waves.
  float hv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float up = __shfl_xor(acc[r], 8, kWave);
    const float sw = swiglu(acc[r], up);
    const float v = A8 ? sw : bf16_to_f32(f32_to_bf16(sw));
    hv[r] = j < 8 ? v : 0.f;
    float mx = __builtin_fabsf(hv[r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 1, kWave));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 2, kWave));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 4, kWave));
    if (j == 0) red[wave][4 * g + r] = mx;
  }
  __syncthreads();
  const HSplit hs = h_split_rows(a, shared, p0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = 4 * g + r;
    if (j < 8 && slot < count) {
      float amax = red[0][slot];
#pragma unroll
      for (int q = 1; q < kGateWaves; ++q) amax = __builtin_fmaxf(amax, red[q][slot]);
      const size_t o = static_cast<size_t>(slot) * hs.K + i0 + j;
      uint32_t code;
      if constexpr (A8) {
        code = mxfp8_scale_code(amax);
        hs.hi[o] = static_cast<uint8_t>(f32x2_to_e4m3x2(hv[r] * mx_inv_scale(code), 0.f) & 0xFF);
      } else {
        code = mx_split_scale_code(amax);
        uint32_t h2, l2;
        mx_split_pair(hv[r] * mx_inv_scale(code), 0.f, &h2, &l2);
        hs.hi[o] = static_cast<uint8_t>(h2 & 0xFF);
        hs.lo[o] = static_cast<uint8_t>(l2 & 0xFF);
      }
      if (wave == 0 && j == 0) hs.sc[static_cast<size_t>(slot) * a.hsc_pitch + c0 / 32] = static_cast<uint8_t>(code);
    }
  }
}

// down: 16 output rows per wave against the block's split (or MXFP8) h rows.
template <int NB, bool PACK, bool A8>
__global__ __launch_bounds__(64 * kDownWaves) void decode_down_mx_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const int ex = shared ? 0 : a.block_expert[b];
  if (ex < 0) return;
  const QW& w = shared ? a.sdn : a.dn;
  const int e = expert_slot(w, ex);   // slot of its matrices
  if (e < 0) return;                  // served by another pass
  const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
  const int K = shared ? a.Is : a.I;
  const int H = a.H, nch = K / 128;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int n0 = blockIdx.x * kDownTileN + wave * 16;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * H + n0 + j;
  const HSplit hs = h_split_rows(a, shared, p0);

  const int raw = slot_fetch(a, b, shared);
  const uint8_t* codes = w.codes + wrow * (K / 2);
  const uint8_t* scales = w.scales + wrow * (K / 32);
  MxW<NB, PACK> wt;
  mx_wload(wt, codes, scales, 0, nch, g);
  __builtin_amdgcn_sched_barrier(0);
  const LaneSlot ls = slot_decode(a, shared, p0, raw);
  // the h rows of the valid slots -> LDS rows 0 .. count - 1
  const int count = __popcll(__ballot(ls.valid && lane < kDecodeBM));
  const MxRows m = mx_rows<A8>(smem, K, a.hsc_pitch, count);
  dma_split_rows(smem, count, K, a.hsc_pitch, hs.hi, A8 ? nullptr : hs.lo, hs.sc, [](int r) { return r; });
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mx_row_dot<NB, PACK, A8>(wt, codes, scales, m, j, j < count, nch, g, acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = 4 * g + r;
    const int flat = __shfl(ls.flat, slot, kWave);
    if (slot < count) {
      if (shared)
        a.s32[static_cast<size_t>(p0 + slot) * H + n0 + j] = acc[r];
      else
        a.o32[static_cast<size_t>(flat) * H + n0 + j] = acc[r];
    }
  }
}

// ================================================ NVFP4 / FP8 / BF16 kernels
// (BF16 weights go to the bf16 MFMA as they are.)
// Per-lane weight slice of one 128-element K chunk (elements [32g, 32g+32)).
struct WSlice4 {   // NVFP4: 16 bytes of codes + two E4M3 block scales
  uint4 c;
  uint32_t sc;
};
struct WSlice8 {   // FP8: 32 bytes of codes
  uint4 c0, c1;
};
struct WSlice16 {  // BF16: 32 values, 8 per MFMA step
  uint4 c[4];
};
template <int WFMT> struct WSliceT { using type = WSlice4; };
template <> struct WSliceT<kFP8> { using type = WSlice8; };
template <> struct WSliceT<kBF16> { using type = WSlice16; };

template <int WFMT>
__device__ __forceinline__ typename WSliceT<WFMT>::type load_wslice(const QW& w, size_t row, int K, int kb) {
  typename WSliceT<WFMT>::type s;
  if constexpr (WFMT == kFP8) {
    const uint8_t* p = w.codes + row * K + kb;
    s.c0 = load16(p);
    s.c1 = load16(p + 16);
  } else if constexpr (WFMT == kBF16) {
    const uint8_t* p = w.codes + (row * K + kb) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) s.c[i] = load16(p + 16 * i);
  } else {
    s.c = load16(w.codes + row * (K / 2) + kb / 2);
    s.sc = *reinterpret_cast<const uint16_t*>(w.scales + row * (K / 16) + kb / 16);
  }
  return s;
}

// bf16 operand (8 values) for MFMA step `st` (0..3) of an NVFP4 slice.
__device__ __forceinline__ bf16x8 nvfp4_bf16(const WSlice4& s, int st) {
  uint32_t o[4];
  const uint32_t word = st == 0 ? s.c.x : st == 1 ? s.c.y : st == 2 ? s.c.z : s.c.w;
  const float sc = e4m3_to_f32((s.sc >> (st < 2 ? 0 : 8)) & 0xFF);
  fp4x8_to_bf16_nv(word, sc, nv_scale_significand(sc), o);
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// bf16 operand (8 values) for MFMA step `st` (0..3) of an FP8 slice.
__device__ __forceinline__ bf16x8 fp8_bf16(const WSlice8& s, int st) {
  const uint4 c = st < 2 ? s.c0 : s.c1;
  uint32_t o[4];
  fp8x4_to_bf16((st & 1) ? c.z : c.x, o);
  fp8x4_to_bf16((st & 1) ? c.w : c.y, o + 2);
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

__device__ __forceinline__ float scale_from_amax(const uint32_t* bits) {
  const float a = __uint_as_float(*bits);
  return a > 0.f ? a / 448.0f : 1.0f;
}

// 8 bf16 -> 8 E4M3 codes of v / sh (fp32 quotient, round to nearest even).
__device__ __forceinline__ uint2 bf16x8_to_e4m3(const uint4& v, float sh) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = f32x2_to_e4m3x2(bf16_to_f32(w[i] & 0xFFFF) / sh, bf16_to_f32(w[i] >> 16) / sh);
  return make_uint2(p[0] | (p[1] << 16), p[2] | (p[3] << 16));
}

// A operand rows in LDS, swizzled: bf16 rows (ABF16) or FP8 rows.
// ABF16 + FP8 MFMA (down with FP8 activations) quantises with sh on the fly.
template <int WFMT, bool FP8MMA, bool ABF16, int NB>
__device__ __forceinline__ void mma_batch(const typename WSliceT<WFMT>::type* ws, int kc0, int K, int g,
                                          const uint8_t* xs, int row_bytes, int r, bool valid, float sh,
                                          f32x4& acc) {
  const uint8_t* row = xs + r * row_bytes;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    if (kc0 + u * 128 >= K) break;
    const int kb = kc0 + u * 128 + g * 32;
    if constexpr (FP8MMA) {
      i32x8 av = {};
      if (valid) {
        if constexpr (ABF16) {
          uint2 p[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) p[q] = bf16x8_to_e4m3(lds16(row, r, kb / 8 + q), sh);
          av = i32x8{static_cast<int>(p[0].x), static_cast<int>(p[0].y), static_cast<int>(p[1].x),
                     static_cast<int>(p[1].y), static_cast<int>(p[2].x), static_cast<int>(p[2].y),
                     static_cast<int>(p[3].x), static_cast<int>(p[3].y)};
        } else {
          av = u4x2(lds16(row, r, kb / 16), lds16(row, r, kb / 16 + 1));
        }
      }
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, u4x2(ws[u].c0, ws[u].c1), acc, 0, 0, 0, 127, 0,
                                                             127);
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 bw;
        if constexpr (WFMT == kFP8)
          bw = fp8_bf16(ws[u], st);
        else if constexpr (WFMT == kBF16)
          bw = __builtin_bit_cast(bf16x8, ws[u].c[st]);
        else
          bw = nvfp4_bf16(ws[u], st);
        const bf16x8 av = valid ? __builtin_bit_cast(bf16x8, lds16(row, r, kb / 8 + st)) : bf16x8{};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw, acc, 0, 0, 0);
      }
    }
  }
}

template <int WFMT, bool FP8ACT, int NB, int WPB>
__global__ __launch_bounds__(64 * WPB) void decode_gateup_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ float red[16];
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const int ex = shared ? 0 : a.block_expert[b];
  if (ex < 0) return;
  const QW& w = shared ? a.sgu : a.gu;
  const int e = expert_slot(w, ex);   // slot of its matrices
  if (e < 0) return;                  // served by another pass
  const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
  const int I = shared ? a.Is : a.I;
  const int H = a.H;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  // I is a multiple of 128, so a workgroup's waves are all inside or all past it
  static_assert(16 % WPB == 0, "waves per workgroup");
  if (blockIdx.x * WPB * 8 >= I) return;
  const int i0 = (blockIdx.x * WPB + wave) * 8;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * (2 * I) + (j < 8 ? i0 + j : I + i0 + (j - 8));
  const int row_bytes = FP8ACT ? H : 2 * H;

  // the block's slots, the weight stream, then the token rows of the valid
  // slots -> LDS rows 0 .. count - 1
  const int raw = slot_fetch(a, b, shared);
  typename WSliceT<WFMT>::type ws[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) ws[u] = load_wslice<WFMT>(w, wrow, H, min(u * 128, H - 128) + g * 32);
  __builtin_amdgcn_sched_barrier(0);
  const LaneSlot ls = slot_decode(a, shared, p0, raw);
  const int count = __popcll(__ballot(ls.valid && lane < kDecodeBM));
  dma_rows(xs, count, row_bytes / 16, [&](int r) -> const void* {
    const size_t t = static_cast<size_t>(__shfl(ls.tok, r, kWave));
    return FP8ACT ? a.xq + t * H : reinterpret_cast<const uint8_t*>(a.x + t * H);
  });
  __syncthreads();

  const int arow = j;
  const bool aval = j < count;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mma_batch<WFMT, FP8ACT, false, NB>(ws, 0, H, g, xs, row_bytes, arow, aval, 1.0f, acc);
  for (int kc0 = NB * 128; kc0 < H; kc0 += NB * 128) {
#pragma unroll
    for (int u = 0; u < NB; ++u) ws[u] = load_wslice<WFMT>(w, wrow, H, min(kc0 + u * 128, H - 128) + g * 32);
    mma_batch<WFMT, FP8ACT, false, NB>(ws, kc0, H, g, xs, row_bytes, arow, aval, 1.0f, acc);
  }

  // this lane's weight row's multiplier (and the activation scale)
  float f = WFMT == kBF16 ? 1.0f : row_scale(w, e, j < 8 ? i0 + j : I + i0 + (j - 8));
  if constexpr (FP8ACT) f *= scale_from_amax(a.amax_x);
  uint16_t* h = shared ? a.hs : a.h;
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float val = acc[r] * f;
    const float up = __shfl_xor(val, 8, kWave);
    const int slot = 4 * g + r;
    if (j < 8 && slot < count) {
      const float v = swiglu(val, up);
      h[static_cast<size_t>(p0 + slot) * I + i0 + j] = f32_to_bf16(v);
      mx = __builtin_fmaxf(mx, __builtin_fabsf(v));
    }
  }
  if constexpr (FP8ACT) wg_amax_to_slots(mx, a.amax_slots, red);
}

// One- and two-token batches: the KS waves of a workgroup share one group of
// 16 weight rows (8 gate + 8 up) and split it along K, so the step's stream
// is carried by KS times as many waves and each wave's dequantisation and
// MFMA chain is 1/KS as long.  The partial sums meet in LDS and are added in
// wave order (fixed, so the result does not depend on timing).
template <int WFMT, bool FP8ACT, int NB, int KS>
__global__ __launch_bounds__(64 * KS) void decode_gateup_ks_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ f32x4 part[KS][kWave];
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const int ex = shared ? 0 : a.block_expert[b];
  if (ex < 0) return;
  const QW& w = shared ? a.sgu : a.gu;
  const int e = expert_slot(w, ex);   // slot of its matrices
  if (e < 0) return;                  // served by another pass
  const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
  const int I = shared ? a.Is : a.I;
  const int H = a.H;
  if (static_cast<int>(blockIdx.x) * 8 >= I) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int i0 = blockIdx.x * 8;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * (2 * I) + (j < 8 ? i0 + j : I + i0 + (j - 8));
  const int row_bytes = FP8ACT ? H : 2 * H;
  const int kq = H / KS, k0 = wave * kq, k1 = k0 + kq;   // this wave's K range (multiples of 128)

  const int raw = slot_fetch(a, b, shared);
  typename WSliceT<WFMT>::type ws[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) ws[u] = load_wslice<WFMT>(w, wrow, H, min(k0 + u * 128, k1 - 128) + g * 32);
  __builtin_amdgcn_sched_barrier(0);
  const LaneSlot ls = slot_decode(a, shared, p0, raw);
  const int count = __popcll(__ballot(ls.valid && lane < kDecodeBM));
  dma_rows(xs, count, row_bytes / 16, [&](int r) -> const void* {
    const size_t t = static_cast<size_t>(__shfl(ls.tok, r, kWave));
    return FP8ACT ? a.xq + t * H : reinterpret_cast<const uint8_t*>(a.x + t * H);
  });
  __syncthreads();

  const bool aval = j < count;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mma_batch<WFMT, FP8ACT, false, NB>(ws, k0, k1, g, xs, row_bytes, j, aval, 1.0f, acc);
  for (int kc0 = k0 + NB * 128; kc0 < k1; kc0 += NB * 128) {
#pragma unroll
    for (int u = 0; u < NB; ++u) ws[u] = load_wslice<WFMT>(w, wrow, H, min(kc0 + u * 128, k1 - 128) + g * 32);
    mma_batch<WFMT, FP8ACT, false, NB>(ws, kc0, k1, g, xs, row_bytes, j, aval, 1.0f, acc);
  }
  if (wave > 0) part[wave][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int q = 1; q < KS; ++q) {
    const f32x4 p = part[q][lane];
    acc[0] += p[0];
    acc[1] += p[1];
    acc[2] += p[2];
    acc[3] += p[3];
  }

  float f = WFMT == kBF16 ? 1.0f : row_scale(w, e, j < 8 ? i0 + j : I + i0 + (j - 8));
  if constexpr (FP8ACT) f *= scale_from_amax(a.amax_x);
  uint16_t* h = shared ? a.hs : a.h;
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float val = acc[r] * f;
    const float up = __shfl_xor(val, 8, kWave);
    const int slot = 4 * g + r;
    if (j < 8 && slot < count) {
      const float v = swiglu(val, up);
      h[static_cast<size_t>(p0 + slot) * I + i0 + j] = f32_to_bf16(v);
      mx = __builtin_fmaxf(mx, __builtin_fabsf(v));
    }
  }
  if constexpr (FP8ACT) wave_amax_to_slots(mx, a.amax_slots);
}

template <int WFMT, bool FP8ACT, int NB>
__global__ __launch_bounds__(64 * kDownWaves) void decode_down_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t hsm[];
  const int b = blockIdx.y;
  const bool shared = b >= a.nb_routed;
  const int ex = shared ? 0 : a.block_expert[b];
  if (ex < 0) return;
  const QW& w = shared ? a.sdn : a.dn;
  const int e = expert_slot(w, ex);   // slot of its matrices
  if (e < 0) return;                  // served by another pass
  const int p0 = (shared ? b - a.nb_routed : b) * kDecodeBM;
  const int K = shared ? a.Is : a.I;
  const int H = a.H;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int n0 = blockIdx.x * kDownTileN + wave * 16;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * H + n0 + j;
  const uint16_t* hsrc = shared ? a.hs : a.h;

  const int raw = slot_fetch(a, b, shared);
  typename WSliceT<WFMT>::type ws[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u)
    ws[u] = load_wslice<WFMT>(w, wrow, K, min(u * 128, K - 128) + g * 32);
  __builtin_amdgcn_sched_barrier(0);
  const LaneSlot ls = slot_decode(a, shared, p0, raw);
  // the h rows of the valid slots -> LDS
  const int count = __popcll(__ballot(ls.valid && lane < kDecodeBM));
  dma_rows(hsm, count, K / 8, [&](int r) -> const void* { return hsrc + static_cast<size_t>(p0 + r) * K; });
  float sh = 1.0f;
  if constexpr (FP8ACT) sh = scale_from_amax(a.amax_h);
  __syncthreads();
  const bool aval = j < count;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  mma_batch<WFMT, FP8ACT, true, NB>(ws, 0, K, g, hsm, 2 * K, j, aval, sh, acc);
  for (int kc0 = NB * 128; kc0 < K; kc0 += NB * 128) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      ws[u] = load_wslice<WFMT>(w, wrow, K, min(kc0 + u * 128, K - 128) + g * 32);
    mma_batch<WFMT, FP8ACT, true, NB>(ws, kc0, K, g, hsm, 2 * K, j, aval, sh, acc);
  }
  const float f = (WFMT == kBF16 ? 1.0f : row_scale(w, e, n0 + j)) * sh;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int slot = 4 * g + r;
    const int flat = __shfl(ls.flat, slot, kWave);
    if (slot < count) {
      if (shared)
        a.s32[static_cast<size_t>(p0 + slot) * H + n0 + j] = acc[r] * f;
      else
        a.o32[static_cast<size_t>(flat) * H + n0 + j] = acc[r] * f;
    }
  }
}

// ============================================ one token: down + combine ====
// A one-token step routes its k rows to k distinct experts, one row per block.
// For MXFP4 experts one workgroup then takes 16 output columns of every block
// at once: wave b streams block b's 16 weight rows (the shared expert's block
// last) against the block's split h row, the 16 fp32 outputs of each block
// meet in LDS, and wave 0 adds them exactly as the combine kernel does
// (ascending j, then the gated shared expert), so the step needs no separate
// combine launch and gives the same bits as down followed by combine.  (The
// formats dequantised in registers are VALU-bound here: with every block's
// conversion on half as many CUs the fused launch took as long as the two.)
constexpr int kFusedMaxBlocks = 16;   // waves per workgroup

// y[n0 .. n0 + 15] of the token from the blocks' outputs ob[block][column].
__device__ __forceinline__ void combine_one_token(const DecodeArgs& a, const float (*ob)[16], const int* blk_of,
                                                  int n0) {
  const int lane = lane_id();
  if (threadIdx.x >= 16) return;
  float acc = 0.f;
  for (int jj = 0; jj < a.k; ++jj) acc = fmaf(a.w[jj], ob[blk_of[jj]][lane], acc);
  if (a.sg) acc = fmaf(a.sg[0], ob[a.nb_routed][lane], acc);
  a.y[n0 + lane] = f32_to_bf16(acc);
}

template <int NB, bool PACK, bool A8>
__global__ __launch_bounds__(64 * kFusedMaxBlocks) void decode_down_combine1_mx_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float ob[kFusedMaxBlocks][16];
  __shared__ int blk_of[kFusedMaxBlocks];
  const int nbl = a.nb_routed + a.nb_shared;
  const int b = threadIdx.x >> 6, lane = lane_id();   // one wave per block
  const bool shared = b >= a.nb_routed;
  const int ex = shared ? 0 : a.block_expert[b];
  const bool live = ex >= 0;
  const QW& w = shared ? a.sdn : a.dn;
  const int e = live ? expert_slot(w, ex) : 0;
  const int K = a.I, H = a.H, nch = K / 128;   // (the shared expert has the same K)
  const int n0 = blockIdx.x * 16;
  const int j = lane & 15, g = lane >> 4;
  const size_t wrow = static_cast<size_t>(e) * H + n0 + j;
  const uint8_t* codes = w.codes + wrow * (K / 2);
  const uint8_t* scales = w.scales + wrow * (K / 32);
  MxW<NB, PACK> wt;
  if (live) mx_wload(wt, codes, scales, 0, nch, g);
  const int flat = live && !shared ? a.sorted_ids[b * kDecodeBM] : -1;
  __builtin_amdgcn_sched_barrier(0);
  // the h row of every block (slot 0 of block r is h row 16 r, the shared
  // expert's rows following the routed ones) -> LDS row r
  const MxRows m = mx_rows<A8>(smem, K, a.hsc_pitch, nbl);
  dma_split_rows(smem, nbl, K, a.hsc_pitch, a.hhi, A8 ? nullptr : a.hlo, a.hsc,
                 [](int r) { return r * kDecodeBM; });
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (live) mx_row_dot<NB, PACK, A8>(wt, codes, scales, m, b, j == 0, nch, g, acc);
  if (g == 0) ob[b][j] = live ? acc[0] : 0.f;   // column n0 + j of the block's slot 0
  if (flat >= 0 && lane == 0) blk_of[flat] = b;
  __syncthreads();
  combine_one_token(a, ob, blk_of, n0);
}

// ============================================================ combine =====
// y[t] = sum_j w[t,j] o[t*k+j] (ascending j) + sg[t] s[t], from the fp32
// partial outputs; one thread per 4 columns.  Every row's load is issued
// before the sums (MAXK >= k rows, unrolled).
template <int MAXK>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int per_row = a.H / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.T * per_row) return;
  const int t = idx / per_row, c = (idx % per_row) * 4;
  float4 v[MAXK];
  float wj[MAXK];
#pragma unroll
  for (int jj = 0; jj < MAXK; ++jj) {
    if (jj < a.k) {
      const size_t r = static_cast<size_t>(t) * a.k + jj;
      wj[jj] = a.w[r];
      v[jj] = *reinterpret_cast<const float4*>(a.o32 + r * a.H + c);
    }
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int jj = 0; jj < MAXK; ++jj) {
    if (jj < a.k) {
      acc.x = fmaf(wj[jj], v[jj].x, acc.x);
      acc.y = fmaf(wj[jj], v[jj].y, acc.y);
      acc.z = fmaf(wj[jj], v[jj].z, acc.z);
      acc.w = fmaf(wj[jj], v[jj].w, acc.w);
    }
  }
  if (a.sg) {
    const float gt = a.sg[t];
    const float4 q = *reinterpret_cast<const float4*>(a.s32 + static_cast<size_t>(t) * a.H + c);
    acc.x = fmaf(gt, q.x, acc.x);
    acc.y = fmaf(gt, q.y, acc.y);
    acc.z = fmaf(gt, q.z, acc.z);
    acc.w = fmaf(gt, q.w, acc.w);
  }
  *reinterpret_cast<uint2*>(a.y + static_cast<size_t>(t) * a.H + c) =
      make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

// ========================================================= x split prep ===
// xhi / xlo [T][H] and xsc [T][xsc_pitch] of bf16 x: one thread per 32-block
// (xlo NULL: MXFP8 codes in xhi).
__global__ __launch_bounds__(256) void x_split_kernel(const uint16_t* __restrict__ x, int T, int H, int xsc_pitch,
                                                      uint8_t* __restrict__ xhi, uint8_t* __restrict__ xlo,
                                                      uint8_t* __restrict__ xsc) {
  const int nb = H / 32;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * nb) return;
  const int t = i / nb, blk = i % nb;
  const uint4* p = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + blk * 32);
  uint4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = p[q];
  uint8_t* sc = xsc + static_cast<size_t>(t) * xsc_pitch + blk;
  if (xlo)
    mx_split_block(v, xhi + static_cast<size_t>(t) * H + blk * 32, xlo + static_cast<size_t>(t) * H + blk * 32, sc);
  else
    mxfp8_block(v, xhi + static_cast<size_t>(t) * H + blk * 32, sc);
}

hipError_t launch_x_split(const uint16_t* x, int T, int H, int xsc_pitch, uint8_t* xhi, uint8_t* xlo,
                          uint8_t* xsc, hipStream_t s) {
  const int n = T * (H / 32);
  return launch(x_split_kernel, dim3((n + 255) / 256), dim3(256), 0, s, x, T, H, xsc_pitch, xhi, xlo, xsc);
}

// ============================================================ launches ====
// Kernels that may need more than 64 KB of dynamic LDS opt in.
template <class Kern>
static hipError_t allow_lds(Kern kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  if (bytes > 150 * 1024) return hipErrorInvalidValue;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

template <bool PACK, bool A8>
static hipError_t run_gateup_mx_p(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = 16;
  const int imax = a.Is > a.I ? a.Is : a.I;
  const size_t lds = mx_rows_bytes<A8>(a.H, a.xsc_pitch, decode_rows(a.T));
  dim3 grid(imax / (8 * kGateWaves), a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_gateup_mx_kernel<NB, PACK, A8>, lds);
  if (e != hipSuccess) return e;
  return launch(decode_gateup_mx_kernel<NB, PACK, A8>, grid, dim3(64 * kGateWaves), lds, s, a);
}

static hipError_t run_gateup_mx(const DecodeArgs& a, hipStream_t s) {
  const bool pack = (a.H / 128) % 4 == 0;
  if (a.a8) return pack ? run_gateup_mx_p<true, true>(a, s) : run_gateup_mx_p<false, true>(a, s);
  return pack ? run_gateup_mx_p<true, false>(a, s) : run_gateup_mx_p<false, false>(a, s);
}

template <int WFMT, bool FP8ACT, int WPB>
static hipError_t run_gateup(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = WFMT == kBF16 ? 4 : WFMT == kFP8 ? 8 : 16;
  const int imax = a.Is > a.I ? a.Is : a.I;
  const size_t lds = static_cast<size_t>(decode_rows(a.T)) * (FP8ACT ? a.H : 2 * a.H);
  dim3 grid((imax / 8 + WPB - 1) / WPB, a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_gateup_kernel<WFMT, FP8ACT, NB, WPB>, lds);
  if (e != hipSuccess) return e;
  return launch(decode_gateup_kernel<WFMT, FP8ACT, NB, WPB>, grid, dim3(64 * WPB), lds, s, a);
}

template <bool PACK, bool A8>
static hipError_t run_down_mx_p(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = 8;
  const int kmax = a.Is > a.I ? a.Is : a.I;
  const size_t lds = mx_rows_bytes<A8>(kmax, a.hsc_pitch, decode_rows(a.T));
  dim3 grid(decode_down_tiles(a.H), a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_down_mx_kernel<NB, PACK, A8>, lds);
  if (e != hipSuccess) return e;
  return launch(decode_down_mx_kernel<NB, PACK, A8>, grid, dim3(64 * kDownWaves), lds, s, a);
}

static hipError_t run_down_mx(const DecodeArgs& a, hipStream_t s) {
  // PACK needs every K of the launch (routed and shared) to hold whole dwords of scales
  const bool pack = (a.I / 128) % 4 == 0 && (a.Is / 128) % 4 == 0;
  if (a.a8) return pack ? run_down_mx_p<true, true>(a, s) : run_down_mx_p<false, true>(a, s);
  return pack ? run_down_mx_p<true, false>(a, s) : run_down_mx_p<false, false>(a, s);
}

template <int WFMT, bool FP8ACT>
static hipError_t run_down(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = WFMT == kBF16 ? 2 : WFMT == kFP8 ? 4 : 8;
  const int kmax = a.Is > a.I ? a.Is : a.I;
  const size_t lds = static_cast<size_t>(decode_rows(a.T)) * 2 * kmax;
  dim3 grid(decode_down_tiles(a.H), a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_down_kernel<WFMT, FP8ACT, NB>, lds);
  if (e != hipSuccess) return e;
  return launch(decode_down_kernel<WFMT, FP8ACT, NB>, grid, dim3(64 * kDownWaves), lds, s, a);
}

// One- and two-token batches touch few experts: each group of 16 weight rows
// is split along K over the 4 waves of a workgroup when H allows it (else one
// wave per group), so the stream is spread over every CU; larger batches
// share each LDS token copy among 4 waves on different row groups.
template <int WFMT, bool FP8ACT>
static hipError_t run_gateup_small(const DecodeArgs& a, hipStream_t s) {
  if (a.H % (4 * 128)) return run_gateup<WFMT, FP8ACT, 1>(a, s);
  constexpr int KS = 4;
  constexpr int NB = 4;   // K chunks in flight per wave: a quarter of H = 2048
  const int imax = a.Is > a.I ? a.Is : a.I;
  const size_t lds = static_cast<size_t>(decode_rows(a.T)) * (FP8ACT ? a.H : 2 * a.H);
  dim3 grid(imax / 8, a.nb_routed + a.nb_shared);
  const hipError_t e = allow_lds(decode_gateup_ks_kernel<WFMT, FP8ACT, NB, KS>, lds);
  if (e != hipSuccess) return e;
  return launch(decode_gateup_ks_kernel<WFMT, FP8ACT, NB, KS>, grid, dim3(64 * KS), lds, s, a);
}

hipError_t launch_decode_gateup(const DecodeArgs& a, hipStream_t s) {
  const bool fp8act = a.xq != nullptr;
  const bool small = a.T <= 2;
  switch (a.gu.fmt) {
    case kMXFP4: return run_gateup_mx(a, s);
    case kNVFP4: return small ? run_gateup_small<kNVFP4, false>(a, s) : run_gateup<kNVFP4, false, 4>(a, s);
    case kFP8:
      if (fp8act) return small ? run_gateup_small<kFP8, true>(a, s) : run_gateup<kFP8, true, 4>(a, s);
      return small ? run_gateup_small<kFP8, false>(a, s) : run_gateup<kFP8, false, 4>(a, s);
    case kBF16:
      if (fp8act) return hipErrorInvalidValue;
      return small ? run_gateup_small<kBF16, false>(a, s) : run_gateup<kBF16, false, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s) {
  const bool fp8act = a.amax_h != nullptr;
  switch (a.dn.fmt) {
    case kMXFP4: return run_down_mx(a, s);
    case kNVFP4: return run_down<kNVFP4, false>(a, s);
    case kFP8: return fp8act ? run_down<kFP8, true>(a, s) : run_down<kFP8, false>(a, s);
    case kBF16: return fp8act ? hipErrorInvalidValue : run_down<kBF16, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

bool decode_fused_one_token(const DecodeArgs& a) {
  const int nbl = a.nb_routed + a.nb_shared;
  return a.T == 1 && a.dn.fmt == kMXFP4 && nbl <= kFusedMaxBlocks && (a.nb_shared == 0 || a.Is == a.I) &&
         a.H % 16 == 0 && !a.dn.slot_of;
}

template <bool PACK, bool A8>
static hipError_t run_down_combine1_mx(const DecodeArgs& a, hipStream_t s) {
  constexpr int NB = 8;
  const int nbl = a.nb_routed + a.nb_shared;
  const size_t lds = mx_rows_bytes<A8>(a.I, a.hsc_pitch, nbl);
  const hipError_t e = allow_lds(decode_down_combine1_mx_kernel<NB, PACK, A8>, lds);
  if (e != hipSuccess) return e;
  return launch(decode_down_combine1_mx_kernel<NB, PACK, A8>, dim3(a.H / 16), dim3(64 * nbl), lds, s, a);
}

hipError_t launch_decode_down_combine1(const DecodeArgs& a, hipStream_t s) {
  if (!decode_fused_one_token(a)) return hipErrorInvalidValue;
  const bool pack = (a.I / 128) % 4 == 0;
  if (a.a8) return pack ? run_down_combine1_mx<true, true>(a, s) : run_down_combine1_mx<false, true>(a, s);
  return pack ? run_down_combine1_mx<true, false>(a, s) : run_down_combine1_mx<false, false>(a, s);
}

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s) {
  const int n = a.T * (a.H / 4);
  if (a.k <= 8) return launch(decode_combine_kernel<8>, dim3((n + 255) / 256), dim3(256), 0, s, a);
  return launch(decode_combine_kernel<16>, dim3((n + 255) / 256), dim3(256), 0, s, a);
}

}  // namespace ftmoe
