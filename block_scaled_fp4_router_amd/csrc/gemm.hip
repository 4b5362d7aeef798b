// Prefill experts: grouped GEMMs over the expert-sorted row blocks.
//
// A workgroup is 8 waves over one (row block, column tile): BM token rows of
// one expert (BM = 128 or 64) times a tile of the expert's weight rows.  Each
// wave owns a 64 x 64 output tile (2 x 2 MFMA tiles of 32 x 32), or 64 x 128
// (2 x 4) with 128-row blocks; the waves are laid out BM/64 along rows and
// 8 / (BM/64) along columns.  NVFP4 gate_up launches with 64-row blocks and
// enough tiles to fill the chip twice take 64 x 128 wave tiles too: the
// workgroup then spans two 512-row weight tiles (1024 weight rows), and each
// activation fragment read from LDS, as well as each activation stage
// fetched, serves twice the columns.
//   gate_up: a wave's two column tiles are 32 gate rows and the 32 matching up
//            rows, so h = silu(gate) * up is formed in registers;
//   down:    a wave's two column tiles are 64 consecutive output columns.
//
// K advances in stages of 64.  Both operands of a stage -- the activation
// rows, gathered through the sorted row ids, and the weight rows in their
// packed format -- are copied HBM -> LDS by LDS DMA (global_load_lds_dwordx4)
// into a ring of kRing stage buffers, kRing - 1 stages ahead of the MFMA work,
// so the long latency of the gathered rows and of the weight stream is
// covered by several stages of MFMA work.  The ring buffers are distinct LDS
// objects, so the compiler's wait before a read covers only the DMA into that
// buffer; each wave additionally waits for its own DMA of the stage before
// the one barrier per stage.  16-byte vectors are XOR-swizzled by row so that
// the 8 lanes of a ds_read_b128 phase hit 8 different bank groups.
//
// MXFP4 weights never leave their format: the activations arrive split into
// two E4M3 codes per element with an E8M0 scale per 32 (x = s (hi + lo/16),
// as exact as bf16), and v_mfma_scale_f32_32x32x64_f8f6f4 multiplies them
// with the E2M1 codes, applying both E8M0 block scales in hardware -- two
// MFMAs (hi, lo) per 64 K, no per-element conversion.  The gate_up epilogue
// writes h in the same split form for the down GEMM.  In the MXFP8
// activation mode (W4A8) x and h are single E4M3 codes under E8M0 block
// scales: one scaled MFMA per 64 K, and half the activation bytes.  NVFP4 weights (E4M3
// block scales are not powers of two) are converted to bf16 (E2M1 x E4M3 is
// exact in bf16) for v_mfma_f32_32x32x16_bf16.  FP8 weights with FP8
// activations feed the scaled MFMA with unit scales; tensor and activation
// scales are applied in the epilogue.  Block scales travel with their stage
// (one dword per row per stage or per two stages).
//
// Within a stage, lane group g (lane / 32) of the bf16 MFMA takes K elements
// [32g + 8t, 32g + 8t + 8) at MFMA step t: both operands use this assignment,
// so a lane's weight bytes for the stage are one contiguous 16-byte run (two
// E4M3 scales for NVFP4).  The scaled MFMA takes E2M1 K [32g, 32g + 32) and
// 8-bit K [16g, 16g + 16) + [32 + 16g, 48 + 16g) in lane group g.
//
// Workgroups are numbered so that each XCD (workgroup w runs on XCD w % 8)
// receives runs of consecutive (block, tile) pairs: the column tiles of a
// row block, and the row blocks of one expert, then share that XCD's L2.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

constexpr int kGemmWaves = 8;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kStageK = 64;

using lds_void = __attribute__((address_space(3))) void;

int gemm_block_m(int T, int k, int E, int wfmt, bool a8) {
  // Small experts (few rows each) waste less padding with 64-row blocks; FP8
  // weight stages are twice as wide, and MXFP8 activation stages half as
  // wide, so both always use 128-row blocks (whole DMA chunks per wave).
  if (wfmt == kFP8 || wfmt == kBF16 || a8) return 128;
  return static_cast<long long>(T) * k >= 192LL * E ? 128 : 64;
}

template <int WFMT, bool FP8ACT, int BM, bool WIDE = false>
struct Cfg {
  static constexpr int kWM = BM / 64;                  // waves along rows
  static constexpr int kWN = kGemmWaves / kWM;         // waves along columns
  // WIDE (NVFP4 gate_up with 64-row blocks): each wave takes 4 column tiles,
  // so a workgroup covers two 512-row weight tiles and every activation
  // fragment it reads feeds twice the MFMAs
  static constexpr bool kWide = WIDE;
  static_assert(!WIDE || (WFMT == kNVFP4 && BM == 64), "wide tiles: NVFP4, 64-row blocks");
  // 32-column MFMA tiles per wave (BF16 weight stages are 4x as wide as
  // FP4's, so their tile has half the columns)
  static constexpr int kNT = WFMT == kBF16 ? 2 : (BM == 128 || kWide) ? 4 : 2;
  static constexpr int kBN = 32 * kNT * kWN;           // weight rows per workgroup
  static constexpr int kSub = kWide ? 2 : 1;           // packed weight tiles per workgroup tile
  static constexpr int kTileW = kBN / kSub;            // rows of one packed tile
  static constexpr int kAV = FP8ACT ? 4 : 8;           // 16-byte vectors per activation row and stage
  static constexpr int kARowB = 16 * kAV;
  static constexpr int kBRowB = WFMT == kBF16 ? 128 : WFMT == kFP8 ? 64 : 32;  // weight bytes per row and stage
  static constexpr int kBV = kBRowB / 16;
  static constexpr int kABytes = BM * kARowB;
  static constexpr int kBBytes = kBN * kBRowB;
  static constexpr bool kScales = WFMT == kMXFP4 || WFMT == kNVFP4;   // FP4: one scale dword per weight row and stage
  static constexpr int kSBytes = kScales ? 4 * kBN : 0;
  // MXFP4: split E4M3 activations (a row's stage = 64 hi + 64 lo bytes), or
  // with FP8ACT the MXFP8 form (64 bytes), and one E8M0 scale dword per
  // activation row and two stages
  static constexpr bool kAScales = WFMT == kMXFP4;
  static constexpr bool kSplitA = kAScales && !FP8ACT;
  static constexpr int kASBytes = kAScales ? 4 * BM : 0;
  static constexpr int kSlotBytes = kABytes + kBBytes + kSBytes + kASBytes;
  static constexpr int kRing = kSlotBytes * 4 <= 150 * 1024 ? 4 : 3;   // stage buffers in LDS
  static_assert(kRing * kSlotBytes <= 150 * 1024, "LDS");
  static constexpr int kAChunks = kABytes / 1024;     // 1 KB = one wave's 16-byte DMA instruction
  static constexpr int kChunks = (kABytes + kBBytes) / 1024;
  static constexpr int kChunksPerWave = kChunks / kGemmWaves;
  static_assert(kChunks % kGemmWaves == 0, "every wave issues the same number of DMA instructions");
  static constexpr int kScaleRowsPerWave = kBN / kGemmWaves;
  static constexpr int kScaleInstr = (kScaleRowsPerWave + 63) / 64;   // 4-byte DMA instructions per wave and stage
  static_assert(kScaleRowsPerWave <= 64 || kScaleRowsPerWave == 128, "scale rows per wave");
  static constexpr int kARowsPerWave = BM / kGemmWaves;   // activation scale rows per wave
  static constexpr int kVmPerStage = kChunksPerWave + (kScales ? kScaleInstr : 0) + (kAScales ? 1 : 0);
  static_assert(kVmPerStage * (kRing - 2) < 64, "vmcnt range");
};

// ------------------------------------------------------------ helpers -----
// Workgroup w runs on XCD w % 8.  Tiles are dealt to the XCDs in chunks of
// kXcdChunk consecutive tiles (chunk c to XCD c % 8), so each XCD's L2 sees
// runs of tiles of the same expert, while the empty tail of the padded block
// list (the grid covers the largest possible one) is spread over all XCDs.
constexpr int kXcdChunk = 32;
__device__ __forceinline__ int logical_tile(int w) {
  const int x = w & 7, li = w >> 3;
  return ((li / kXcdChunk) * 8 + x) * kXcdChunk + li % kXcdChunk;
}

// Position of vector q in an LDS row of V 16-byte vectors (V = 8, 4 or 2).
// A fragment read takes one vector from each of 32 consecutive rows; the XOR
// pattern spreads them over the LDS banks.  The patterns were checked with
// the LDS bank-conflict counter (SQ_LDS_BANK_CONFLICT against
// SQ_LDS_IDX_ACTIVE) on the GEMMs that use them: none for V = 8 and V = 2.
// For the 64-byte rows (V = 4) q ^ ((r >> 2) & 3) measured no conflicts,
// where q ^ (((r >> 1) ^ (r >> 3)) & 3) measured one conflict cycle per access
// and q ^ (r & 3) three.
template <int V>
__device__ __forceinline__ int swz(int r, int q) {
  if constexpr (V == 8)
    return q ^ ((r & 7) ^ ((r >> 3) & 1));
  else if constexpr (V == 4)
    return q ^ ((r >> 2) & 3);
  else
    return q ^ (((r >> 2) ^ (r >> 3)) & 1);
}

// Waits until at most N vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS DMA of 16 (4) bytes per lane: lane l's bytes land at dst + 16 l (4 l);
// dst is the same for every lane of the wave.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
}

// Workgroup barrier that also keeps the compiler from moving memory accesses
// across it (no fence: outstanding DMA is waited for explicitly).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

__device__ __forceinline__ i32x8 u4x2(const uint4& p, const uint4& q) {
  return i32x8{static_cast<int>(p.x), static_cast<int>(p.y), static_cast<int>(p.z), static_cast<int>(p.w),
               static_cast<int>(q.x), static_cast<int>(q.y), static_cast<int>(q.z), static_cast<int>(q.w)};
}


// ---- LDS fragment reads --------------------------------------------------
// The ring buffers are written by LDS DMA, which the compiler can only order
// against LDS reads by waiting for every DMA in flight (all later stages
// included).  Fragment reads therefore go through these asm blocks, which
// wait for their own results before returning; the stage's DMA has been
// waited for explicitly before the barrier.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}

// One LDS dword, waited for.
__device__ __forceinline__ int lds_i32(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n s_waitcnt lgkmcnt(0)\n" : "=v"(v) : "v"(addr));
  return v;
}

// Completes the LDS reads a fragment reader left in flight.  The vectors are
// passed through the asm, so no use of them can be scheduled before the wait
// and their registers stay allocated until it.
__device__ __forceinline__ void frag_wait4(u32x4& a, u32x4& b, u32x4& c, u32x4& d) {
  asm volatile("s_waitcnt lgkmcnt(0)\n" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void frag_wait2(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(0)\n" : "+v"(a), "+v"(b));
}

// FP4 weights, 4 column tiles: weight vectors, scale dwords, activation vectors.
template <int OB1, int OB2, int OB3, int OS1, int OS2, int OS3, int OAM>
__device__ __forceinline__ void frag_read_fp4_4(uint32_t vB, uint32_t vS, const uint32_t (&vA)[4], u32x4 (&b)[4],
                                                uint32_t (&s)[4], u32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:%22\n"
      "ds_read_b128 %2, %16 offset:%23\n"
      "ds_read_b128 %3, %16 offset:%24\n"
      "ds_read_b32 %4, %17\n"
      "ds_read_b32 %5, %17 offset:%25\n"
      "ds_read_b32 %6, %17 offset:%26\n"
      "ds_read_b32 %7, %17 offset:%27\n"
      "ds_read_b128 %8, %18\n"
      "ds_read_b128 %9, %19\n"
      "ds_read_b128 %10, %20\n"
      "ds_read_b128 %11, %21\n"
      "ds_read_b128 %12, %18 offset:%28\n"
      "ds_read_b128 %13, %19 offset:%28\n"
      "ds_read_b128 %14, %20 offset:%28\n"
      "ds_read_b128 %15, %21 offset:%28\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(vB), "v"(vS), "v"(vA[0]), "v"(vA[1]), "v"(vA[2]), "v"(vA[3]), "n"(OB1), "n"(OB2), "n"(OB3), "n"(OS1), "n"(OS2), "n"(OS3), "n"(OAM));
}

// FP4 weights, 2 column tiles.
template <int OB1, int OS1, int OAM>
__device__ __forceinline__ void frag_read_fp4_2(uint32_t vB, uint32_t vS, const uint32_t (&vA)[4], u32x4 (&b)[2],
                                                uint32_t (&s)[2], u32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %12 offset:%18\n"
      "ds_read_b32 %2, %13\n"
      "ds_read_b32 %3, %13 offset:%19\n"
      "ds_read_b128 %4, %14\n"
      "ds_read_b128 %5, %15\n"
      "ds_read_b128 %6, %16\n"
      "ds_read_b128 %7, %17\n"
      "ds_read_b128 %8, %14 offset:%20\n"
      "ds_read_b128 %9, %15 offset:%20\n"
      "ds_read_b128 %10, %16 offset:%20\n"
      "ds_read_b128 %11, %17 offset:%20\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(s[0]), "=&v"(s[1]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(vB), "v"(vS), "v"(vA[0]), "v"(vA[1]), "v"(vA[2]), "v"(vA[3]), "n"(OB1), "n"(OS1), "n"(OAM));
}

// MXFP4 weights with split activations, 4 column tiles: as frag_read_fp4_4
// plus the activation scale dwords of the wave's two row tiles.  The second
// row tile's activation vectors (a[4..7], read last) may still be in flight
// on return: frag_wait4 completes them before their first use, so the first
// row tile's MFMAs run while they arrive.
template <int OB1, int OB2, int OB3, int OS1, int OS2, int OS3, int OAM, int OAS>
__device__ __forceinline__ void frag_read_mx_4(uint32_t vB, uint32_t vS, uint32_t vAS, const uint32_t (&vA)[4],
                                               u32x4 (&b)[4], uint32_t (&s)[4], uint32_t (&as)[2], u32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %18\n"
      "ds_read_b128 %1, %18 offset:%25\n"
      "ds_read_b128 %2, %18 offset:%26\n"
      "ds_read_b128 %3, %18 offset:%27\n"
      "ds_read_b32 %4, %19\n"
      "ds_read_b32 %5, %19 offset:%28\n"
      "ds_read_b32 %6, %19 offset:%29\n"
      "ds_read_b32 %7, %19 offset:%30\n"
      "ds_read_b32 %8, %20\n"
      "ds_read_b32 %9, %20 offset:%32\n"
      "ds_read_b128 %10, %21\n"
      "ds_read_b128 %11, %22\n"
      "ds_read_b128 %12, %23\n"
      "ds_read_b128 %13, %24\n"
      "ds_read_b128 %14, %21 offset:%31\n"
      "ds_read_b128 %15, %22 offset:%31\n"
      "ds_read_b128 %16, %23 offset:%31\n"
      "ds_read_b128 %17, %24 offset:%31\n"
      "s_waitcnt lgkmcnt(4)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3]),
        "=&v"(as[0]), "=&v"(as[1]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7])
      : "v"(vB), "v"(vS), "v"(vAS), "v"(vA[0]), "v"(vA[1]), "v"(vA[2]), "v"(vA[3]), "n"(OB1), "n"(OB2), "n"(OB3),
        "n"(OS1), "n"(OS2), "n"(OS3), "n"(OAM), "n"(OAS));
}

// MXFP4 weights with split activations, 2 column tiles (a[4..7] as for
// frag_read_mx_4).
template <int OB1, int OS1, int OAM, int OAS>
__device__ __forceinline__ void frag_read_mx_2(uint32_t vB, uint32_t vS, uint32_t vAS, const uint32_t (&vA)[4],
                                               u32x4 (&b)[2], uint32_t (&s)[2], uint32_t (&as)[2], u32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %14\n"
      "ds_read_b128 %1, %14 offset:%21\n"
      "ds_read_b32 %2, %15\n"
      "ds_read_b32 %3, %15 offset:%22\n"
      "ds_read_b32 %4, %16\n"
      "ds_read_b32 %5, %16 offset:%24\n"
      "ds_read_b128 %6, %17\n"
      "ds_read_b128 %7, %18\n"
      "ds_read_b128 %8, %19\n"
      "ds_read_b128 %9, %20\n"
      "ds_read_b128 %10, %17 offset:%23\n"
      "ds_read_b128 %11, %18 offset:%23\n"
      "ds_read_b128 %12, %19 offset:%23\n"
      "ds_read_b128 %13, %20 offset:%23\n"
      "s_waitcnt lgkmcnt(4)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(s[0]), "=&v"(s[1]), "=&v"(as[0]), "=&v"(as[1]), "=&v"(a[0]), "=&v"(a[1]),
        "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(vB), "v"(vS), "v"(vAS), "v"(vA[0]), "v"(vA[1]), "v"(vA[2]), "v"(vA[3]), "n"(OB1), "n"(OS1), "n"(OAM),
        "n"(OAS));
}

// MXFP4 weights with MXFP8 activations, 4 column tiles: FP4 weight vectors
// and scale dwords, the activation scale dwords of the two row tiles, and two
// activation vectors per row tile.
template <int OB1, int OB2, int OB3, int OS1, int OS2, int OS3, int OAM, int OAS>
__device__ __forceinline__ void frag_read_mx8_4(uint32_t vB, uint32_t vS, uint32_t vAS, uint32_t vA0, uint32_t vA1,
                                                u32x4 (&b)[4], uint32_t (&s)[4], uint32_t (&as)[2], u32x4 (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %14\n"
      "ds_read_b128 %1, %14 offset:%19\n"
      "ds_read_b128 %2, %14 offset:%20\n"
      "ds_read_b128 %3, %14 offset:%21\n"
      "ds_read_b32 %4, %15\n"
      "ds_read_b32 %5, %15 offset:%22\n"
      "ds_read_b32 %6, %15 offset:%23\n"
      "ds_read_b32 %7, %15 offset:%24\n"
      "ds_read_b32 %8, %16\n"
      "ds_read_b32 %9, %16 offset:%26\n"
      "ds_read_b128 %10, %17\n"
      "ds_read_b128 %11, %18\n"
      "ds_read_b128 %12, %17 offset:%25\n"
      "ds_read_b128 %13, %18 offset:%25\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3]),
        "=&v"(as[0]), "=&v"(as[1]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(vB), "v"(vS), "v"(vAS), "v"(vA0), "v"(vA1), "n"(OB1), "n"(OB2), "n"(OB3), "n"(OS1), "n"(OS2), "n"(OS3),
        "n"(OAM), "n"(OAS));
}

// Fragment groups of the software-pipelined MXFP8-activation stage (read
// while the previous stage's MFMAs run): the four weight vectors; the
// weight and activation scale dwords; the two activation vectors of one row
// tile.
template <int OB1, int OB2, int OB3>
__device__ __forceinline__ void frag_read_b4(uint32_t vB, u32x4 (&b)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:%5\n"
      "ds_read_b128 %2, %4 offset:%6\n"
      "ds_read_b128 %3, %4 offset:%7\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
      : "v"(vB), "n"(OB1), "n"(OB2), "n"(OB3));
}

template <int OS1, int OS2, int OS3, int OAS>
__device__ __forceinline__ void frag_read_sc(uint32_t vS, uint32_t vAS, uint32_t (&s)[4], uint32_t (&as)[2]) {
  asm volatile(
      "ds_read_b32 %0, %6\n"
      "ds_read_b32 %1, %6 offset:%8\n"
      "ds_read_b32 %2, %6 offset:%9\n"
      "ds_read_b32 %3, %6 offset:%10\n"
      "ds_read_b32 %4, %7\n"
      "ds_read_b32 %5, %7 offset:%11\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3]), "=&v"(as[0]), "=&v"(as[1])
      : "v"(vS), "v"(vAS), "n"(OS1), "n"(OS2), "n"(OS3), "n"(OAS));
}

template <int OFF>
__device__ __forceinline__ void frag_read_a2(uint32_t vA0, uint32_t vA1, u32x4& a0, u32x4& a1) {
  asm volatile(
      "ds_read_b128 %0, %2 offset:%4\n"
      "ds_read_b128 %1, %3 offset:%4\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(a0), "=&v"(a1)
      : "v"(vA0), "v"(vA1), "n"(OFF));
}

// BF16 weights (and activations), 2 column tiles: four vectors per operand
// row, one per MFMA step, at per-lane offsets (the swizzle differs per step).
template <int OB1, int OAM>
__device__ __forceinline__ void frag_read_bf16w_2(const uint32_t (&vB)[4], const uint32_t (&vA)[4], u32x4 (&b)[8],
                                                  u32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %17\n"
      "ds_read_b128 %2, %18\n"
      "ds_read_b128 %3, %19\n"
      "ds_read_b128 %4, %16 offset:%24\n"
      "ds_read_b128 %5, %17 offset:%24\n"
      "ds_read_b128 %6, %18 offset:%24\n"
      "ds_read_b128 %7, %19 offset:%24\n"
      "ds_read_b128 %8, %20\n"
      "ds_read_b128 %9, %21\n"
      "ds_read_b128 %10, %22\n"
      "ds_read_b128 %11, %23\n"
      "ds_read_b128 %12, %20 offset:%25\n"
      "ds_read_b128 %13, %21 offset:%25\n"
      "ds_read_b128 %14, %22 offset:%25\n"
      "ds_read_b128 %15, %23 offset:%25\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7]),
        "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(vB[0]), "v"(vB[1]), "v"(vB[2]), "v"(vB[3]), "v"(vA[0]), "v"(vA[1]), "v"(vA[2]), "v"(vA[3]), "n"(OB1),
        "n"(OAM));
}

// FP8 weights and activations, 4 column tiles: two vectors per operand row.
// The second row tile's activation vectors (a[2], a[3], read last) may still
// be in flight on return: frag_wait2 completes them before their first use.
template <int OB1, int OB2, int OB3, int OAM>
__device__ __forceinline__ void frag_read_fp8_4(uint32_t vB0, uint32_t vB1, uint32_t vA0, uint32_t vA1, u32x4 (&b)[8],
                                                u32x4 (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %13\n"
      "ds_read_b128 %2, %12 offset:%16\n"
      "ds_read_b128 %3, %13 offset:%16\n"
      "ds_read_b128 %4, %12 offset:%17\n"
      "ds_read_b128 %5, %13 offset:%17\n"
      "ds_read_b128 %6, %12 offset:%18\n"
      "ds_read_b128 %7, %13 offset:%18\n"
      "ds_read_b128 %8, %14\n"
      "ds_read_b128 %9, %15\n"
      "ds_read_b128 %10, %14 offset:%19\n"
      "ds_read_b128 %11, %15 offset:%19\n"
      "s_waitcnt lgkmcnt(2)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
      : "v"(vB0), "v"(vB1), "v"(vA0), "v"(vA1), "n"(OB1), "n"(OB2), "n"(OB3), "n"(OAM));
}

// FP8 weights with bf16 activations, 4 column tiles.
template <int OB1, int OB2, int OB3, int OAM>
__device__ __forceinline__ void frag_read_fp8_bf16_4(uint32_t vB0, uint32_t vB1, const uint32_t (&vA)[4], u32x4 (&b)[8],
                                                     u32x4 (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %17\n"
      "ds_read_b128 %2, %16 offset:%22\n"
      "ds_read_b128 %3, %17 offset:%22\n"
      "ds_read_b128 %4, %16 offset:%23\n"
      "ds_read_b128 %5, %17 offset:%23\n"
      "ds_read_b128 %6, %16 offset:%24\n"
      "ds_read_b128 %7, %17 offset:%24\n"
      "ds_read_b128 %8, %18\n"
      "ds_read_b128 %9, %19\n"
      "ds_read_b128 %10, %20\n"
      "ds_read_b128 %11, %21\n"
      "ds_read_b128 %12, %18 offset:%25\n"
      "ds_read_b128 %13, %19 offset:%25\n"
      "ds_read_b128 %14, %20 offset:%25\n"
      "ds_read_b128 %15, %21 offset:%25\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3]), "=&v"(b[4]), "=&v"(b[5]), "=&v"(b[6]), "=&v"(b[7]), "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
      : "v"(vB0), "v"(vB1), "v"(vA[0]), "v"(vA[1]), "v"(vA[2]), "v"(vA[3]), "n"(OB1), "n"(OB2), "n"(OB3), "n"(OAM));
}

__device__ __forceinline__ uint4 to_u4(const u32x4& v) { return make_uint4(v.x, v.y, v.z, v.w); }

// bf16 operand of MFMA step t from a lane's weight bytes of the stage:
// FP4 c0 = 32 nibbles ([32g, 32g+32)), FP8 c0|c1 = 32 bytes.
template <int WFMT>
__device__ __forceinline__ bf16x8 weight_bf16(const uint4& c0, const uint4& c1, uint32_t sc, int t) {
  uint32_t o[4];
  if constexpr (WFMT == kFP8) {
    const uint4 c = t < 2 ? c0 : c1;
    fp8x4_to_bf16((t & 1) ? c.z : c.x, o);
    fp8x4_to_bf16((t & 1) ? c.w : c.y, o + 2);
  } else {
    const uint32_t word = t == 0 ? c0.x : t == 1 ? c0.y : t == 2 ? c0.z : c0.w;
    if constexpr (WFMT == kMXFP4) {
      fp4x8_to_bf16(word, e8m0_as_scale(sc & 0xFF), o);
    } else {
      const float s = e4m3_to_f32((sc >> (t < 2 ? 0 : 8)) & 0xFF);
      fp4x8_to_bf16_nv(word, s, nv_scale_significand(s), o);
    }
  }
  return __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
}

// ------------------------------------------------------------- kernel ----
struct GemmArgs {
  QW w;
  Rows rows;
  const uint8_t* a;          // activation rows: bf16 (x or h), E4M3 (x_q or h_q) or split E4M3 (MXFP4)
  const uint8_t* a_sc;       // MXFP4: E8M0 scales of the split / MXFP8 activations [rows][a_sc_pitch]
  int a_sc_pitch;
  int K;                     // reduction length (H for gate_up, I for down)
  int N;                     // gate_up: I (gate columns); down: H (output columns)
  int a_row_bytes;           // bytes per activation row
  const uint32_t* amax_a;    // FP8 activations: amax bits of the activation tensor
  void* out;                 // gate_up: h [rows][I] (bf16, or split E4M3 / MXFP8 for MXFP4); down: o [flat][H] bf16
  uint8_t* out_sc;           // gate_up, MXFP4: E8M0 scales of h [rows][out_sc_pitch]
  int out_sc_pitch;
  uint32_t* amax_slots;      // gate_up with FP8 activations: partial maxima of |h|
};

template <int WFMT, bool FP8ACT, int BM, bool GATEUP, bool PERSIST, bool WIDE = false>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs ga) {
  using C = Cfg<WFMT, FP8ACT, BM, WIDE>;
  constexpr int NT = C::kNT;
  // MXFP8 activations: fragments of the next stage are read while the
  // current stage's MFMAs run (two register sets)
  constexpr bool kPipe = C::kAScales && FP8ACT;
  constexpr int kAhead = kPipe ? C::kRing : C::kRing - 1;   // stages in flight ahead of the MFMA work
  __shared__ __attribute__((aligned(16))) uint8_t ring[C::kRing * C::kSlotBytes];

  const Rows& rows = ga.rows;
  const QW& w = ga.w;
  const int K = ga.K, N = ga.N;
  const int ntile = GATEUP ? (N + C::kBN / 2 - 1) / (C::kBN / 2) : (N + C::kBN - 1) / C::kBN;
  const int total = rows.num_blocks * ntile;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int wm = wave % C::kWM, wn = wave / C::kWM;
  const int arow0 = wm * 64;
  const int j = lane & 31, g = lane >> 5;
  const int ns = K / kStageK;

  // weight row (within the expert's matrix) of tile row R of column tile nt,
  // or -1 past N.  A tile of kSub packed tiles holds them one after another
  // (gate_up: each packed tile pairs its gate rows with the matching up rows).
  auto tile_col = [&](int nt, int R) -> int {
    if constexpr (C::kSub > 1) {
      nt = C::kSub * nt + R / C::kTileW;
      R %= C::kTileW;
    }
    if constexpr (GATEUP) {
      const int half = C::kTileW / 2;
      const int c = nt * half + (R < half ? R : R - half);
      if (c >= N) return -1;
      return R < half ? c : N + c;
    } else {
      const int c = nt * C::kTileW + R;
      return c < N ? c : -1;
    }
  };
  // first tile row of each of this wave's column tiles: gate_up pairs gate
  // tile u with up tile u + NT/2; down takes NT consecutive tiles
  int Rt[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    if constexpr (GATEUP) {
      constexpr int kWps = C::kWN / C::kSub;   // waves per packed tile
      Rt[ct] = (wn / kWps) * C::kTileW + (ct < NT / 2 ? 0 : C::kTileW / 2) + 32 * ((wn % kWps) * (NT / 2) + ct % (NT / 2));
    } else
      Rt[ct] = 32 * (wn * NT + ct);
  }

  // ---- the workgroup's tiles ----
  // Tile k of this workgroup is logical_tile(blockIdx.x + k * gridDim.x):
  // ascending in k, and the grid is a multiple of 8 workgroups, so every
  // tile of a workgroup comes from its own XCD's chunks.  The sequence ends
  // at `total` or at the first block without an expert (the padding blocks
  // are at the end of the list).
  // Within one expert's run of row blocks the (block, tile) pairs go tile by
  // tile: t / ntile is a block of the expert that owns pair t (the run of an
  // expert with nb blocks spans nb * ntile pairs), and the pair's place in
  // that run gives the column tile and then the block.  A chunk of pairs on
  // one XCD then holds a weight tile across many row blocks (reused from its
  // L2) rather than every tile of a few blocks.
  auto tile_bnt = [&](int k, int& b, int& nt) -> bool {
    const int t = logical_tile(static_cast<int>(blockIdx.x) + k * static_cast<int>(gridDim.x));
    if (t >= total) return false;
    int first = 0, nb = rows.num_blocks;
    if (rows.sorted_ids) {
      const int e = rows.block_expert[t / ntile];
      if (e < 0) {   // padding blocks past the last expert's run: exits at once
        b = t / ntile;
        nt = t % ntile;
        return true;
      }
      first = rows.offsets[e] / BM;
      nb = rows.offsets[e + 1] / BM - first;
    }
    const int local = t - first * ntile;
    nt = local / nb;
    b = first + local % nb;
    return true;
  };
  // The sorted row ids of a tile's block are copied into LDS (meta[k & 1]) by
  // wave 0 while the tile before it is fetched, so that no register holds
  // them across the stages.
  __shared__ __attribute__((aligned(16))) int meta[2][BM];
  const int* const sid = rows.sorted_ids;
  auto meta_fetch = [&](int k, int b) {
    if (sid && wave == 0 && lane < BM / 4) dma16(sid + b * BM + 4 * lane, reinterpret_cast<uint8_t*>(meta[k & 1]));
  };
  // sorted id of tile row r of tile k (from LDS), or of block b directly
  auto meta_row = [&](int k, int r) -> int { return lds_i32(lds_addr(&meta[k & 1][r])); };
  // activation row of a sorted id, or of tile row r of block b without sorted ids
  auto act_row = [&](int f, int b, int r) -> int {
    if (GATEUP && sid) return f < rows.n_flat ? f / rows.top_k : 0;
    if (GATEUP) {
      const int p = b * BM + r;
      return p < rows.n_flat ? p : 0;
    }
    return b * BM + r;   // h rows of the block (padding rows hold unused values)
  };

  // ---- DMA side: the tile whose stages are being fetched ----
  // 32-bit per-lane offsets from uniform bases (one expert's matrix < 4 GiB)
  const size_t wrows = static_cast<size_t>(GATEUP ? 2 * N : N);
  const uint32_t wrow_bytes = WFMT == kBF16 ? 2u * static_cast<uint32_t>(K)
                              : WFMT == kFP8 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(K) / 2;
  // Weight stages come from the row-major matrices, or from the packed tile
  // layout, where a stage of this tile is one contiguous run: codes in LDS
  // order, then (FP4) one scale dword per tile row.
  const bool packed = w.packed != nullptr;
  constexpr uint32_t kPackStage = packed_stage_bytes(WFMT);
  const uint32_t badv = packed ? kPackStage : C::kBRowB;   // weight source advance per stage
  const uint32_t spitch = WFMT == kMXFP4 ? K / 32 : K / 16;  // row-major block-scale bytes per row
  const uint8_t* wbase = nullptr;   // the tile's weight stages
  const uint8_t* sbase = nullptr;   // its block scales
  uint32_t src[C::kChunksPerWave];
  uint32_t soff = 0, aoff = 0;      // this lane's block-scale and activation-scale offsets
  uint32_t soff2 = 0;               // (second scale row group, kScaleInstr == 2)
  // packed tiles per expert matrix, and the distance between consecutive ones
  const int ptiles = C::kSub == 1 ? ntile : GATEUP ? (N + C::kTileW / 2 - 1) / (C::kTileW / 2) : (N + C::kTileW - 1) / C::kTileW;
  const uint32_t ptile_bytes = static_cast<uint32_t>(ns) * kPackStage;
  int dnext = 0;        // next stage of the DMA tile
  bool dlive = false;   // the DMA tile exists (else stages are refetched into buffers nobody reads)
  // sources of tile k (block b, column tile nt, expert e); f(r) gives the
  // sorted id of tile row r
  auto set_sources = [&](int b, int nt, int e, auto f) {
    wbase = packed ? w.packed + (static_cast<size_t>(e) * ptiles + C::kSub * nt) * ns * kPackStage
                   : w.codes + static_cast<size_t>(e) * wrows * wrow_bytes;
    // packed tile q of the workgroup tile (past the matrix's last: its first, unused)
    auto sub_off = [&](int q) -> uint32_t {
      if constexpr (C::kSub == 1) return 0u;
      return C::kSub * nt + q < ptiles ? q * ptile_bytes : 0u;
    };
#pragma unroll
    for (int i = 0; i < C::kChunksPerWave; ++i) {
      const int c = wave + kGemmWaves * i;
      if (c < C::kAChunks) {
        const int v = c * 64 + lane;
        const int r = v / C::kAV;
        src[i] = static_cast<uint32_t>(act_row(f(r), b, r)) * ga.a_row_bytes + 16 * swz<C::kAV>(r, v % C::kAV);
      } else {
        const int v = (c - C::kAChunks) * 64 + lane;
        const int R = v / C::kBV, q = swz<C::kBV>(R, v % C::kBV);
        const int col = tile_col(nt, R);
        constexpr int kSubV = C::kTileW * C::kBV;   // 16-byte vectors of one packed tile's stage
        src[i] = packed ? sub_off(v / kSubV) + 16u * static_cast<uint32_t>(v % kSubV)
                        : static_cast<uint32_t>(col < 0 ? 0 : col) * wrow_bytes + 16 * q;
      }
    }
    // Block scales: lanes l < kScaleRowsPerWave of wave w fetch the scale
    // dword of tile row w * kScaleRowsPerWave + l per stage (for MXFP4 it
    // holds the scales of two stages, for NVFP4 those of one; the byte is
    // picked at use).
    if constexpr (C::kScales) {
      const int R = wave * C::kScaleRowsPerWave + (lane < C::kScaleRowsPerWave ? lane : 0);
      const int R2 = R + 64;   // second instruction's row (kScaleInstr == 2)
      if (packed) {
        sbase = wbase;
        soff = sub_off(R / C::kTileW) + C::kTileW * C::kBRowB + 4 * (R % C::kTileW);
        if constexpr (C::kScaleInstr == 2) soff2 = sub_off(R2 / C::kTileW) + C::kTileW * C::kBRowB + 4 * (R2 % C::kTileW);
      } else {
        const int col = tile_col(nt, R);
        sbase = w.scales + static_cast<size_t>(e) * wrows * spitch;
        soff = static_cast<uint32_t>(col < 0 ? 0 : col) * spitch;
        if constexpr (C::kScaleInstr == 2) {
          const int col2 = tile_col(nt, R2);
          soff2 = static_cast<uint32_t>(col2 < 0 ? 0 : col2) * spitch;
        }
      }
    }
    // Activation scales (MXFP4): lanes l < kARowsPerWave of wave w fetch the
    // scale dword of tile row w * kARowsPerWave + l (two stages).
    if constexpr (C::kAScales) {
      const int r = wave * C::kARowsPerWave + (lane < C::kARowsPerWave ? lane : 0);
      aoff = static_cast<uint32_t>(act_row(f(r), b, r)) * ga.a_sc_pitch;
    }
    dnext = 0;
  };

  // ---- compute side: the tile whose MFMA work runs (ce: its matrix slot) ----
  int cb = 0, cnt = 0, ce = 0, cflat = 0, nvalid = 0;
  bool wact = false, rows_ok[2] = {false, false};
  auto enter = [&](int b, int nt, int e, int nv, int flat) {
    cb = b;
    cnt = nt;
    ce = e;
    cflat = flat;
    nvalid = nv;
    wact = tile_col(cnt, Rt[0]) >= 0;
    rows_ok[0] = wact && arow0 < nvalid;
    rows_ok[1] = wact && arow0 + 32 < nvalid;
  };

  // first tile: metadata straight from global memory
  int dk = 0;   // sequence number of the DMA tile
  {
    int b, nt;
    if (!tile_bnt(0, b, nt)) return;
    const int e = sid ? rows.block_expert[b] : 0;
    if (e < 0) return;
    const int slot = expert_slot(w, e);   // slot of its matrices (< 0: served by another pass)
    if (slot < 0) return;
    auto fsid = [&](int r) -> int { return sid ? sid[b * BM + r] : 0; };
    set_sources(b, nt, slot, fsid);
    dlive = true;
    int flat = 0;
    if constexpr (!GATEUP) flat = sid ? sid[b * BM + arow0 + lane] : b * BM + arow0 + lane;
    enter(b, nt, slot, block_rows(rows, b, e, BM), flat);
  }
  // the tile after the DMA tile: block, column tile, expert (uniform)
  int nb = 0, nnt = 0, ne = -1;
  if constexpr (PERSIST) {
    const bool nok0 = tile_bnt(1, nb, nnt);
    ne = nok0 ? (sid ? rows.block_expert[nb] : 0) : -1;
    if (nok0) meta_fetch(1, nb);
  }
  // the compute side's next tile, once the DMA side reached it
  int qb = 0, qnt = 0, qe = 0, qnv = 0;
  bool have_next = false;

  // After the DMA tile's last stage has been issued, the fetching continues
  // with the workgroup's next tile (called at the step whose issue would be
  // its first stage); past the last tile the sources stop advancing and the
  // last stage is fetched again into buffers nobody reads.
  auto next_dma_tile = [&]() {
    if (PERSIST && ne >= 0) {
      ++dk;
      const int k = dk;
      // (persistent launches have no slot table: the slot is the expert)
      set_sources(nb, nnt, ne, [&](int r) -> int { return sid ? meta_row(k, r) : 0; });
      qb = nb;
      qnt = nnt;
      qe = ne;
      qnv = block_rows(rows, nb, ne, BM);
      have_next = true;
      const bool ok = tile_bnt(dk + 1, nb, nnt);
      ne = ok ? (sid ? rows.block_expert[nb] : 0) : -1;
      if (ok) meta_fetch(dk + 1, nb);
    } else {
      dlive = false;
    }
  };

  // Issues the next stage into `buf`: the wave's DMA chunks, then its scale
  // rows.  Every step issues exactly one stage, so the number of memory
  // operations in flight per stage is a constant.
  auto issue = [&](uint8_t* buf) {
    const int cur_stage = dnext;
    const bool adv = dlive && dnext + 1 < ns;
    dnext += dnext < ns ? 1 : 0;
#pragma unroll
    for (int i = 0; i < C::kChunksPerWave; ++i) {
      const int c = wave + kGemmWaves * i;
      dma16((c < C::kAChunks ? ga.a : wbase) + src[i], buf + c * 1024);
      src[i] += adv ? (c < C::kAChunks ? static_cast<uint32_t>(C::kARowB) : badv) : 0;
    }
    if constexpr (C::kScales) {
      if (lane < C::kScaleRowsPerWave) dma4(sbase + soff, buf + C::kABytes + C::kBBytes + wave * 4 * C::kScaleRowsPerWave);
      if constexpr (C::kScaleInstr == 2)
        dma4(sbase + soff2, buf + C::kABytes + C::kBBytes + wave * 4 * C::kScaleRowsPerWave + 256);
      // row-major MXFP4: stages 2m and 2m + 1 share the dword at 4m
      const uint32_t sadv = packed ? (adv ? kPackStage : 0) : (adv && (WFMT == kNVFP4 || (cur_stage & 1)) ? 4 : 0);
      soff += sadv;
      if constexpr (C::kScaleInstr == 2) soff2 += sadv;
    }
    if constexpr (C::kAScales) {
      if (lane < C::kARowsPerWave)
        dma4(ga.a_sc + aoff, buf + C::kABytes + C::kBBytes + C::kSBytes + wave * 4 * C::kARowsPerWave);
      aoff += adv && (cur_stage & 1) ? 4 : 0;
    }
  };

  // Per-lane fragment addresses within a ring buffer: the first weight row
  // and the first activation row of the wave; the other column and row tiles
  // are 32 rows further on, where the swizzle repeats, so they are reached
  // through immediate offsets of the same read instructions.
  const int RB = Rt[0] + j, RA = arow0 + j;
  const uint32_t brow = C::kABytes + RB * C::kBRowB, arow = RA * C::kARowB;
  uint32_t bo[4], ao[4];
  const uint32_t so = C::kABytes + C::kBBytes + 4 * RB;
  const uint32_t sao = C::kABytes + C::kBBytes + C::kSBytes + 4 * RA;
  if constexpr (WFMT == kBF16) {
    // K [32g + 8t, 32g + 8t + 8) of a row at MFMA step t, as for the activations
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) bo[tt] = brow + 16 * swz<C::kBV>(RB, 4 * g + tt);
  } else if constexpr (WFMT != kFP8) {
    bo[0] = bo[1] = brow + 16 * swz<C::kBV>(RB, g);
  } else if constexpr (FP8ACT) {
    bo[0] = brow + 16 * swz<C::kBV>(RB, g);
    bo[1] = brow + 16 * swz<C::kBV>(RB, 2 + g);
  } else {
    bo[0] = brow + 16 * swz<C::kBV>(RB, 2 * g);
    bo[1] = brow + 16 * swz<C::kBV>(RB, 2 * g + 1);
  }
  if constexpr (FP8ACT) {
    ao[0] = arow + 16 * swz<C::kAV>(RA, g);
    ao[1] = arow + 16 * swz<C::kAV>(RA, 2 + g);
    ao[2] = ao[3] = ao[0];
  } else if constexpr (C::kSplitA) {
    // The 8-bit operand of the scaled 32x32x64 MFMA holds K [16g, 16g + 16)
    // and [32 + 16g, 48 + 16g) in lane group g (hi vectors g, 2 + g; lo
    // vectors 4 + g, 6 + g), while the 4-bit operand holds K [32g, 32g + 32);
    // the scale of K block b (32 wide) is the one lane group b supplies.
    ao[0] = arow + 16 * swz<C::kAV>(RA, g);
    ao[1] = arow + 16 * swz<C::kAV>(RA, 2 + g);
    ao[2] = arow + 16 * swz<C::kAV>(RA, 4 + g);
    ao[3] = arow + 16 * swz<C::kAV>(RA, 6 + g);
  } else {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) ao[tt] = arow + 16 * swz<C::kAV>(RA, 4 * g + tt);
  }
  // tile-row distances of this wave's column tiles from the first
  constexpr int kHalf = C::kBN / 2;
  constexpr int kUpD = C::kTileW / 2;   // gate_up: tile rows from a gate row to its up row
  constexpr int kD1 = GATEUP ? (NT == 4 ? 32 : kUpD) : 32;
  constexpr int kD2 = GATEUP ? kUpD : 64;
  constexpr int kD3 = GATEUP ? kUpD + 32 : 96;
  constexpr int kOAM = 32 * C::kARowB;
  constexpr int kBVec = WFMT == kBF16 ? 4 * NT : WFMT == kFP8 ? 2 * NT : NT;
  constexpr int kAVec = FP8ACT ? 4 : 8;

  f32x16 acc[2][NT];

  // One stage of the compute tile from ring buffer `cur`: wait for its DMA,
  // barrier, read the fragments, refill the buffer the previous stage used,
  // then the MFMA work.
  auto step = [&](int s, uint8_t* cur, uint8_t* refill) {
    if constexpr (!kPipe) {
    wait_vm<C::kVmPerStage * (C::kRing - 2)>();
    stage_barrier();
    const uint32_t base = lds_addr(cur);
    u32x4 bv[kBVec], av[kAVec];
    uint32_t scw[NT], asw[2];
    if constexpr (C::kSplitA) {
      const uint32_t vA[4] = {base + ao[0], base + ao[1], base + ao[2], base + ao[3]};
      if constexpr (NT == 4)
        frag_read_mx_4<kD1 * C::kBRowB, kD2 * C::kBRowB, kD3 * C::kBRowB, kD1 * 4, kD2 * 4, kD3 * 4, kOAM, 32 * 4>(
            base + bo[0], base + so, base + sao, vA, bv, scw, asw, av);
      else
        frag_read_mx_2<kD1 * C::kBRowB, kD1 * 4, kOAM, 32 * 4>(base + bo[0], base + so, base + sao, vA, bv, scw, asw,
                                                               av);
    } else if constexpr (WFMT == kBF16) {
      static_assert(NT == 2, "BF16 weight tiles");
      const uint32_t vA[4] = {base + ao[0], base + ao[1], base + ao[2], base + ao[3]};
      const uint32_t vB[4] = {base + bo[0], base + bo[1], base + bo[2], base + bo[3]};
      frag_read_bf16w_2<kD1 * C::kBRowB, kOAM>(vB, vA, bv, av);
    } else if constexpr (WFMT != kFP8) {
      const uint32_t vA[4] = {base + ao[0], base + ao[1], base + ao[2], base + ao[3]};
      if constexpr (NT == 4)
        frag_read_fp4_4<kD1 * C::kBRowB, kD2 * C::kBRowB, kD3 * C::kBRowB, kD1 * 4, kD2 * 4, kD3 * 4, kOAM>(
            base + bo[0], base + so, vA, bv, scw, av);
      else
        frag_read_fp4_2<kD1 * C::kBRowB, kD1 * 4, kOAM>(base + bo[0], base + so, vA, bv, scw, av);
    } else if constexpr (FP8ACT) {
      frag_read_fp8_4<kD1 * C::kBRowB, kD2 * C::kBRowB, kD3 * C::kBRowB, kOAM>(base + bo[0], base + bo[1],
                                                                               base + ao[0], base + ao[1], bv, av);
    } else {
      const uint32_t vA[4] = {base + ao[0], base + ao[1], base + ao[2], base + ao[3]};
      frag_read_fp8_bf16_4<kD1 * C::kBRowB, kD2 * C::kBRowB, kD3 * C::kBRowB, kOAM>(base + bo[0], base + bo[1], vA,
                                                                                    bv, av);
    }
    issue(refill);
    if constexpr (C::kSplitA) {
      // the E8M0 bytes of this lane's K block: byte 2 (s & 1) + g of the dwords
      const int sh = 16 * (s & 1) + 8 * g;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m == 1) frag_wait4(av[4], av[5], av[6], av[7]);   // (unconditional: the reads are in flight)
        if (!rows_ok[m]) continue;
        const int sa = static_cast<int>(asw[m] >> sh);
        const i32x8 ah = u4x2(to_u4(av[4 * m]), to_u4(av[4 * m + 1]));
        const i32x8 al = u4x2(to_u4(av[4 * m + 2]), to_u4(av[4 * m + 3]));
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const uint4 c = to_u4(bv[ct]);
          const i32x8 bq = {static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z), static_cast<int>(c.w),
                            0, 0, 0, 0};
          const int sb = static_cast<int>(scw[ct] >> sh);
          // lo codes carry 2^4 times the residual: scale exponent lowered by 4
          // (split scales are at least 4, so the low byte does not borrow)
          acc[m][ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ah, bq, acc[m][ct], 0, 4, 0, sa, 0, sb);
          acc[m][ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(al, bq, acc[m][ct], 0, 4, 0, sa - 4, 0, sb);
        }
      }
    } else if constexpr (FP8ACT && WFMT == kFP8) {
      i32x8 bq[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) bq[ct] = u4x2(to_u4(bv[2 * ct]), to_u4(bv[2 * ct + 1]));
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m == 1) frag_wait2(av[2], av[3]);   // (unconditional: the reads are in flight)
        if (!rows_ok[m]) continue;
        const i32x8 a = u4x2(to_u4(av[2 * m]), to_u4(av[2 * m + 1]));
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          acc[m][ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq[ct], acc[m][ct], 0, 0, 0, 127, 0, 127);
      }
    } else {
      // this lane's scale byte(s): MXFP4 byte 2 (s & 1) + g, NVFP4 bytes 2g, 2g + 1
      const int sh = WFMT == kMXFP4 ? 16 * (s & 1) + 8 * g : 16 * g;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          bf16x8 bt;
          if constexpr (WFMT == kBF16)
            bt = __builtin_bit_cast(bf16x8, to_u4(bv[4 * ct + tt]));
          else if constexpr (WFMT == kFP8)
            bt = weight_bf16<WFMT>(to_u4(bv[2 * ct]), to_u4(bv[2 * ct + 1]), 0, tt);
          else
            bt = weight_bf16<WFMT>(to_u4(bv[ct]), to_u4(bv[ct]), scw[ct] >> sh, tt);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            if (!rows_ok[m]) continue;
            const bf16x8 a = __builtin_bit_cast(bf16x8, to_u4(av[4 * m + tt]));
            acc[m][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bt, acc[m][ct], 0, 0, 0);
          }
        }
      }
    }
    }
  };

  // MXFP8 activations: the fragments of stage s are in registers when step s
  // starts; its MFMAs are issued in four groups, and between them the
  // fragments of the next stage are read into the other register set.  The
  // buffer of stage s is refilled at step s, after the barrier that follows
  // every wave's reads of it in step s - 1.
  struct Frag {
    u32x4 b[4];
    uint32_t s[4], as[2];
    u32x4 a[4];
  };
  Frag fr[2];
  auto read_frags = [&](uint32_t base, Frag& f, int part) {
    if constexpr (kPipe) {
      if (part == 0) frag_read_b4<kD1 * C::kBRowB, kD2 * C::kBRowB, kD3 * C::kBRowB>(base + bo[0], f.b);
      if (part == 1) frag_read_sc<kD1 * 4, kD2 * 4, kD3 * 4, 32 * 4>(base + so, base + sao, f.s, f.as);
      if (part == 2) frag_read_a2<0>(base + ao[0], base + ao[1], f.a[0], f.a[1]);
      if (part == 3) frag_read_a2<kOAM>(base + ao[0], base + ao[1], f.a[2], f.a[3]);
    }
  };
  auto pipe_step = [&](int s, Frag& cur, Frag& nxt, uint8_t* refill, uint8_t* nextbuf) {
    if constexpr (kPipe) {
      wait_vm<C::kVmPerStage * (C::kRing - 2)>();
      stage_barrier();
      issue(refill);
      const int sh = 16 * (s & 1) + 8 * g;
      int sa[2], sb[4];
#pragma unroll
      for (int m = 0; m < 2; ++m) sa[m] = static_cast<int>(cur.as[m] >> sh);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) sb[ct] = static_cast<int>(cur.s[ct] >> sh);
      const i32x8 a[2] = {u4x2(to_u4(cur.a[0]), to_u4(cur.a[1])), u4x2(to_u4(cur.a[2]), to_u4(cur.a[3]))};
      const uint32_t base = lds_addr(nextbuf);
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int m = grp >> 1;
        if (rows_ok[m]) {
#pragma unroll
          for (int ct = 2 * (grp & 1); ct < 2 * (grp & 1) + 2; ++ct) {
            const uint4 c = to_u4(cur.b[ct]);
            const i32x8 bq = {static_cast<int>(c.x), static_cast<int>(c.y), static_cast<int>(c.z),
                              static_cast<int>(c.w), 0, 0, 0, 0};
            acc[m][ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[m], bq, acc[m][ct], 0, 4, 0, sa[m], 0, sb[ct]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        read_frags(base, nxt, grp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- prologue: the first kAhead stages, then (pipelined) stage 0's fragments ----
  uint32_t G = 0;   // global stage number of the compute side (ring position)
  auto buf_of = [&](uint32_t stage) -> uint8_t* { return ring + (stage % C::kRing) * C::kSlotBytes; };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) issue(buf_of(i));
  if constexpr (kPipe) {
    static_assert(C::kRing % 2 == 0 && NT == 4, "pipelined stages");
    wait_vm<C::kVmPerStage * (C::kRing - 1)>();
    stage_barrier();
#pragma unroll
    for (int part = 0; part < 4; ++part) read_frags(lds_addr(ring), fr[0], part);
  }

  for (;;) {   // compute tiles
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) acc[m][ct] = f32x16{};
    // the step at which the DMA side moves on to the next tile
    const int s_next = PERSIST && dlive ? ns - kAhead : -1;
    if constexpr (!PERSIST) {
      // one tile: ring positions known at compile time (G = 0 here)
      for (int s = 0; s < ns; s += C::kRing) {
#pragma unroll
        for (int r = 0; r < C::kRing; ++r) {
          if (s + r >= ns) break;
          if constexpr (kPipe)
            pipe_step(s + r, fr[r & 1], fr[(r + 1) & 1], ring + r * C::kSlotBytes,
                      ring + ((r + 1) % C::kRing) * C::kSlotBytes);
          else
            step(s + r, ring + r * C::kSlotBytes, ring + ((r + C::kRing - 1) % C::kRing) * C::kSlotBytes);
        }
      }
      G += ns;
    } else if constexpr (kPipe) {
      // ns is even (K is a multiple of 128) and so is G here
      for (int s = 0; s < ns; s += 2, G += 2) {
        if (s == s_next) next_dma_tile();
        pipe_step(s, fr[0], fr[1], buf_of(G), buf_of(G + 1));
        if (s + 1 == s_next) next_dma_tile();
        pipe_step(s + 1, fr[1], fr[0], buf_of(G + 1), buf_of(G + 2));
      }
    } else {
      for (int s = 0; s < ns; ++s, ++G) {
        if (s == s_next) next_dma_tile();
        step(s, buf_of(G), buf_of(G + C::kRing - 1));
      }
    }

    // ---- epilogue (registers to global memory; the ring keeps filling) ----
    const int b = cb, e = ce, nt = cnt;
    // NVFP4 / FP8: the matrix's fp32 multiplier (one, or one per row), and
    // for FP8 activations the activation scale
    float fa = 1.0f;
    if constexpr (FP8ACT && WFMT == kFP8) fa = amax_scale(ga.amax_a);
    // (gate_up runs one tile per workgroup: once the refetches are done the
    // whole ring is free for the epilogue)
    if constexpr (GATEUP && C::kAScales) {
      static_assert(!PERSIST, "the MXFP4 gate_up epilogue uses the ring");
      wait_vm<0>();
    }
    if constexpr (GATEUP && C::kAScales && FP8ACT) {
      // MXFP8 h from the fp32 accumulators: the 32 columns of a block are the
      // 32 lanes of a half-wave (one row per register), so the block maximum
      // is a half-wave reduction.  Codes and scales are collected in LDS (the
      // ring is free now) and leave as 16-byte pieces of rows.
      constexpr int kSBlk = kHalf / 32;   // scale bytes per tile row
      __syncthreads();
      uint8_t* qt = ring;                  // [BM][kHalf] codes
      uint8_t* st = ring + BM * kHalf;     // [BM][kSBlk] scale codes
#pragma unroll
      for (int u = 0; u < NT / 2; ++u) {
        const int cl = Rt[u] + j;   // column within the workgroup's half tile
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // the 16 rows of this register set at once: independent reduction
          // chains (|v| compared as integers, exact for non-negative floats)
          float v[16];
          int am[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            v[r] = swiglu(acc[m][u][r], acc[m][u + NT / 2][r]);
            am[r] = static_cast<int>(__float_as_uint(v[r]) & 0x7FFFFFFFu);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) am[r] = max(am[r], dpp_i<kDppXor1>(am[r]));
#pragma unroll
          for (int r = 0; r < 16; ++r) am[r] = max(am[r], dpp_i<kDppXor2>(am[r]));
#pragma unroll
          for (int r = 0; r < 16; ++r) am[r] = max(am[r], dpp_i<kDppHalfMirror>(am[r]));
#pragma unroll
          for (int r = 0; r < 16; ++r) am[r] = max(am[r], dpp_i<kDppMirror>(am[r]));
#pragma unroll
          for (int r = 0; r < 16; ++r) am[r] = max(am[r], __builtin_amdgcn_ds_swizzle(am[r], 0x401F));   // lane ^ 16
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = arow0 + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
            const uint32_t code = mxfp8_scale_code(__int_as_float(am[r]));
            qt[i * kHalf + cl] = static_cast<uint8_t>(f32x2_to_e4m3x2(v[r] * mx_inv_scale(code), 0.f) & 0xFF);
            if (j == 0) st[i * kSBlk + cl / 32] = static_cast<uint8_t>(code);
          }
        }
      }
      __syncthreads();
      uint8_t* hq = static_cast<uint8_t*>(ga.out);
      constexpr int kRowVec = kHalf / 16;
      for (int q = threadIdx.x; q < BM * kRowVec; q += kGemmThreads) {
        const int i = q / kRowVec, c = 16 * (q % kRowVec);
        const int col = nt * kHalf + c;
        if (i >= nvalid || col >= N) continue;
        *reinterpret_cast<uint4*>(hq + static_cast<size_t>(b * BM + i) * N + col) =
            *reinterpret_cast<const uint4*>(qt + i * kHalf + c);
      }
      for (int q = threadIdx.x; q < BM * kSBlk; q += kGemmThreads) {
        const int i = q / kSBlk, cb = q % kSBlk;
        const int col = nt * kHalf + 32 * cb;
        if (i >= nvalid || col >= N) continue;
        ga.out_sc[static_cast<size_t>(b * BM + i) * ga.out_sc_pitch + col / 32] = st[i * kSBlk + cb];
      }
    } else if constexpr (GATEUP && C::kSplitA) {
      // h rounded to bf16 goes through LDS (the ring is free now) so that each
      // thread then splits one 32-column block of a row: tile [BM][kHalf].
      __syncthreads();
      uint16_t* tile = reinterpret_cast<uint16_t*>(ring);
#pragma unroll
      for (int u = 0; u < NT / 2; ++u) {
        const int cl = Rt[u] + j;   // column within the workgroup's half tile
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = arow0 + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
            tile[i * kHalf + cl] = f32_to_bf16(swiglu(acc[m][u][r], acc[m][u + NT / 2][r]));
          }
        }
      }
      __syncthreads();
      constexpr int kBlocks = kHalf / 32;   // 32-column blocks per tile row
      uint8_t* hsp = static_cast<uint8_t*>(ga.out);
      for (int q = threadIdx.x; q < BM * kBlocks; q += kGemmThreads) {
        const int i = q / kBlocks, cb = q % kBlocks;
        const int col = nt * kHalf + 32 * cb;   // first intermediate index of the block
        if (i >= nvalid || col >= N) continue;
        const uint4* src = reinterpret_cast<const uint4*>(tile + i * kHalf + 32 * cb);
        const uint4 v[4] = {src[0], src[1], src[2], src[3]};
        const size_t row = static_cast<size_t>(b * BM + i);
        // a row of split h: per 64 columns, 64 hi codes then 64 lo codes
        uint8_t* hi = hsp + row * (2 * static_cast<size_t>(N)) + (col / 64) * 128 + (col % 64);
        mx_split_block(v, hi, hi + 64, ga.out_sc + row * ga.out_sc_pitch + col / 32);
      }
    } else if constexpr (GATEUP) {
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < NT / 2; ++u) {
        const int col = tile_col(nt, Rt[u] + j);   // gate column of this lane
        // multipliers of its gate row and of the matching up row
        const float fg = WFMT == kBF16 ? 1.0f : wact ? row_scale(w, e, col) * fa : 0.f;
        const float fu = WFMT == kBF16 ? 1.0f : wact ? row_scale(w, e, N + col) * fa : 0.f;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = arow0 + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
            if (!wact || i >= nvalid) continue;
            const float v = swiglu(acc[m][u][r] * fg, acc[m][u + NT / 2][r] * fu);
            mx = __builtin_fmaxf(mx, __builtin_fabsf(v));
            static_cast<uint16_t*>(ga.out)[static_cast<size_t>(b * BM + i) * N + col] = f32_to_bf16(v);
          }
        }
      }
      if constexpr (FP8ACT) wave_amax_to_slots(mx, ga.amax_slots);
    } else {
      const int c0 = nt * C::kBN + Rt[0] + j;
      float fc[NT];   // multiplier of each of this lane's output columns
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) fc[ct] = 1.0f;
      if constexpr (WFMT == kNVFP4 || WFMT == kFP8) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) fc[ct] = wact ? row_scale(w, e, c0 + 32 * ct) * fa : 0.f;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);   // row within the wave's 64
          const size_t fr_row = static_cast<size_t>(__shfl(cflat, il, kWave));
          if (!wact || arow0 + il >= nvalid) continue;
#pragma unroll
          for (int ct = 0; ct < NT; ++ct)
            static_cast<uint16_t*>(ga.out)[fr_row * N + c0 + 32 * ct] = f32_to_bf16(acc[m][ct][r] * fc[ct]);
        }
      }
    }

    if (!PERSIST || !have_next) break;
    have_next = false;
    int flat = 0;
    if constexpr (!GATEUP) flat = sid ? meta_row(dk, arow0 + lane) : qb * BM + arow0 + lane;
    enter(qb, qnt, qe, qnv, flat);
  }
  wait_vm<0>();   // no DMA into LDS may outlive the workgroup
}

// ------------------------------------------------------------ launches ----
template <int WFMT, bool FP8ACT, int BM, bool GATEUP, bool WIDE = false>
static hipError_t run(const GemmArgs& ga, hipStream_t s) {
  using C = Cfg<WFMT, FP8ACT, BM, WIDE>;
  const int ntile = GATEUP ? (ga.N + C::kBN / 2 - 1) / (C::kBN / 2) : (ga.N + C::kBN - 1) / C::kBN;
  const int total = ga.rows.num_blocks * ntile;
  if (total == 0) return hipSuccess;
  if (ga.K % (2 * kStageK)) return hipErrorInvalidValue;
  // whole chunks for every XCD, so that every tile index is reached
  const int per_round = 8 * kXcdChunk;
  int grid = per_round * ((total + per_round - 1) / per_round);
  // One workgroup fits a CU (LDS), so a grid of about one workgroup per CU
  // runs every tile with the next tile's first stages fetched during the
  // current one's last; that needs at least as many stages per tile as are
  // fetched ahead (else one workgroup per tile).
  // (The down GEMMs run this way; the gate_up GEMMs, whose epilogue is
  // longer and whose registers are all in use, run one tile per workgroup.)
  constexpr int kAhead = C::kAScales && FP8ACT ? C::kRing : C::kRing - 1;
  if constexpr (!GATEUP) {
    // (not with an expert-slot table: tiles of experts outside the call are skipped one tile per workgroup)
    if (ga.K / kStageK >= kAhead && !ga.w.slot_of) {
      int dev = 0, ncu = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
        return hipErrorInvalidValue;
      grid = std::min(grid, per_round * ((ncu + per_round - 1) / per_round));
      return launch(gemm_kernel<WFMT, FP8ACT, BM, GATEUP, true>, dim3(grid), dim3(kGemmThreads), 0, s, ga);
    }
  }
  return launch(gemm_kernel<WFMT, FP8ACT, BM, GATEUP, false, WIDE>, dim3(grid), dim3(kGemmThreads), 0, s, ga);
}

// Compute units of the current device (0 if the query fails).
static int device_cus() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return ncu;
}

template <bool GATEUP>
static hipError_t dispatch(const GemmArgs& ga, bool fp8act, hipStream_t s) {
  const int bm = ga.rows.block_m;
  switch (ga.w.fmt) {
    case kMXFP4:   // fp8act: MXFP8 activations
      if (!ga.a_sc || (GATEUP && !ga.out_sc)) return hipErrorInvalidValue;
      if (fp8act) return bm == 128 ? run<kMXFP4, true, 128, GATEUP>(ga, s) : hipErrorInvalidValue;
      return bm == 128 ? run<kMXFP4, false, 128, GATEUP>(ga, s) : run<kMXFP4, false, 64, GATEUP>(ga, s);
    case kNVFP4:
      if (fp8act) return hipErrorInvalidValue;
      if (bm == 128) return run<kNVFP4, false, 128, GATEUP>(ga, s);
      if constexpr (GATEUP) {
        // wide tiles once they still give every CU two (the shared expert's
        // dense rows alone would leave half the chip idle)
        const long long wide_tiles = static_cast<long long>(ga.rows.num_blocks) *
                                     ((ga.N + Cfg<kNVFP4, false, 64, true>::kBN / 2 - 1) / (Cfg<kNVFP4, false, 64, true>::kBN / 2));
        const int ncu = device_cus();
        if (ncu > 0 && wide_tiles >= 2LL * ncu) return run<kNVFP4, false, 64, true, true>(ga, s);
      }
      return run<kNVFP4, false, 64, GATEUP>(ga, s);
    case kFP8:
      if (bm != 128) return hipErrorInvalidValue;
      return fp8act ? run<kFP8, true, 128, GATEUP>(ga, s) : run<kFP8, false, 128, GATEUP>(ga, s);
    case kBF16:
      if (bm != 128 || fp8act || ga.w.packed) return hipErrorInvalidValue;
      return run<kBF16, false, 128, GATEUP>(ga, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_gateup(const QW& w, const Rows& rows, const GemmAct& x, int H, int inter, void* h,
                              uint8_t* h_sc, uint32_t* amax_h, hipStream_t s) {
  GemmArgs ga{};
  ga.w = w;
  ga.rows = rows;
  ga.K = H;
  ga.N = inter;
  if (w.fmt == kMXFP4) {
    ga.a = x.split;
    ga.a_sc = x.split_sc;
    ga.a_sc_pitch = H / 32;
    ga.a_row_bytes = x.mx8 ? H : 2 * H;
    ga.out_sc = h_sc;
    ga.out_sc_pitch = inter / 32;
  } else if (x.q) {
    ga.a = x.q;
    ga.a_row_bytes = H;
  } else {
    ga.a = reinterpret_cast<const uint8_t*>(x.bf16);
    ga.a_row_bytes = 2 * H;
  }
  ga.amax_a = x.amax;
  ga.out = h;
  ga.amax_slots = amax_h;
  return dispatch<true>(ga, w.fmt == kMXFP4 ? x.mx8 : x.q != nullptr, s);
}

hipError_t launch_gemm_down(const QW& w, const Rows& rows, const GemmAct& h, int H, int inter, uint16_t* o,
                            hipStream_t s) {
  GemmArgs ga{};
  ga.w = w;
  ga.rows = rows;
  ga.K = inter;
  ga.N = H;
  if (w.fmt == kMXFP4) {
    ga.a = h.split;
    ga.a_sc = h.split_sc;
    ga.a_sc_pitch = inter / 32;
    ga.a_row_bytes = h.mx8 ? inter : 2 * inter;
  } else if (h.q) {
    ga.a = h.q;
    ga.a_row_bytes = inter;
  } else {
    ga.a = reinterpret_cast<const uint8_t*>(h.bf16);
    ga.a_row_bytes = 2 * inter;
  }
  ga.amax_a = h.amax;
  ga.out = o;
  return dispatch<false>(ga, w.fmt == kMXFP4 ? h.mx8 : h.q != nullptr, s);
}

// ---------------------------------------------------- packed weights -----
// The weight operand of a workgroup is a tile of kTileRows matrix rows (the
// same for every configuration: 512), gate_up tiles pairing gate rows
// [256 nt, 256 nt + 256) with the matching up rows.  The packed layout holds,
// for each expert, tile and 64-wide K stage, the stage's codes in the order
// the kernel keeps them in LDS (16-byte vector v = R * V + p of tile row R is
// row R's vector swz(R, p)), then for FP4 one scale dword per tile row (MXFP4:
// the dword of the stage pair; NVFP4: the stage's).  Rows past N are zero.
constexpr int kTileRows = 512;
static_assert(Cfg<kMXFP4, false, 128>::kTileW == kTileRows && Cfg<kMXFP4, false, 64>::kTileW == kTileRows &&
                  Cfg<kMXFP4, true, 128>::kTileW == kTileRows && Cfg<kNVFP4, false, 128>::kTileW == kTileRows &&
                  Cfg<kNVFP4, false, 64>::kTileW == kTileRows && Cfg<kFP8, true, 128>::kTileW == kTileRows,
              "one packed layout serves every tile configuration");

int packed_tiles(int n, bool gate_up) {
  return gate_up ? (n / 2 + kTileRows / 2 - 1) / (kTileRows / 2) : (n + kTileRows - 1) / kTileRows;
}

size_t packed_bytes(int fmt, int E, int n, int k, bool gate_up) {
  return static_cast<size_t>(E) * packed_tiles(n, gate_up) * (k / kStageK) * packed_stage_bytes(fmt);
}

template <int WFMT>
__global__ __launch_bounds__(256) void pack_weights_kernel(QW w, int E, int ntile, int gate_up, uint8_t* out) {
  constexpr int kRowB = WFMT == kFP8 ? 64 : 32;   // bytes of a row per stage
  constexpr int kV = kRowB / 16;
  const int N = w.n, K = w.k, ns = K / kStageK;
  const int st = blockIdx.x;   // (expert, tile, stage)
  const int s = st % ns, nt = (st / ns) % ntile, e = st / (ns * ntile);
  const int half = kTileRows / 2, I = N / 2;
  const uint32_t row_bytes = WFMT == kFP8 ? K : K / 2;
  uint8_t* dst = out + static_cast<size_t>(st) * packed_stage_bytes(WFMT);
  auto row_of = [&](int R) -> int {   // matrix row of tile row R, or -1
    if (gate_up) {
      const int c = nt * half + (R < half ? R : R - half);
      return c < I ? (R < half ? c : I + c) : -1;
    }
    const int c = nt * kTileRows + R;
    return c < N ? c : -1;
  };
  for (int v = threadIdx.x; v < kTileRows * kV; v += blockDim.x) {
    const int R = v / kV, p = v % kV;
    const int row = row_of(R);
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row >= 0)
      val = *reinterpret_cast<const uint4*>(w.codes + (static_cast<size_t>(e) * N + row) * row_bytes +
                                            static_cast<size_t>(s) * kRowB + 16 * swz<kV>(R, p));
    reinterpret_cast<uint4*>(dst)[v] = val;
  }
  if constexpr (WFMT != kFP8) {
    uint32_t* sd = reinterpret_cast<uint32_t*>(dst + kTileRows * kRowB);
    for (int R = threadIdx.x; R < kTileRows; R += blockDim.x) {
      const int row = row_of(R);
      uint32_t val = 0u;
      if (row >= 0) {
        const size_t base = static_cast<size_t>(e) * N + row;
        val = WFMT == kMXFP4 ? *reinterpret_cast<const uint32_t*>(w.scales + base * (K / 32) + 4 * (s / 2))
                             : *reinterpret_cast<const uint32_t*>(w.scales + base * (K / 16) + 4 * s);
      }
      sd[R] = val;
    }
  }
}

hipError_t launch_pack_weights(const QW& w, int E, bool gate_up, uint8_t* out, hipStream_t s) {
  if (w.k % kStageK || (gate_up && w.n % 2)) return hipErrorInvalidValue;
  const int ntile = packed_tiles(w.n, gate_up);
  const int blocks = E * ntile * (w.k / kStageK);
  if (blocks == 0) return hipSuccess;
  switch (w.fmt) {
    case kMXFP4: return launch(pack_weights_kernel<kMXFP4>, dim3(blocks), dim3(256), 0, s, w, E, ntile, gate_up ? 1 : 0, out);
    case kNVFP4: return launch(pack_weights_kernel<kNVFP4>, dim3(blocks), dim3(256), 0, s, w, E, ntile, gate_up ? 1 : 0, out);
    case kFP8: return launch(pack_weights_kernel<kFP8>, dim3(blocks), dim3(256), 0, s, w, E, ntile, gate_up ? 1 : 0, out);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------- split activations ------
// Split E4M3 form of x for the MXFP4 GEMMs, or with a8 the MXFP8 form (one
// thread per 32-block).
__global__ __launch_bounds__(256) void x_split_gemm_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                           uint8_t* __restrict__ xs, uint8_t* __restrict__ xsc,
                                                           int a8) {
  const int nb = H / 32;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * nb) return;
  const int t = i / nb, blk = i % nb;
  const uint4* p = reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + blk * 32);
  const uint4 v[4] = {p[0], p[1], p[2], p[3]};
  uint8_t* sc = xsc + static_cast<size_t>(t) * nb + blk;
  if (a8) {
    mxfp8_block(v, xs + static_cast<size_t>(t) * H + blk * 32, sc);
  } else {
    uint8_t* hi = xs + static_cast<size_t>(t) * (2 * H) + (blk / 2) * 128 + (blk & 1) * 32;
    mx_split_block(v, hi, hi + 64, sc);
  }
}

hipError_t launch_x_split_gemm(const uint16_t* x, int T, int H, uint8_t* xs, uint8_t* xsc, bool a8, hipStream_t s) {
  const int n = T * (H / 32);
  if (n == 0) return hipSuccess;
  return launch(x_split_gemm_kernel, dim3((n + 255) / 256), dim3(256), 0, s, x, T, H, xs, xsc, a8 ? 1 : 0);
}

}  // namespace ftmoe
