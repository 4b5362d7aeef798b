// Internal launchers of the ftmoe kernels.  Host code only sees these; every
// launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ftmoe {

// ---- launches ----
// Kernel timing (diagnostics): while a pair of events is parked in this
// thread's slot, the next kernel launched through launch() carries them, and
// the runtime records them at that kernel's own start and end (no extra
// stream operations, so the elapsed time is the kernel's execution alone).
struct KernelEvents {
  hipEvent_t start, stop;
};
KernelEvents& kernel_events();

template <class... P, class... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A... args) {
  KernelEvents& ev = kernel_events();
  if (ev.start) {
    const KernelEvents e = ev;
    ev = KernelEvents{nullptr, nullptr};
    hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), s, e.start, e.stop, 0u,
                          static_cast<P>(args)...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<P>(args)...);
  }
  return hipGetLastError();
}


// Device view of one stacked packed matrix set [E][N][K].
struct QW {
  int fmt = 0;                 // kMXFP4 | kNVFP4 | kFP8 | kBF16
  int n = 0, k = 0;
  const uint8_t* codes = nullptr;   // fp4: [E][N][K/2]; fp8: [E][N][K]; bf16: [E][N][K] x 2 bytes
  const uint8_t* scales = nullptr;  // mxfp4 [E][N][K/32]; nvfp4 [E][N][K/16]; fp8 / bf16 unused
  const float* tscale = nullptr;    // nvfp4 / fp8: [E], or [E][N] with rowsc; mxfp4 unused
  const uint8_t* packed = nullptr;  // optional: the same matrices in the prefill tile layout, or NULL
  int rowsc = 0;                    // tscale holds one multiplier per matrix row
  const int32_t* slot_of = nullptr; // optional [E]: the matrix slot holding expert e, < 0 if none (NULL: slot e)
};

// Slot of expert e's matrices (an expert-slot pool), or < 0 when this call
// does not serve it.
__device__ __forceinline__ int expert_slot(const QW& w, int e) { return w.slot_of ? w.slot_of[e] : e; }

// fp32 multiplier of row `row` of expert e's matrix (NVFP4 / FP8).
__device__ __forceinline__ float row_scale(const QW& w, int e, int row) {
  return w.rowsc ? w.tscale[static_cast<size_t>(e) * w.n + row] : w.tscale[e];
}

// Bytes of one packed stage (512 tile rows x 64 K): codes, then for FP4 one
// block-scale dword per row.
__host__ __device__ constexpr uint32_t packed_stage_bytes(int fmt) {
  return fmt == kFP8 ? 512u * 64u : 512u * 32u + 512u * 4u;
}

// Row source of an expert GEMM: either an expert-sorted block list (routed
// experts) or the identity over T tokens (the shared expert).
struct Rows {
  const int32_t* sorted_ids;   // [P] flat row ids t*k+j, sentinel = n_flat; NULL = identity
  const int32_t* block_expert; // [P/BM]
  const int32_t* counts;       // [E] rows per expert (routed) or NULL
  const int32_t* offsets;      // [E+1] padded segment starts (routed) or NULL
  int32_t n_flat;              // T*k (routed) or T (identity)
  int32_t top_k;               // flat id -> token divisor (1 for identity)
  int32_t num_blocks;          // grid extent in blocks of block_m rows
  int32_t block_m;             // rows per block: 64 or 128
};

// ---- router ----
// logits [S][T][E+1] fp32, S = router_splits_gemm(T, H, rows) K splits (rows = E + shared).
int router_splits_gemm(int T, int H, int rows);
// Many tokens: the router GEMM reads the fp32 router rows (and the shared
// gate vector as row E) split into three bf16 planes [3][rows][H], made by
// launch_router_split into router_planes_bytes of scratch; few tokens read
// router_w directly (planes may then be null).
size_t router_planes_bytes(int E, int H, bool shared);
hipError_t launch_router_split(const float* router_w, int E, int H, const float* shared_gate_w, uint16_t* planes,
                               hipStream_t s);
// With xs (many tokens only) the GEMM also writes x for MXFP4 expert GEMMs:
// split E4M3 pairs, or MXFP8 codes with a8, and E8M0 scales (xssc).
hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* router_w, int E,
                                const float* shared_gate_w, const uint16_t* planes, float* logits, uint8_t* xs,
                                uint8_t* xssc, bool a8, hipStream_t s);
// bias_select: the bias ranks the experts only; the weights are the softmax
// of the selected logits without it.
hipError_t launch_topk(const float* logits, int nsplit, int T, int E, int k, const float* bias, bool bias_select,
                       bool has_shared, int32_t* ids, float* w, float* sgate, hipStream_t s);

// ---- align ----
size_t align_scratch_bytes(int T, int k, int E, int BM);
hipError_t launch_align(const int32_t* ids, int T, int k, int E, int BM, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_ids, int32_t* block_expert,
                        int32_t* num_padded, void* scratch, uint32_t* zero_words, int n_zero,
                        hipStream_t s);

// ---- utilities ----
// Fills n words with 0 (a kernel, so the sequence stays capturable).
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);

// ---- FP8 per-tensor activation quantisation ----
hipError_t launch_amax_bf16(const uint16_t* x, int64_t n, uint32_t* amax_bits, hipStream_t s);
hipError_t launch_quant_fp8(const uint16_t* x, int64_t n, const uint32_t* amax_bits, uint8_t* q,
                            float* scale_out, hipStream_t s);
// Max over the kAmaxSlots partial maxima written by the gate_up kernels.
hipError_t launch_amax_fold(const uint32_t* slots, uint32_t* out, hipStream_t s);

// ---- decode path (T <= kDecodeMaxT; bandwidth-bound) ----
constexpr int kDecodeBM = 16;
constexpr int kDecodeMaxT = 16;
// Router partial logits part[t][row][s], s over S = router_splits(H) slices
// of H (a multiple of 4).  With xhi non-NULL the kernel also writes the split
// E4M3 form of x (xhi / xlo [T][H], xsc [T][xsc_pitch]) for the MXFP4 MFMA,
// or with xlo NULL the MXFP8 form (codes in xhi, scales in xsc).
int router_splits(int H);
hipError_t launch_router_partial(const uint16_t* x, int T, int H, const float* router_w, int E,
                                 const float* shared_gate_w, float* part, uint8_t* xhi, uint8_t* xlo,
                                 uint8_t* xsc, int xsc_pitch, hipStream_t s);
// Split E4M3 form of x without the router (one thread per 32-block); with
// xlo NULL the MXFP8 form.
hipError_t launch_x_split(const uint16_t* x, int T, int H, int xsc_pitch, uint8_t* xhi, uint8_t* xlo,
                          uint8_t* xsc, hipStream_t s);
inline int xsc_pitch_of(int H) { return (H / 32 + 15) / 16 * 16; }
// Sums the partial logits, top-k + softmax (+ sigmoid gate), aligns the T*k
// rows into blocks of kDecodeBM and zeroes `zero_words`.  One workgroup.
hipError_t launch_topk_align_decode(const float* part, int S, int T, int E, int k, const float* bias,
                                    bool bias_select, bool has_shared, int32_t* ids, float* w, float* sg, int32_t* counts,
                                    int32_t* offsets, int32_t* sorted_ids, int32_t* block_expert,
                                    int32_t* num_padded, int P, uint32_t* zero_words, int n_zero,
                                    hipStream_t s);

struct DecodeArgs {
  QW gu, dn;                  // routed experts
  QW sgu, sdn;                // shared expert (used when Is > 0)
  const int32_t* sorted_ids;  // [nb_routed * kDecodeBM]
  const int32_t* block_expert;
  int T, k, H, I, Is;
  int nb_routed, nb_shared;   // grid blocks: routed blocks, then shared blocks
  const uint16_t* x;
  int a8;                     // MXFP4 with MXFP8 activations: single E4M3 codes in xhi / hhi, no lo
  const uint8_t* xhi;         // MXFP4: split activations [T][H] (hi codes, or the MXFP8 codes)
  const uint8_t* xlo;         //        [T][H] (lo codes; NULL with a8)
  const uint8_t* xsc;         //        [T][xsc_pitch] E8M0 scale per 32-block
  int xsc_pitch;
  const uint8_t* xq;          // FP8 activations or NULL
  const uint32_t* amax_x;
  uint16_t* h;                // [nb_routed * 16][I] bf16 (NVFP4 / FP8)
  uint16_t* hs;               // [nb_shared * 16][Is] bf16 (NVFP4 / FP8)
  uint8_t* hhi;               // MXFP4: split h, routed rows [nb_routed * 16][I] then shared [nb_shared * 16][Is]
  uint8_t* hlo;               //        (lo codes, same layout; NULL with a8)
  uint8_t* hsc;               //        [(nb_routed + nb_shared) * 16][hsc_pitch] E8M0 scales
  int hsc_pitch;
  uint32_t* amax_slots;       // FP8 activations: gate_up partial maxima of |h| (or NULL)
  const uint32_t* amax_h;     // FP8 activations: folded max of |h| read by down (or NULL)
  float* o32;                 // [T*k][H] fp32
  float* s32;                 // [T][H] fp32
  const float* w;             // [T*k]
  const float* sg;            // [T] or NULL
  uint16_t* y;                // [T][H] bf16
};
int decode_down_tiles(int H);
hipError_t launch_decode_gateup(const DecodeArgs& a, hipStream_t s);
// Down projection of every block into fp32 rows o32 / s32.
hipError_t launch_decode_down(const DecodeArgs& a, hipStream_t s);
// y = routed rows summed in ascending slot order j, then the gated shared expert.
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t s);
// One-token steps of MXFP4 layers: down and combine in one launch (same
// results as the two); decode_fused_one_token tells whether the step qualifies.
bool decode_fused_one_token(const DecodeArgs& a);
hipError_t launch_decode_down_combine1(const DecodeArgs& a, hipStream_t s);

// ---- prefill experts (grouped GEMMs on MFMA) ----
// Rows per block of the prefill GEMMs for a layer routing T*k rows over E experts.
// MXFP8 activations (a8) always take 128-row blocks.
int gemm_block_m(int T, int k, int E, int wfmt, bool a8);
// Activation operand of a prefill GEMM, by weight format: MXFP4 takes the
// split E4M3 form (per 64 columns of a row: 64 hi codes then 64 lo codes,
// 2 bytes per element; E8M0 scales [rows][K/32]), or with mx8 the MXFP8
// form (one E4M3 code per element, [rows][K], same scales); FP8 weights
// with FP8 activations take q (E4M3, per-tensor scale from amax); otherwise
// bf16.
struct GemmAct {
  const uint16_t* bf16;
  const uint8_t* q;
  const uint32_t* amax;
  const uint8_t* split;
  const uint8_t* split_sc;
  bool mx8;
};
// gate_up writes h [rows][I]: bf16, or for MXFP4 split (h [rows][2I] codes,
// h_sc [rows][I/32] scales) or, with x.mx8, MXFP8 (h [rows][I] codes, same
// scales).  amax_h: FP8 activations only, the kAmaxSlots partial maxima of
// |h|.
hipError_t launch_gemm_gateup(const QW& w, const Rows& rows, const GemmAct& x, int H, int inter, void* h,
                              uint8_t* h_sc, uint32_t* amax_h, hipStream_t s);
hipError_t launch_gemm_down(const QW& w, const Rows& rows, const GemmAct& h, int H, int inter, uint16_t* o,
                            hipStream_t s);
// Packed tile layout of a matrix set for the prefill GEMMs (see gemm.hip).
size_t packed_bytes(int fmt, int E, int n, int k, bool gate_up);
hipError_t launch_pack_weights(const QW& w, int E, bool gate_up, uint8_t* out, hipStream_t s);
// Split E4M3 form of x for the MXFP4 GEMMs: xs [T][2H], xsc [T][H/32]; with
// a8 the MXFP8 form xs [T][H] and the same scales.
hipError_t launch_x_split_gemm(const uint16_t* x, int T, int H, uint8_t* xs, uint8_t* xsc, bool a8, hipStream_t s);

// ---- expert-slot pool fills ----
// Copies the arrays of n experts from host memory the device can read
// (pinned, mapped) into their pool slots: for each array j, expert e[m]'s
// bytes [e*bytes[j], (e+1)*bytes[j]) of src[j] go to dst[j] + s[m]*bytes[j].
// One launch reads the PCIe link at its full rate where one DMA copy per
// array would pay a fixed cost for each.
constexpr int kFillArrays = 6;
constexpr int kFillMax = 64;    // experts per launch
struct FillArgs {
  const uint8_t* src[kFillArrays];
  uint8_t* dst[kFillArrays];
  uint32_t bytes[kFillArrays];  // per expert; 0 = array absent; multiples of 4
  int32_t n;
  int32_t e[kFillMax], s[kFillMax];
};
hipError_t launch_expert_fill(const FillArgs& a, hipStream_t s);

// Expert output rows computed on the host (device-readable host memory:
// rows [n][H] fp32, flat row ids [n]) into the device path's o buffer:
// fp32 o32 [T*k][H] (decode) or, with o32 NULL, bf16 o16 (nearest even).
hipError_t launch_host_rows_scatter(const float* rows, const int32_t* flat, int n, int H, float* o32, uint16_t* o16,
                                    hipStream_t s);

// ---- combine ----
// y[t] = sum_j w[t,j] o[t*k+j] (+ sg[t] * sh[t]) -> bf16.
hipError_t launch_combine(const uint16_t* o, const float* w, int T, int k, int H, const float* sg,
                          const uint16_t* sh, uint16_t* y, hipStream_t s);

}  // namespace ftmoe
