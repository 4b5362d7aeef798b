// Internal launchers of the ftmoe kernels.  Host code only sees these; every
// launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ftmoe {

// Device view of one stacked packed matrix set [E][N][K].
struct QW {
  int fmt;                     // kMXFP4 | kNVFP4 | kFP8
  int n, k;
  const uint8_t* codes;        // fp4: [E][N][K/2]; fp8: [E][N][K]
  const uint8_t* scales;       // mxfp4 [E][N][K/32]; nvfp4 [E][N][K/16]; fp8 unused
  const float* tscale;         // nvfp4 / fp8: [E]; mxfp4 unused
};

// Row source of an expert GEMM: either an expert-sorted block list (routed
// experts) or the identity over T tokens (the shared expert).
struct Rows {
  const int32_t* sorted_ids;   // [P] flat row ids t*k+j, sentinel = n_flat; NULL = identity
  const int32_t* block_expert; // [P/BM]
  int32_t n_flat;              // T*k (routed) or T (identity)
  int32_t top_k;               // flat id -> token divisor (1 for identity)
  int32_t num_blocks;          // grid extent in blocks of BM rows
};

// ---- router ----
hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* router_w, int E,
                                const float* shared_gate_w, float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, const float* bias, bool has_shared,
                       int32_t* ids, float* w, float* sgate, hipStream_t s);

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

// ---- decode experts (small token counts; bandwidth-bound) ----
constexpr int kDecodeBM = 16;
// h[p][0..inter) for every row p of every block (identity rows when
// rows.sorted_ids == NULL).  act_q: fp8 activations (x_q + amax_x) or NULL.
hipError_t launch_decode_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                                const uint32_t* amax_x, int H, int inter, uint16_t* h,
                                uint32_t* amax_h, int max_tokens_per_block, hipStream_t s);
hipError_t launch_decode_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h,
                              int H, int inter, uint16_t* o, hipStream_t s);

// ---- prefill experts (grouped GEMMs on MFMA) ----
constexpr int kPrefillBM = 64;
hipError_t launch_gemm_gateup(const QW& w, const Rows& rows, const uint16_t* x, const uint8_t* xq,
                              const uint32_t* amax_x, int H, int inter, uint16_t* h,
                              uint32_t* amax_h, hipStream_t s);
hipError_t launch_gemm_down(const QW& w, const Rows& rows, const uint16_t* h, const uint32_t* amax_h,
                            int H, int inter, uint16_t* o, hipStream_t s);

// ---- combine ----
// y[t] = sum_j w[t,j] o[t*k+j] (+ sg[t] * sh[t]) -> bf16.
hipError_t launch_combine(const uint16_t* o, const float* w, int T, int k, int H, const float* sg,
                          const uint16_t* sh, uint16_t* y, hipStream_t s);

}  // namespace ftmoe
