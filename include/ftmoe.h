/*
 * ftmoe.h -- routed Mixture-of-Experts layer forward over block-quantised
 * expert weights (MXFP4, NVFP4, FP8 E4M3) on AMD Instinct MI355X (gfx950).
 *
 * Sources: the FreeToken README.  Its "About" section presents the project
 * as an engine that serves Mixture-of-Experts models on consumer hardware;
 * its "Broad MoE & Ecosystem Support" item lists the MoE model families it
 * runs and the expert weight formats MXFP4, NVFP4, FP8 and BF16.  Neither
 * writes the layer's arithmetic down.  The reading taken here (the routed
 * MoE layer of those model families, with SwiGLU experts) is:
 *
 *   l[t,e]   = x_t . W_r[e] + b[e]                       router GEMM
 *   ids_t    = k largest l[t,:], descending, ties -> lower expert index
 *   w_t      = softmax of the k selected logits          renormalised weights
 * (with a selection-only bias, FTMOE_BIAS_SELECT, l = x_t . W_r[e] and the
 *  k largest l[t,e] + b[e] are selected)
 *   h_tj     = silu(Wg[e] x_t) * (Wu[e] x_t),  e = ids_t[j]     gate_up + SwiGLU
 *   y_t      = sum_j w_tj Wd[e] h_tj   (j ascending)    down + weighted combine
 *   y_t     += sigmoid(x_t . w_sg) * shared_mlp(x_t)    optional shared expert
 *
 * With per-tensor FP8 activations, x and h are each quantised to E4M3 with
 * one scale amax/448 over the whole GEMM input (all T rows of x; all T*k rows
 * of h) before their GEMM.  With MXFP8 activations, every row of x, of h and
 * of the shared expert's h is quantised per block of 32 (OCP Microscaling
 * v1.0 conversion, see ftmoe_afmt) before its GEMM.
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers owned by the caller.  Structs
 *    (ftmoe_layer, ftmoe_qweight) live in HOST memory and are only read
 *    during the call.  The library never allocates, frees or synchronises
 *    device memory; scratch comes from the caller's workspace, sized by
 *    ftmoe_workspace_size().
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous on it, enqueue a fixed sequence of kernels whose
 *    grid sizes depend only on the arguments (never on device data), and
 *    issue no host synchronisation, so they can be captured in a HIP graph.
 *  - Arguments are validated on the host before anything is enqueued.  On
 *    error nothing is enqueued and no output is written; the status says why
 *    (ftmoe_last_error() gives a message).  A failed kernel launch returns
 *    FTMOE_ERR_HIP.  No C++ exception crosses this interface.
 *  - No mutable global state is touched by the compute entry points, so
 *    concurrent calls on different streams with different workspaces are
 *    safe.  Two calls sharing one workspace must be ordered by the caller.
 *  - Layouts are row-major with the last index contiguous.  bf16 tensors are
 *    passed as uint16_t bit patterns.
 */
#ifndef FTMOE_H
#define FTMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FTMOE_OK = 0,
  FTMOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, ... */
  FTMOE_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle */
  FTMOE_ERR_WORKSPACE = 3,    /* workspace missing or too small            */
  FTMOE_ERR_HIP = 4           /* HIP runtime reported an error             */
} ftmoe_status;

/* Expert weight formats (FreeToken README, "Broad MoE & Ecosystem Support":
 * MXFP4, NVFP4, FP8 and BF16).
 *  MXFP4: OCP Microscaling v1.0.  E2M1 codes, two per byte (element 2i in the
 *         low nibble), one E8M0 scale byte (2^(s-127)) per 32 elements along K.
 *  NVFP4: E2M1 codes as above, one E4M3FN scale byte per 16 elements along K,
 *         and one fp32 multiplier per matrix: w = e2m1 * e4m3(s_blk) * g.
 *  FP8:   one E4M3FN (OCP: bias 7, max 448, no inf) byte per element and one
 *         fp32 multiplier per matrix: w = e4m3 * g.
 *  BF16:  one bf16 per element (codes hold [E][N][K] 16-bit patterns), no
 *         scales; bf16 activations only; no packed prefill layout.        */
typedef enum {
  FTMOE_W_MXFP4 = 1,
  FTMOE_W_NVFP4 = 2,
  FTMOE_W_FP8_E4M3 = 3,
  FTMOE_W_BF16 = 4
} ftmoe_wfmt;

/* Activation format fed to the expert GEMMs.  FP8_PER_TENSOR is the W8A8
 * scheme of the FreeToken commit message on per-tensor FP8 projections: one
 * dynamic E4M3 scale per GEMM input.  It requires FP8 weights.
 * MXFP8 is a W4A8 scheme for MXFP4 weights (the FreeToken README lists MXFP4
 * among the formats; the MX specification defines the 8-bit element type):
 * each block of 32 consecutive activations along K becomes E4M3 codes under
 * one E8M0 scale 2^X, X = floor(log2 max|v|) - 8 (at least -127), codes the
 * nearest E4M3 of v / 2^X saturating at 448.  Both operands then feed the
 * scaled MFMA with their own block scales.  It requires MXFP4 weights.    */
typedef enum {
  FTMOE_ACT_BF16 = 0,
  FTMOE_ACT_FP8_PER_TENSOR = 1,
  FTMOE_ACT_MXFP8 = 2
} ftmoe_afmt;

/* Role of the router bias.  LOGITS adds it to the logits, so it shapes both
 * the selection and the weights.  SELECT adds it for the ranking only and
 * weights the selected experts by the softmax of their logits without it
 * (a load-balancing bias that must not change the mixture).              */
typedef enum {
  FTMOE_BIAS_LOGITS = 0,
  FTMOE_BIAS_SELECT = 1
} ftmoe_bias_mode;

/* Expert-kernel family.  AUTO picks the bandwidth-bound decode kernels for
 * small token counts and the MFMA grouped GEMMs otherwise; the other values
 * force one for A/B comparisons (both compute the same function).        */
typedef enum {
  FTMOE_PATH_AUTO = 0,
  FTMOE_PATH_DECODE = 1,
  FTMOE_PATH_PREFILL = 2
} ftmoe_path;

/* One stacked set of expert matrices, [E][N][K], K contiguous.
 *  codes:         FP4: [E][N][K/2] bytes.  FP8: [E][N][K] bytes.  BF16: [E][N][K] bf16.
 *  block_scales:  MXFP4: [E][N][K/32] E8M0.  NVFP4: [E][N][K/16] E4M3.  FP8, BF16: NULL.
 *  tensor_scales: NVFP4, FP8: fp32 dequantisation multipliers, [E] (one per
 *                 matrix) or, with row_scales = 1, [E][N] (one per matrix
 *                 row: row-wise scaling).  MXFP4, BF16: NULL.
 * A fused projection whose parts were quantised with separate per-tensor
 * scales (the FreeToken commit message on FP8 projections: gate and up of a
 * gate_up matrix, each with its own scale) is passed with row_scales = 1 and
 * each part's scale repeated over its rows.
 * codes and block_scales must be 16-byte aligned, tensor_scales 4-byte.   */
typedef struct {
  int32_t fmt;          /* ftmoe_wfmt */
  int32_t num_experts;
  int32_t n;
  int32_t k;
  const void* codes;
  const void* block_scales;
  const float* tensor_scales;
  const void* packed;   /* optional (NULL = none): the same matrices in the
                           prefill tile layout written by ftmoe_pack_qweight,
                           256-byte aligned; read by the prefill GEMMs only */
  int32_t row_scales;   /* 0: tensor_scales [E]; 1: [E][N] (NVFP4, FP8)   */
  int32_t reserved;     /* must be 0                                       */
} ftmoe_qweight;

/* One MoE layer.
 *  router_w     [E][H] fp32.   router_bias [E] fp32 or NULL, used as
 *               router_bias_mode says (ftmoe_bias_mode).
 *  gate_up      N = 2*inter, K = hidden: rows [0, inter) are the gate
 *               projection, rows [inter, 2*inter) the up projection.
 *  down         N = hidden, K = inter.
 *  shared_inter 0 for no shared expert; otherwise shared_gate_up (E = 1,
 *               N = 2*shared_inter, K = hidden), shared_down (E = 1,
 *               N = hidden, K = shared_inter) in the routed experts' format,
 *               and shared_gate_w [H] fp32: the shared expert's output is
 *               scaled by sigmoid(x . shared_gate_w) and added after the
 *               routed combine.
 * Limits: hidden, inter and shared_inter multiples of 128 and at most 4096;
 * 1 <= top_k <= 16; top_k <= num_experts <= 1024.                          */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t num_experts;
  int32_t top_k;
  int32_t act;          /* ftmoe_afmt */
  int32_t path;         /* ftmoe_path */
  const float* router_w;
  const float* router_bias;
  ftmoe_qweight gate_up;
  ftmoe_qweight down;
  int32_t shared_inter;
  int32_t router_bias_mode;   /* ftmoe_bias_mode */
  ftmoe_qweight shared_gate_up;
  ftmoe_qweight shared_down;
  const float* shared_gate_w;
} ftmoe_layer;

/* Role of a matrix set in a layer: the prefill tile layout pairs the gate
 * and up rows of gate_up.                                                 */
typedef enum { FTMOE_ROLE_GATE_UP = 0, FTMOE_ROLE_DOWN = 1 } ftmoe_role;

/* Prefill tile layout of one matrix set (a load-time step, for callers that
 * run prefill).  The prefill GEMMs read the weight operand in stages of 64
 * K for a tile of 512 matrix rows (gate_up: 256 gate rows and the 256
 * matching up rows); in the packed layout every such stage is one
 * contiguous run -- the codes in the order the kernel keeps them in LDS,
 * then for FP4 one block-scale dword per row -- so it streams as whole cache
 * lines instead of 32-byte pieces of 512 rows.  The row-major matrices stay
 * in use (decode reads them), so a packed copy doubles the weights'
 * footprint.  The layout is private to this library version.
 *  ftmoe_packed_size: bytes of the packed copy of `w` in `role`.
 *  ftmoe_pack_qweight: enqueues the repack on `stream`; `packed` is device
 *  memory of ftmoe_packed_size bytes, 256-byte aligned; `w` is validated as
 *  in a layer (fmt, shape, pointers; w->packed is ignored).               */
ftmoe_status ftmoe_packed_size(const ftmoe_qweight* w, int32_t role, size_t* bytes);
ftmoe_status ftmoe_pack_qweight(const ftmoe_qweight* w, int32_t role, void* packed, size_t packed_bytes,
                                void* stream);

/* Bytes of workspace that ftmoe_forward / ftmoe_experts_forward /
 * ftmoe_route need for T tokens of this layer (T >= 0).  The workspace must
 * be 256-byte aligned; its contents need no initialisation and are
 * meaningless after a call.
 *  ftmoe_workspace_bytes returns the size directly, or 0 when the layer or
 *  T is invalid (ftmoe_last_error() says why; a valid query is never 0).
 *  ftmoe_workspace_size is the same query with a status.                  */
size_t ftmoe_workspace_bytes(const ftmoe_layer* layer, int32_t T);
ftmoe_status ftmoe_workspace_size(const ftmoe_layer* layer, int32_t T, size_t* bytes);

/* Capacity of the padded expert-sorted row list written by ftmoe_align:
 * roundup(T*k + min(E, T*k)*(block_m - 1), block_m).  Returns -1 on bad
 * arguments.                                                              */
int32_t ftmoe_align_max_padded(int32_t T, int32_t k, int32_t E, int32_t block_m);

/* Scratch bytes ftmoe_align needs (device, 256-byte aligned).             */
size_t ftmoe_align_workspace_size(int32_t T, int32_t k, int32_t E, int32_t block_m);

/* Router: logits, softmax top-k with renormalised weights, and the shared
 * expert's sigmoid gate (the first two lines of the layer arithmetic at the
 * top of this file).  Source: FreeToken README, "Broad MoE & Ecosystem
 * Support" (the MoE model families it serves); the pages give no formula.
 * Reading: the routing of those families -- every token goes to the k
 * experts of largest router logit, weighted by a softmax over those k
 * logits, and a shared expert is gated by the sigmoid of the token's
 * projection on a gate vector; logits accumulate in fp32 from the exact
 * widening of bf16 x against fp32 W_r (never rounded to a narrower type),
 * and ties go to the lower expert index.
 *  x           [T][H] bf16.
 *  topk_ids    [T][k] int32 out: experts by descending logit.
 *  topk_w      [T][k] fp32 out: softmax over the k selected logits.
 *  shared_gate [T] fp32 out, or NULL; required when the layer has a shared
 *              expert.
 *  ws          scratch of ftmoe_workspace_size(layer, T) bytes.          */
ftmoe_status ftmoe_route(const ftmoe_layer* layer, const uint16_t* x, int32_t T,
                         void* ws, size_t ws_bytes,
                         int32_t* topk_ids, float* topk_w, float* shared_gate,
                         void* stream);

/* Token-to-expert alignment (count, prefix-sum, padded scatter): the
 * grouping that lets each expert's routed rows run as one GEMM over whole
 * blocks.  Source: FreeToken README, "About" (MoE serving); the pages do
 * not describe the grouping.  Reading: a stable counting sort of the flat
 * rows by expert, each expert's segment padded to a multiple of block_m,
 * so that the result is unique.
 * Flat row i = t*k + j goes to expert topk_ids[i] (each in [0, E)).
 *  counts       [E]     rows per expert.
 *  offsets      [E+1]   exclusive prefix sum of counts rounded up to block_m.
 *  sorted_ids   [P]     P = ftmoe_align_max_padded(T, k, E, block_m): each
 *               expert's rows in ascending i at [offsets[e], offsets[e+1]),
 *               padded with the sentinel T*k; entries >= num_padded are T*k.
 *  block_expert [P/block_m] expert of each block of block_m rows, -1 past
 *               num_padded.
 *  num_padded   [1]     offsets[E].
 *  ws           ftmoe_align_workspace_size() bytes of scratch.
 * The result is unique (stable order), hence bit-reproducible.           */
ftmoe_status ftmoe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_ids,
                         int32_t* block_expert, int32_t* num_padded,
                         void* ws, size_t ws_bytes, void* stream);

/* Experts given a routing: align, gate_up GEMM with fused SwiGLU, down GEMM,
 * weighted combine and the optional gated shared expert (lines 3-6 of the
 * layer arithmetic at the top of this file).  Source: FreeToken README,
 * "Broad MoE & Ecosystem Support" (MoE families whose experts are stored
 * as MXFP4, NVFP4, FP8 or BF16 weights) and the FreeToken commit page of
 * commit 58f4b9e (its message on FP8 projections with per-tensor
 * activation scales, for FTMOE_ACT_FP8_PER_TENSOR); the pages give no
 * formula.  Reading: SwiGLU experts with the gate rows first in gate_up,
 * h = silu(gate) * up, the k expert outputs summed in ascending slot order,
 * the gated shared expert added last, y rounded once to bf16; h may be
 * rounded to bf16 between the GEMMs.
 *  topk_ids, topk_w  as written by ftmoe_route.
 *  shared_gate       [T] fp32 sigmoid gate, required iff shared_inter > 0.
 *  y                 [T][H] bf16 out (round to nearest even).             */
ftmoe_status ftmoe_experts_forward(const ftmoe_layer* layer, const uint16_t* x, int32_t T,
                                   const int32_t* topk_ids, const float* topk_w,
                                   const float* shared_gate,
                                   void* ws, size_t ws_bytes, uint16_t* y, void* stream);

/* The whole layer: ftmoe_route then ftmoe_experts_forward (the full layer
 * arithmetic at the top of this file; sources and readings as for those
 * two entry points).
 *  topk_ids_out / topk_w_out: optional [T][k] copies of the routing (NULL
 *  to keep it in the workspace only).                                    */
ftmoe_status ftmoe_forward(const ftmoe_layer* layer, const uint16_t* x, int32_t T,
                           void* ws, size_t ws_bytes, uint16_t* y,
                           int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* The whole layer as ftmoe_forward, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): no workspace argument, and no allocation of any kind.
 * Its scratch is a fixed device array inside the library, 32 MiB, which
 * every GPU the library runs on holds until the process ends (its address
 * is looked up, not allocated, on the first call on each device).  Layers
 * and token counts whose ftmoe_workspace_size exceeds 32 MiB return
 * FTMOE_ERR_WORKSPACE (nothing enqueued): decode batches of up to 8 tokens
 * fit at the largest shapes the library takes (hidden and intermediate
 * 4096, 1024 experts, top-16: under 19 MiB), 16 tokens only at smaller
 * ones (about 37 MiB there).  Every call on one GPU shares that scratch: calls on
 * one GPU must not overlap (order them on one stream or synchronise), or
 * they race.  Results equal ftmoe_forward's bit for bit.  Per-kernel timing
 * is not recorded for these calls.                                        */
ftmoe_status ftmoe_forward_noalloc(const ftmoe_layer* layer, const uint16_t* x, int32_t T, uint16_t* y,
                                   int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* ---- Expert residency: an HBM slot pool over experts kept in host memory ----
 * The FreeToken README ("About", its runtime features) lists an LRU cache of
 * experts held in GPU memory, and the atomicmilkshake fork README ("Verified
 * on my hardware") runs with the routed experts in host memory.  Here the
 * routed experts of one layer live in host memory (caller-owned, preferably
 * pinned, so that the copies are asynchronous); a device pool of `slots`
 * expert slots (gate_up and down of one expert each, in the layer's format)
 * holds the ones last used.  The router, the shared expert and everything
 * else stay in device memory as in a plain layer.  The cache object is host
 * memory the library allocates (ftmoe_cache_destroy frees it); the pool is
 * device memory the caller provides.  A cache is used by one thread at a
 * time.                                                                   */
typedef struct ftmoe_cache ftmoe_cache;

/* Device bytes of a pool of `slots` expert slots for `layer` (slots >= 1;
 * 256-byte aligned regions).                                             */
ftmoe_status ftmoe_cache_pool_size(const ftmoe_layer* layer, int32_t slots, size_t* bytes);

/* Creates the residency state for `layer` (its gate_up and down are not
 * used), whose routed experts are `host_gate_up` and `host_down` (HOST
 * pointers, same layout and format as in a layer, no packed layout).
 * `pool`: device memory of ftmoe_cache_pool_size bytes, 256-byte aligned.
 * All slots start empty.  The descriptors are copied.  Host only: the copy
 * stream and events are made on the first ftmoe_cache_forward, which also
 * asks HIP for device addresses of the host arrays: if every one is pinned
 * and mapped (hipHostMalloc), one kernel per pass reads the missing experts
 * straight from them (each array must then lie in one allocation),
 * otherwise each array of each missing expert is one DMA copy.           */
ftmoe_status ftmoe_cache_create(const ftmoe_layer* layer, const ftmoe_qweight* host_gate_up,
                                const ftmoe_qweight* host_down, int32_t slots, void* pool, size_t pool_bytes,
                                ftmoe_cache** cache);
void ftmoe_cache_destroy(ftmoe_cache* cache);

/* The residency policy (host only, no device work): for the n distinct
 * experts one step needs (each in [0, E), distinct), gives each a slot:
 * an expert that holds a slot keeps it; another takes the least recently
 * used slot that this step does not need, evicting its expert.  Every
 * expert of the step then counts as used now.  out_miss = 0 (a hit) when
 * the expert's bytes are in its slot, 1 (a miss) when they must be copied
 * there.  This call copies nothing: the slots it gives stay unfilled, and
 * the next ftmoe_cache_forward that routes to such an expert copies it
 * (a miss then too); evicted experts are gone from the pool at once.
 * FTMOE_ERR_UNSUPPORTED if n > slots (nothing changes).                  */
ftmoe_status ftmoe_cache_plan(ftmoe_cache* cache, const int32_t* experts, int32_t n, int32_t* out_slot,
                              int32_t* out_miss);

/* Workspace bytes of ftmoe_cache_forward for T tokens.                    */
ftmoe_status ftmoe_cache_workspace_size(const ftmoe_cache* cache, int32_t T, size_t* bytes);

/* The layer forward with the routed experts served from the pool.  Routes
 * on `stream`, copies the routing to the host and waits for it (this entry
 * point synchronises `stream` once, and the previous call's stream if it
 * was another), then runs the step's distinct experts in passes, each
 * planned as above: first the resident ones (hits), then the missing ones,
 * in one pass when they fit beside the hits, else in groups of half the
 * pool.  A pass's copies (host -> pool) run on a copy stream the cache owns
 * and overlap the previous pass's kernels, except where they evict a slot
 * that an unfinished pass reads (then they wait for it); each pass's
 * gate_up and down wait for their copies; the combine follows the last
 * pass.  Layers with per-tensor FP8 activations run in one pass (their h
 * scale spans every expert): FTMOE_ERR_UNSUPPORTED if the step needs more
 * experts than there are slots.  Arguments as in ftmoe_forward; the
 * outputs equal ftmoe_forward's on a layer whose experts are in device
 * memory.  Call with the device current that was current at creation.
 * After FTMOE_ERR_HIP the pool forgets what it held (every slot empty).   */
ftmoe_status ftmoe_cache_forward(ftmoe_cache* cache, const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                                 uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* Counters since creation: slot hits and misses (experts copied), bytes
 * copied host -> pool, and passes run.  Any output may be NULL.          */
ftmoe_status ftmoe_cache_stats(const ftmoe_cache* cache, int64_t* hits, int64_t* misses, int64_t* bytes_copied,
                               int64_t* passes);

/* ---- CPU-GPU co-execution over the expert-slot pool ----
 * The FreeToken README ("About", its runtime features) lists bandwidth-
 * adaptive co-execution that splits MoE work between the host CPU and the
 * GPU, without giving the policy.  With it enabled, ftmoe_cache_forward
 * splits each step's missing experts (the hits always run on the GPU):
 * taking them fewest routed rows first, the host computes the first q and
 * the pool fills the rest, where q minimises the larger of the host's time
 * (sum over its experts of expert_s + rows * row_s) and the link's (their
 * bytes / link_bytes_per_s), the smaller q on ties.  The host computes
 * from the host arrays while the GPU runs the passes.  It uses `threads`
 * threads of its own and the calling thread, in fp32 with h rounded as the
 * device path rounds it.  Its rows then go into the device's expert output
 * buffer before the combine.  Host-computed experts count as neither hits
 * nor misses and do not enter the pool.
 * threads = 0 disables it.  expert_s <= 0 or row_s < 0 asks for
 * calibration: expert 0 is timed here with 1 and 65 rows.  The model is
 * then adaptive: after each step that computed experts on the host, it is
 * rescaled toward the measured host time (a running average).
 * link_bytes_per_s <= 0 means 50e9.  FTMOE_ERR_UNSUPPORTED for per-tensor
 * FP8 activations (h's scale spans every expert) and on CPUs without AVX2
 * and FMA.                                                               */
ftmoe_status ftmoe_cache_set_host_compute(ftmoe_cache* cache, int32_t threads, double expert_s, double row_s,
                                          double link_bytes_per_s);

/* Counters of host-computed experts and rows, host compute seconds, and
 * the cost model in use (adaptive scaling applied).  Any output may be
 * NULL.                                                                   */
ftmoe_status ftmoe_cache_host_stats(const ftmoe_cache* cache, int64_t* experts, int64_t* rows, double* seconds,
                                    double* expert_s, double* row_s);

/* The host half alone, with HOST pointers throughout.  Row r is token
 * tok[r] of x [*][H] (bf16) through routed expert ex[r] of `layer`, whose
 * gate_up and down are host arrays; the router and shared expert are not
 * used.  o [n][H] fp32 = W_down h.  `threads` >= 1.  Exposed so that the
 * arithmetic can be tested without a GPU; the device path never calls it. */
ftmoe_status ftmoe_host_expert_rows(const ftmoe_layer* layer, const uint16_t* x, const int32_t* tok,
                                    const int32_t* ex, int32_t n, float* o, int32_t threads);

/* Per-tensor E4M3 activation quantiser used by FTMOE_ACT_FP8_PER_TENSOR,
 * exposed for testing: scale[0] = amax(|x|)/448 (1 if amax is 0, fp32) and
 * q = E4M3(x / scale) rounded to nearest even and saturated to +-448.
 *  x [n] bf16 in; q [n] bytes out; scale [1] fp32 out; ws >= 256 bytes.  */
ftmoe_status ftmoe_quantize_fp8_per_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* scale,
                                           void* ws, size_t ws_bytes, void* stream);

/* Diagnostics: per-kernel timing.  While enabled on the calling thread,
 * every step the entry points enqueue is timed by a pair of HIP events: for
 * a step that is a single kernel the events are attached to its launch and
 * recorded at the kernel's own start and end; other steps are bracketed by
 * events on the stream (not for use under graph capture; the events are
 * host objects the library creates and reuses).  ftmoe_timing_collect waits for the recorded
 * events, writes up to max_entries rows -- kernel name (32-byte slots in
 * `names`), summed milliseconds and launch count -- clears the record and
 * returns the number of distinct kernels seen.  Any output may be NULL.    */
void ftmoe_timing_enable(int32_t on);
int32_t ftmoe_timing_collect(int32_t max_entries, char* names, double* total_ms, int64_t* counts);

/* Human-readable name of a status, and the message of the last error seen
 * by this thread (empty if none).                                         */
const char* ftmoe_status_string(ftmoe_status s);
const char* ftmoe_last_error(void);

/* Library version as major*10000 + minor*100 + patch.                     */
int32_t ftmoe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FTMOE_H */
