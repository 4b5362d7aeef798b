// C ABI of the ftmoe library: argument validation, workspace carving and the
// fixed kernel sequence of each entry point.  See include/ftmoe.h.
#include <stdarg.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <memory>
#include <mutex>
#include <new>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/ftmoe.h"
#include "common.hpp"
#include "host_experts.hpp"
#include "kernels.hpp"

namespace {

using namespace ftmoe;

thread_local std::string g_last_error;

ftmoe_status fail(ftmoe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ftmoe_status fail(ftmoe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ftmoe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FTMOE_OK;
  return fail(FTMOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FT_TRY(expr)                          \
  do {                                        \
    const ftmoe_status st_ = (expr);          \
    if (st_ != FTMOE_OK) return st_;          \
  } while (0)

#define FT_HIP(expr, what)                                 \
  do {                                                     \
    const hipError_t e_ = (expr);                          \
    if (e_ != hipSuccess) return hip_status(e_, what);     \
  } while (0)

// ---- optional per-kernel timing (diagnostics) ----
// When enabled on this thread, a step that is one kernel launched through
// launch() carries a pair of events recorded at the kernel's own start and
// end; any other step is bracketed by two events on its stream.
// ftmoe_timing_collect() waits for them and sums durations per step name.
// Events come from a pool that is reused after each collect.
struct TimedLaunch {
  const char* name;
  hipEvent_t a, b;   // the pair that timed the step
  hipEvent_t c, d;   // the other pair (unused), returned to the pool
};
thread_local bool g_timing = false;
thread_local std::vector<TimedLaunch> g_pending;
thread_local std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ftmoe::KernelEvents& ftmoe::kernel_events() {
  thread_local KernelEvents ev{nullptr, nullptr};
  return ev;
}

namespace {

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_timing) return launch();
  TimedLaunch t{name, pool_event(), pool_event(), pool_event(), pool_event()};
  if (!t.a || !t.b || !t.c || !t.d) return launch();
  kernel_events() = KernelEvents{t.a, t.b};
  (void)hipEventRecord(t.c, s);
  const hipError_t e = launch();
  (void)hipEventRecord(t.d, s);
  if (kernel_events().start) {   // not a single launch() kernel: time the stream span
    kernel_events() = KernelEvents{nullptr, nullptr};
    std::swap(t.a, t.c);
    std::swap(t.b, t.d);
  }
  g_pending.push_back(t);
  return e;
}

constexpr int kMaxTopK = 16;
constexpr int kMaxDim = 4096;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTokens = 1 << 20;
constexpr int kDecodeAutoMaxT = kDecodeMaxT;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ftmoe_status check_qweight(const ftmoe_qweight& q, const char* name, int fmt, int E, int n, int k) {
  if (q.fmt != fmt)
    return fail(FTMOE_ERR_INVALID_ARG, "%s.fmt=%d but the layer's routed experts use %d", name, q.fmt, fmt);
  if (q.num_experts != E || q.n != n || q.k != k)
    return fail(FTMOE_ERR_INVALID_ARG, "%s is [%d][%d][%d], expected [%d][%d][%d]", name, q.num_experts, q.n, q.k,
                E, n, k);
  if (!q.codes) return fail(FTMOE_ERR_INVALID_ARG, "%s.codes is NULL", name);
  if (!aligned16(q.codes)) return fail(FTMOE_ERR_INVALID_ARG, "%s.codes is not 16-byte aligned", name);
  if (fmt == FTMOE_W_MXFP4 || fmt == FTMOE_W_NVFP4) {
    if (!q.block_scales) return fail(FTMOE_ERR_INVALID_ARG, "%s.block_scales is NULL", name);
    if (!aligned16(q.block_scales))
      return fail(FTMOE_ERR_INVALID_ARG, "%s.block_scales is not 16-byte aligned", name);
  }
  if (fmt == FTMOE_W_NVFP4 || fmt == FTMOE_W_FP8_E4M3) {
    if (!q.tensor_scales) return fail(FTMOE_ERR_INVALID_ARG, "%s.tensor_scales is NULL", name);
    if (reinterpret_cast<uintptr_t>(q.tensor_scales) & 3u)
      return fail(FTMOE_ERR_INVALID_ARG, "%s.tensor_scales is not 4-byte aligned", name);
  }
  if (q.row_scales != 0 && q.row_scales != 1)
    return fail(FTMOE_ERR_INVALID_ARG, "%s.row_scales=%d is neither 0 nor 1", name, q.row_scales);
  if (q.row_scales && (fmt == FTMOE_W_MXFP4 || fmt == FTMOE_W_BF16))
    return fail(FTMOE_ERR_INVALID_ARG, "%s.row_scales: the format has no fp32 multipliers", name);
  if (q.packed && fmt == FTMOE_W_BF16)
    return fail(FTMOE_ERR_INVALID_ARG, "%s.packed: BF16 experts have no packed layout", name);
  if (q.reserved != 0) return fail(FTMOE_ERR_INVALID_ARG, "%s.reserved=%d is not 0", name, q.reserved);
  if (q.packed && (reinterpret_cast<uintptr_t>(q.packed) & 255u))
    return fail(FTMOE_ERR_INVALID_ARG, "%s.packed is not 256-byte aligned", name);
  return FTMOE_OK;
}

ftmoe_status check_layer(const ftmoe_layer* L) {
  if (!L) return fail(FTMOE_ERR_INVALID_ARG, "layer is NULL");
  if (L->hidden <= 0 || L->hidden % 128 || L->hidden > kMaxDim)
    return fail(FTMOE_ERR_UNSUPPORTED, "hidden=%d must be a positive multiple of 128, at most %d", L->hidden,
                kMaxDim);
  if (L->inter <= 0 || L->inter % 128 || L->inter > kMaxDim)
    return fail(FTMOE_ERR_UNSUPPORTED, "inter=%d must be a positive multiple of 128, at most %d", L->inter, kMaxDim);
  if (L->top_k < 1 || L->top_k > kMaxTopK)
    return fail(FTMOE_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", L->top_k, kMaxTopK);
  if (L->num_experts < L->top_k || L->num_experts > kMaxExperts)
    return fail(FTMOE_ERR_UNSUPPORTED, "num_experts=%d outside [top_k=%d, %d]", L->num_experts, L->top_k,
                kMaxExperts);
  if (L->act != FTMOE_ACT_BF16 && L->act != FTMOE_ACT_FP8_PER_TENSOR && L->act != FTMOE_ACT_MXFP8)
    return fail(FTMOE_ERR_INVALID_ARG, "act=%d is not an ftmoe_afmt", L->act);
  if (L->router_bias_mode != FTMOE_BIAS_LOGITS && L->router_bias_mode != FTMOE_BIAS_SELECT)
    return fail(FTMOE_ERR_INVALID_ARG, "router_bias_mode=%d is not an ftmoe_bias_mode", L->router_bias_mode);
  if (L->path != FTMOE_PATH_AUTO && L->path != FTMOE_PATH_DECODE && L->path != FTMOE_PATH_PREFILL)
    return fail(FTMOE_ERR_INVALID_ARG, "path=%d is not an ftmoe_path", L->path);
  if (!L->router_w) return fail(FTMOE_ERR_INVALID_ARG, "router_w is NULL");
  if (!aligned16(L->router_w)) return fail(FTMOE_ERR_INVALID_ARG, "router_w is not 16-byte aligned");
  const int fmt = L->gate_up.fmt;
  if (fmt != FTMOE_W_MXFP4 && fmt != FTMOE_W_NVFP4 && fmt != FTMOE_W_FP8_E4M3 && fmt != FTMOE_W_BF16)
    return fail(FTMOE_ERR_INVALID_ARG, "gate_up.fmt=%d is not an ftmoe_wfmt", fmt);
  if (L->act == FTMOE_ACT_FP8_PER_TENSOR && fmt != FTMOE_W_FP8_E4M3)
    return fail(FTMOE_ERR_UNSUPPORTED, "FP8 per-tensor activations need FP8 weights");
  if (L->act == FTMOE_ACT_MXFP8 && fmt != FTMOE_W_MXFP4)
    return fail(FTMOE_ERR_UNSUPPORTED, "MXFP8 activations need MXFP4 weights");
  FT_TRY(check_qweight(L->gate_up, "gate_up", fmt, L->num_experts, 2 * L->inter, L->hidden));
  FT_TRY(check_qweight(L->down, "down", fmt, L->num_experts, L->hidden, L->inter));
  if (L->shared_inter < 0) return fail(FTMOE_ERR_INVALID_ARG, "shared_inter=%d is negative", L->shared_inter);
  if (L->shared_inter > 0) {
    if (L->shared_inter % 128 || L->shared_inter > kMaxDim)
      return fail(FTMOE_ERR_UNSUPPORTED, "shared_inter=%d must be a multiple of 128, at most %d", L->shared_inter,
                  kMaxDim);
    if (L->act == FTMOE_ACT_FP8_PER_TENSOR)
      return fail(FTMOE_ERR_UNSUPPORTED, "a shared expert with FP8 per-tensor activations is not supported");
    FT_TRY(check_qweight(L->shared_gate_up, "shared_gate_up", fmt, 1, 2 * L->shared_inter, L->hidden));
    FT_TRY(check_qweight(L->shared_down, "shared_down", fmt, 1, L->hidden, L->shared_inter));
    if (!L->shared_gate_w) return fail(FTMOE_ERR_INVALID_ARG, "shared_gate_w is NULL");
    if (!aligned16(L->shared_gate_w))
      return fail(FTMOE_ERR_INVALID_ARG, "shared_gate_w is not 16-byte aligned");
  }
  return FTMOE_OK;
}

ftmoe_status check_tokens(int32_t T) {
  if (T < 0 || T > kMaxTokens) return fail(FTMOE_ERR_INVALID_ARG, "T=%d outside [0, %d]", T, kMaxTokens);
  return FTMOE_OK;
}

int max_padded(int T, int k, int E, int BM) {
  const long long n = static_cast<long long>(T) * k;
  const long long p = n + std::min<long long>(E, n) * (BM - 1);
  return static_cast<int>((p + BM - 1) / BM * BM);
}

size_t up256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

struct Plan {
  bool decode = false;    // bandwidth-bound decode kernels
  bool small_route = false;  // router via H-sliced partials + fused top-k (T <= kDecodeMaxT)
  int BM = 0, P = 0, nblocks = 0, nb_shared = 0, shared_rows = 0, S = 0, tiles = 0, n_zero = 0, rsplit = 1;
  size_t logits = 0, part = 0, ids = 0, w = 0, sg = 0, counts = 0, offsets = 0, sorted = 0, bexp = 0, npad = 0,
         scal = 0, ascratch = 0, xq = 0, xhi = 0, xlo = 0, xsc = 0, h = 0, o = 0, hs = 0, s = 0, hhi = 0, hlo = 0,
         hsc = 0, hq = 0, xs = 0, xssc = 0, hgsc = 0, hssc = 0, rplanes = 0, total = 0;
  int hsc_pitch = 0;
  bool a8 = false;        // MXFP8 activations: single codes where MXFP4 otherwise splits
  bool mx_split = false;  // MXFP4 decode: activations travel as split E4M3 pairs (or MXFP8)
  bool mx_gemm = false;   // MXFP4 prefill, routed experts: split x and h
  bool mx_gemm_shared = false;  // MXFP4 prefill, shared expert
};

Plan make_plan(const ftmoe_layer* L, int T) {
  Plan p;
  const int E = L->num_experts, k = L->top_k, H = L->hidden, I = L->inter;
  const bool shared = L->shared_inter > 0;
  p.decode = L->path == FTMOE_PATH_DECODE || (L->path == FTMOE_PATH_AUTO && T <= kDecodeAutoMaxT);
  p.small_route = T <= kDecodeMaxT;
  p.a8 = L->act == FTMOE_ACT_MXFP8;
  p.BM = p.decode ? kDecodeBM : gemm_block_m(T, k, E, L->gate_up.fmt, p.a8);
  p.P = max_padded(T, k, E, p.BM);
  p.nblocks = p.P / p.BM;
  p.nb_shared = shared ? (T + p.BM - 1) / p.BM : 0;
  p.shared_rows = p.nb_shared * p.BM;
  p.S = router_splits(H);
  p.tiles = decode_down_tiles(H);
  p.n_zero = 2 + kAmaxSlots * kAmaxStride;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  const size_t tk = static_cast<size_t>(T) * k;
  const size_t obytes = p.decode ? 4 : 2;
  if (p.small_route) {
    p.part = take(static_cast<size_t>(p.S) * T * (E + 1) * 4);
  } else {
    p.rsplit = router_splits_gemm(T, L->hidden, E + (L->shared_inter > 0 ? 1 : 0));
    p.logits = take(static_cast<size_t>(p.rsplit) * T * (E + 1) * 4);
    p.rplanes = take(router_planes_bytes(E, L->hidden, shared));
  }
  p.ids = take(tk * 4);
  p.w = take(tk * 4);
  p.sg = take(static_cast<size_t>(T) * 4);
  p.counts = take(static_cast<size_t>(E) * 4);
  p.offsets = take(static_cast<size_t>(E + 1) * 4);
  p.sorted = take(static_cast<size_t>(p.P) * 4);
  p.bexp = take(static_cast<size_t>(p.nblocks) * 4);
  p.npad = take(4);
  p.scal = take(static_cast<size_t>(p.n_zero) * 4);
  p.ascratch = take(align_scratch_bytes(T, k, E, p.BM));
  p.xq = take(L->act == FTMOE_ACT_FP8_PER_TENSOR ? static_cast<size_t>(T) * H : 0);
  p.mx_split = p.decode && L->gate_up.fmt == FTMOE_W_MXFP4;
  const size_t lo_planes = p.a8 ? 0 : 1;   // MXFP8 activations have no lo codes
  if (p.mx_split) {
    p.xhi = take(static_cast<size_t>(T) * H);
    p.xlo = take(lo_planes * T * H);
    p.xsc = take(static_cast<size_t>(T) * xsc_pitch_of(H));
  }
  if (p.mx_split) {
    // h in the split form the MXFP4 down kernel multiplies
    const int imax = shared && L->shared_inter > I ? L->shared_inter : I;
    const size_t hbytes = static_cast<size_t>(p.P) * I + static_cast<size_t>(p.shared_rows) * L->shared_inter;
    p.hsc_pitch = xsc_pitch_of(imax);
    p.hhi = take(hbytes);
    p.hlo = take(lo_planes * hbytes);
    p.hsc = take(static_cast<size_t>(p.P + p.shared_rows) * p.hsc_pitch);
  } else {
    // bf16 h, or for MXFP4 its split form (2 code bytes per element + scales)
    p.mx_gemm = !p.decode && L->gate_up.fmt == FTMOE_W_MXFP4;
    p.mx_gemm_shared = !p.decode && shared && L->shared_gate_up.fmt == FTMOE_W_MXFP4;
    if (p.mx_gemm || p.mx_gemm_shared) {
      p.xs = take(static_cast<size_t>(T) * H * (1 + lo_planes));
      p.xssc = take(static_cast<size_t>(T) * (H / 32));
    }
    p.h = take(static_cast<size_t>(p.P) * I * 2);
    if (p.mx_gemm) p.hgsc = take(static_cast<size_t>(p.P) * (I / 32));
    if (shared) p.hs = take(static_cast<size_t>(p.shared_rows) * L->shared_inter * 2);
    if (p.mx_gemm_shared) p.hssc = take(static_cast<size_t>(p.shared_rows) * (L->shared_inter / 32));
    // FP8 activations, prefill: h quantised once for the down GEMM
    if (!p.decode && L->act == FTMOE_ACT_FP8_PER_TENSOR) p.hq = take(static_cast<size_t>(p.P) * I);
  }
  p.o = take(tk * H * obytes);
  if (shared) p.s = take(static_cast<size_t>(T) * H * obytes);
  p.total = off;
  return p;
}

QW to_qw(const ftmoe_qweight& q) {
  QW w{};
  w.fmt = q.fmt;
  w.n = q.n;
  w.k = q.k;
  w.codes = static_cast<const uint8_t*>(q.codes);
  w.scales = static_cast<const uint8_t*>(q.block_scales);
  w.tscale = q.tensor_scales;
  w.packed = static_cast<const uint8_t*>(q.packed);
  w.rowsc = q.row_scales;
  return w;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

ftmoe_status check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (ws_bytes < p.total)
    return fail(FTMOE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, p.total);
  if (p.total > 0 && !ws) return fail(FTMOE_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(FTMOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return FTMOE_OK;
}

// Router.  With `align` (decode plans with few tokens) the fused top-k kernel
// also writes the block alignment and clears the per-call counters, so the
// experts stage can skip its own align launch.  With `gemm_x` (prefill plans
// with MXFP4 experts) the router GEMM also writes x in the form the expert
// GEMMs read, so the experts stage can skip its x conversion.
ftmoe_status enqueue_route(const ftmoe_layer* L, const uint16_t* x, int T, const Plan& p, void* ws, int32_t* ids,
                           float* w, float* sg, bool align, bool gemm_x, hipStream_t s) {
  const bool shared = L->shared_inter > 0;
  const int E = L->num_experts, k = L->top_k;
  if (p.small_route) {
    float* part = at<float>(ws, p.part);
    const bool split = align && p.mx_split;  // the experts stage of this call reads the split (MXFP8) x
    FT_HIP(timed("router_partial", s,
                 [&] {
                   return launch_router_partial(x, T, L->hidden, L->router_w, E, shared ? L->shared_gate_w : nullptr,
                                                part, split ? at<uint8_t>(ws, p.xhi) : nullptr,
                                                split && !p.a8 ? at<uint8_t>(ws, p.xlo) : nullptr,
                                                split ? at<uint8_t>(ws, p.xsc) : nullptr, xsc_pitch_of(L->hidden), s);
                 }),
           "router launch");
    FT_HIP(timed("topk_align", s,
                 [&] {
                   return launch_topk_align_decode(part, p.S, T, E, k, L->router_bias,
                                                   L->router_bias_mode == FTMOE_BIAS_SELECT, shared, ids, w, sg,
                                                   at<int32_t>(ws, p.counts), at<int32_t>(ws, p.offsets),
                                                   at<int32_t>(ws, p.sorted), at<int32_t>(ws, p.bexp),
                                                   at<int32_t>(ws, p.npad), align ? p.P : 0,
                                                   at<uint32_t>(ws, p.scal), align ? p.n_zero : 0, s);
                 }),
           "top-k launch");
    return FTMOE_OK;
  }
  float* logits = at<float>(ws, p.logits);
  uint16_t* planes = at<uint16_t>(ws, p.rplanes);
  FT_HIP(timed("router_split", s,
               [&] {
                 return launch_router_split(L->router_w, E, L->hidden, shared ? L->shared_gate_w : nullptr, planes,
                                            s);
               }),
         "router split launch");
  FT_HIP(timed("router_logits", s,
               [&] {
                 return launch_router_logits(x, T, L->hidden, L->router_w, E, shared ? L->shared_gate_w : nullptr,
                                             planes, logits, gemm_x ? at<uint8_t>(ws, p.xs) : nullptr,
                                             gemm_x ? at<uint8_t>(ws, p.xssc) : nullptr, p.a8, s);
               }),
         "router logits launch");
  FT_HIP(timed("topk", s,
               [&] {
                 return launch_topk(logits, p.rsplit, T, E, k, L->router_bias,
                                    L->router_bias_mode == FTMOE_BIAS_SELECT, shared, ids, w, sg, s);
               }),
         "top-k launch");
  return FTMOE_OK;
}

// Expert passes over an expert-slot pool: pass i runs the routed gate_up and
// down of the experts that table i maps to a slot (the others' blocks exit at
// once).  Host hooks: before(i) is called before pass i is enqueued (it makes
// the stream wait for that pass's copies into the pool), after(i) right
// after (it marks the pass done and starts the next pass's copies).  The
// shared expert runs in pass 0; align, the activation preparation and the
// combine run once.
struct Passes {
  int n = 1;
  const int32_t* const* tables = nullptr;   // n device tables [E], or NULL: one pass, no table
  ftmoe_status (*before)(void* ctx, int i) = nullptr;
  ftmoe_status (*after)(void* ctx, int i) = nullptr;
  // after the last pass, before the combine: o is the expert output buffer,
  // fp32 [T*k][H] (decode) or bf16 (prefill)
  ftmoe_status (*before_combine)(void* ctx, void* o, bool fp32) = nullptr;
  void* ctx = nullptr;
};

ftmoe_status enqueue_experts(const ftmoe_layer* L, const uint16_t* x, int T, const int32_t* ids, const float* w,
                             const float* sg, const Plan& p, void* ws, uint16_t* y, bool aligned, bool x_ready,
                             hipStream_t s, const Passes& passes = Passes{}) {
  const int E = L->num_experts, k = L->top_k, H = L->hidden, I = L->inter;
  const bool fp8act = L->act == FTMOE_ACT_FP8_PER_TENSOR;
  const bool shared = L->shared_inter > 0;
  uint32_t* scal = at<uint32_t>(ws, p.scal);
  uint32_t* amax_x = scal + 0;
  uint32_t* amax_h = scal + 1;
  uint32_t* amax_slots = scal + 2;
  int32_t* sorted = at<int32_t>(ws, p.sorted);
  int32_t* bexp = at<int32_t>(ws, p.bexp);
  if (!aligned) {
    FT_HIP(timed("align", s,
                 [&] {
                   return launch_align(ids, T, k, E, p.BM, at<int32_t>(ws, p.counts), at<int32_t>(ws, p.offsets),
                                       sorted, bexp, at<int32_t>(ws, p.npad), at<void>(ws, p.ascratch), scal,
                                       p.n_zero, s);
                 }),
           "align launch");
  }
  const uint8_t* xq = nullptr;
  if (fp8act) {
    FT_HIP(timed("amax_x", s, [&] { return launch_amax_bf16(x, static_cast<int64_t>(T) * H, amax_x, s); }),
           "amax launch");
    FT_HIP(timed("quant_x", s,
                 [&] {
                   return launch_quant_fp8(x, static_cast<int64_t>(T) * H, amax_x, at<uint8_t>(ws, p.xq), nullptr, s);
                 }),
           "quantise launch");
    xq = at<uint8_t>(ws, p.xq);
  }
  const QW gu = to_qw(L->gate_up), dn = to_qw(L->down);
  uint16_t* h = at<uint16_t>(ws, p.h);
  const uint32_t* ax = fp8act ? amax_x : nullptr;
  uint32_t* ah = fp8act ? amax_h : nullptr;
  uint32_t* ahs = fp8act ? amax_slots : nullptr;
  uint16_t* hs = shared ? at<uint16_t>(ws, p.hs) : nullptr;

  if (p.decode) {
    if (p.mx_split && !aligned) {
      // the router of this call did not produce the split x
      FT_HIP(timed("x_split", s,
                   [&] {
                     return launch_x_split(x, T, H, xsc_pitch_of(H), at<uint8_t>(ws, p.xhi),
                                           p.a8 ? nullptr : at<uint8_t>(ws, p.xlo),
                                           at<uint8_t>(ws, p.xsc), s);
                   }),
             "x split launch");
    }
    DecodeArgs a{};
    a.gu = gu;
    a.dn = dn;
    if (shared) {
      a.sgu = to_qw(L->shared_gate_up);
      a.sdn = to_qw(L->shared_down);
    }
    a.sorted_ids = sorted;
    a.block_expert = bexp;
    a.T = T;
    a.k = k;
    a.H = H;
    a.I = I;
    a.Is = shared ? L->shared_inter : 0;
    a.nb_routed = p.nblocks;
    a.nb_shared = p.nb_shared;
    a.x = x;
    a.a8 = p.a8 ? 1 : 0;
    if (p.mx_split) {
      a.xhi = at<uint8_t>(ws, p.xhi);
      a.xlo = p.a8 ? nullptr : at<uint8_t>(ws, p.xlo);
      a.xsc = at<uint8_t>(ws, p.xsc);
      a.xsc_pitch = xsc_pitch_of(H);
    }
    a.xq = xq;
    a.amax_x = ax;
    a.h = h;
    a.hs = hs;
    if (p.mx_split) {
      a.hhi = at<uint8_t>(ws, p.hhi);
      a.hlo = p.a8 ? nullptr : at<uint8_t>(ws, p.hlo);
      a.hsc = at<uint8_t>(ws, p.hsc);
      a.hsc_pitch = p.hsc_pitch;
    }
    a.amax_slots = ahs;
    a.amax_h = ah;
    a.o32 = at<float>(ws, p.o);
    a.s32 = shared ? at<float>(ws, p.s) : nullptr;
    a.w = w;
    a.sg = shared ? sg : nullptr;
    a.y = y;
    // a one-token step in one pass runs down and combine as one launch
    const bool fused = passes.n == 1 && !passes.tables && !passes.before_combine && decode_fused_one_token(a);
    for (int i = 0; i < passes.n; ++i) {
      if (passes.before) FT_TRY(passes.before(passes.ctx, i));
      if (passes.tables) a.gu.slot_of = a.dn.slot_of = passes.tables[i];
      a.nb_shared = i == 0 ? p.nb_shared : 0;
      FT_HIP(timed("decode_gateup", s, [&] { return launch_decode_gateup(a, s); }), "decode gate_up launch");
      if (fp8act) FT_HIP(timed("amax_h", s, [&] { return launch_amax_fold(ahs, ah, s); }), "amax fold launch");
      if (fused) {
        FT_HIP(timed("decode_down", s, [&] { return launch_decode_down_combine1(a, s); }),
               "decode down + combine launch");
        return FTMOE_OK;
      }
      FT_HIP(timed("decode_down", s, [&] { return launch_decode_down(a, s); }), "decode down launch");
      if (passes.after) FT_TRY(passes.after(passes.ctx, i));
    }
    a.nb_shared = p.nb_shared;
    if (passes.before_combine) FT_TRY(passes.before_combine(passes.ctx, a.o32, true));
    FT_HIP(timed("combine", s, [&] { return launch_decode_combine(a, s); }), "combine launch");
    return FTMOE_OK;
  }

  Rows rr;
  rr.sorted_ids = sorted;
  rr.block_expert = bexp;
  rr.counts = at<int32_t>(ws, p.counts);
  rr.offsets = at<int32_t>(ws, p.offsets);
  rr.n_flat = T * k;
  rr.top_k = k;
  rr.num_blocks = p.nblocks;
  rr.block_m = p.BM;
  Rows rs;
  rs.sorted_ids = nullptr;
  rs.block_expert = nullptr;
  rs.counts = nullptr;
  rs.offsets = nullptr;
  rs.n_flat = T;
  rs.top_k = 1;
  rs.num_blocks = p.nb_shared;
  rs.block_m = p.BM;
  uint16_t* o = at<uint16_t>(ws, p.o);
  uint16_t* sh = shared ? at<uint16_t>(ws, p.s) : nullptr;
  GemmAct xa{};
  xa.bf16 = x;
  xa.q = xq;
  xa.amax = ax;
  if (p.mx_gemm || p.mx_gemm_shared) {
    xa.split = at<uint8_t>(ws, p.xs);
    xa.split_sc = at<uint8_t>(ws, p.xssc);
    xa.mx8 = p.a8;
    if (!x_ready) {   // the router of this call did not write it
      FT_HIP(timed("x_split", s,
                   [&] {
                     return launch_x_split_gemm(x, T, H, at<uint8_t>(ws, p.xs), at<uint8_t>(ws, p.xssc), p.a8, s);
                   }),
             "x split launch");
    }
  }
  uint8_t* hgsc = p.mx_gemm ? at<uint8_t>(ws, p.hgsc) : nullptr;
  GemmAct ha{};
  ha.bf16 = h;
  ha.amax = ah;
  if (p.mx_gemm) {
    ha.split = reinterpret_cast<const uint8_t*>(h);
    ha.split_sc = hgsc;
    ha.mx8 = p.a8;
  }
  for (int i = 0; i < passes.n; ++i) {
    if (passes.before) FT_TRY(passes.before(passes.ctx, i));
    QW gup = gu, dnp = dn;
    if (passes.tables) gup.slot_of = dnp.slot_of = passes.tables[i];
    FT_HIP(timed("gemm_gateup", s, [&] { return launch_gemm_gateup(gup, rr, xa, H, I, h, hgsc, ahs, s); }),
           "gate_up GEMM launch");
    if (fp8act) FT_HIP(timed("amax_h", s, [&] { return launch_amax_fold(ahs, ah, s); }), "amax fold launch");
    if (fp8act) {
      uint8_t* hq = at<uint8_t>(ws, p.hq);
      FT_HIP(timed("quant_h", s,
                   [&] { return launch_quant_fp8(h, static_cast<int64_t>(p.P) * I, ah, hq, nullptr, s); }),
             "quantise launch");
      ha.q = hq;
    }
    FT_HIP(timed("gemm_down", s, [&] { return launch_gemm_down(dnp, rr, ha, H, I, o, s); }), "down GEMM launch");
    if (passes.after) FT_TRY(passes.after(passes.ctx, i));
  }
  if (shared) {
    GemmAct xs = xa;
    xs.q = nullptr;
    xs.amax = nullptr;
    uint8_t* hssc = p.mx_gemm_shared ? at<uint8_t>(ws, p.hssc) : nullptr;
    FT_HIP(timed("gemm_shared_gateup", s,
                 [&] {
                   return launch_gemm_gateup(to_qw(L->shared_gate_up), rs, xs, H, L->shared_inter, hs, hssc, nullptr,
                                             s);
                 }),
           "shared gate_up GEMM launch");
    GemmAct hsa{};
    hsa.bf16 = hs;
    if (p.mx_gemm_shared) {
      hsa.split = reinterpret_cast<const uint8_t*>(hs);
      hsa.split_sc = hssc;
      hsa.mx8 = p.a8;
    }
    FT_HIP(timed("gemm_shared_down", s,
                 [&] { return launch_gemm_down(to_qw(L->shared_down), rs, hsa, H, L->shared_inter, sh, s); }),
           "shared down GEMM launch");
  }
  if (passes.before_combine) FT_TRY(passes.before_combine(passes.ctx, o, false));
  FT_HIP(timed("combine", s, [&] { return launch_combine(o, w, T, k, H, shared ? sg : nullptr, sh, y, s); }),
         "combine launch");
  return FTMOE_OK;
}

// The whole layer on a checked workspace: route (with the fused top-k and
// align of small decode batches), then the experts.
ftmoe_status enqueue_forward(const ftmoe_layer* layer, const uint16_t* x, int T, const Plan& p, void* ws, uint16_t* y,
                             int32_t* topk_ids_out, float* topk_w_out, hipStream_t s) {
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, p.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, p.w);
  float* sg = at<float>(ws, p.sg);
  const bool fused_align = p.decode && p.small_route;
  const bool gemm_x = !p.small_route && (p.mx_gemm || p.mx_gemm_shared);
  FT_TRY(enqueue_route(layer, x, T, p, ws, ids, w, sg, fused_align, gemm_x, s));
  return enqueue_experts(layer, x, T, ids, w, sg, p, ws, y, fused_align, gemm_x, s);
}

// ---- allocation-free forward: a fixed scratch array in device memory ----
// The workspace of ftmoe_forward_noalloc is this file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).
// In host code its name is not a device address: the address is asked of
// HIP once per device, with that device current, and only that address is
// used.  Every call on one GPU shares the array (overlapping calls race);
// the forward zeroes what must start at zero with kernels of its own.
constexpr size_t kScratchBytes = static_cast<size_t>(32) << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ftmoe_status device_scratch(void** out) {
  int dev = 0;
  FT_HIP(hipGetDevice(&dev), "current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(FTMOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    FT_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return fail(FTMOE_ERR_HIP, "scratch address is not usable");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FTMOE_OK;
}

// ---- expert-slot pool ----
// Bytes of one expert's matrices in each array of a matrix set.
struct SetBytes {
  size_t codes = 0, scales = 0, ts = 0;
};

SetBytes set_bytes(const ftmoe_qweight& q) {
  SetBytes b;
  const size_t nk = static_cast<size_t>(q.n) * q.k;
  switch (q.fmt) {
    case FTMOE_W_MXFP4: b.codes = nk / 2; b.scales = nk / 32; break;
    case FTMOE_W_NVFP4: b.codes = nk / 2; b.scales = nk / 16; b.ts = 4; break;
    case FTMOE_W_FP8_E4M3: b.codes = nk; b.ts = 4; break;
    default: b.codes = 2 * nk; break;   // BF16
  }
  if (b.ts && q.row_scales) b.ts = 4 * static_cast<size_t>(q.n);
  return b;
}

// Pool regions: gate_up codes, scales, multipliers, then down's, each
// [slots][per-expert bytes], then the residency table [E] (slot of each
// expert, -1 if none), each 256-byte aligned.
struct PoolLayout {
  SetBytes gu, dn;
  size_t gu_codes = 0, gu_scales = 0, gu_ts = 0, dn_codes = 0, dn_scales = 0, dn_ts = 0, resid = 0, total = 0;
};

PoolLayout pool_layout(const ftmoe_qweight& gu, const ftmoe_qweight& dn, int slots, int E) {
  PoolLayout pl;
  pl.gu = set_bytes(gu);
  pl.dn = set_bytes(dn);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += up256(bytes);
    return at;
  };
  pl.gu_codes = take(pl.gu.codes * slots);
  pl.gu_scales = take(pl.gu.scales * slots);
  pl.gu_ts = take(pl.gu.ts * slots);
  pl.dn_codes = take(pl.dn.codes * slots);
  pl.dn_scales = take(pl.dn.scales * slots);
  pl.dn_ts = take(pl.dn.ts * slots);
  pl.resid = take(static_cast<size_t>(E) * 4);
  pl.total = off;
  return pl;
}

}  // namespace

// Residency state of one layer (the C ABI's opaque ftmoe_cache).
struct ftmoe_cache {
  ftmoe_layer layer{};          // gate_up and down point into the pool
  ftmoe_qweight host_gu{}, host_dn{};
  int slots = 0, E = 0;
  PoolLayout pl;
  uint8_t* pool = nullptr;
  std::vector<int> slot_expert, expert_slot;   // -1: empty / not resident
  std::vector<int64_t> last_use;               // per slot; -1: never
  std::vector<char> filled;                    // per slot: its expert's bytes are in it (or their copy is enqueued)
  int64_t clock = 0, hits = 0, misses = 0, bytes = 0, passes = 0;
  // copies run on their own stream, ordered against the passes by events
  hipStream_t copy_stream = nullptr;
  hipStream_t x_stream = nullptr;              // device -> host copies of x for host-computed rows
  std::vector<hipEvent_t> ev_copied, ev_done;  // per pass: its copies landed / its kernels ran
  // per-call state
  int32_t* pin = nullptr;                      // pinned host words: the routing ids [T*k], then the
  size_t pin_words = 0;                        // pass tables [passes][E] (slot of each expert, -1 if not in the pass)
  std::vector<std::vector<int>> copy_e, copy_s;   // per pass: experts to copy and their slots
  std::vector<int> copy_after;                 // per pass: the last earlier pass that reads a slot it overwrites, or -1
  hipStream_t stream = nullptr;                // the stream of the last call
  bool called = false;
  // device-visible addresses of the host arrays (pinned, mapped memory): the
  // pool is then filled by one kernel per pass instead of one DMA per array
  int zero_copy = -1;                          // -1: not probed yet; 0: DMA copies; 1: fill kernel
  const uint8_t* dev_src[kFillArrays] = {};
  // host compute of missing experts (co-execution); cost model in seconds
  std::unique_ptr<ftmoe_host::Pool> host_pool;
  double host_expert_s = 0, host_row_s = 0, link_bps = 0;
  bool host_adaptive = false;                  // calibrated model: rescaled by the measured host times
  double host_scale = 1;                       // measured / modelled host time (running average)
  double host_predicted = 0;                   // modelled host time of this call's host experts
  int64_t host_experts = 0, host_rows = 0;
  double host_seconds = 0;
  // per-call host work: x [T][H] copied back, the rows' tokens, experts, flat ids, outputs
  void* hx = nullptr;
  size_t hx_bytes = 0;
  hipEvent_t ev_x = nullptr;
  // device residency table (in the pool) read by each step's first pass
  bool resid_init = false;
  int32_t* resid_host = nullptr;               // pinned [E]
  hipEvent_t ev_ids = nullptr;                 // the routing ids have reached the host
  // per-call pass state, completed by the first pass's hook
  Passes run;
  std::vector<const int32_t*> tptr;
  int32_t* tables_dev = nullptr;               // workspace tables of passes 1..
  size_t n_ids = 0;
  int step_k = 0, step_T = 0;
  std::vector<int32_t> h_tok, h_ex;
  int32_t* h_flat = nullptr;                   // pinned [rows]
  float* h_out = nullptr;                      // pinned [rows][H]
  size_t h_rows_cap = 0;
  int h_n = 0, h_T = 0;

  ~ftmoe_cache() {
    for (hipStream_t* st : {&copy_stream, &x_stream})
      if (*st) {
        (void)hipStreamSynchronize(*st);
        (void)hipStreamDestroy(*st);
      }
    if (pin) (void)hipHostFree(pin);
    if (resid_host) (void)hipHostFree(resid_host);
    if (ev_ids) (void)hipEventDestroy(ev_ids);
    if (hx) (void)hipHostFree(hx);
    if (h_flat) (void)hipHostFree(h_flat);
    if (h_out) (void)hipHostFree(h_out);
    if (ev_x) (void)hipEventDestroy(ev_x);
    for (hipEvent_t e : ev_copied) (void)hipEventDestroy(e);
    for (hipEvent_t e : ev_done) (void)hipEventDestroy(e);
  }
};

namespace {

// An expert whose bytes are in (or on their way to) its slot.
bool resident(const ftmoe_cache* c, int e) { return c->expert_slot[e] >= 0 && c->filled[c->expert_slot[e]]; }

// The LRU policy (see ftmoe_cache_plan).  `fill`: the caller enqueues the
// copies of the misses (a forward); otherwise (a plan alone) the slots given
// to missing experts stay unfilled, and a later forward copies into them.
// A planned but unfilled expert keeps its slot and counts as a miss again.
ftmoe_status cache_plan(ftmoe_cache* c, const int32_t* experts, int n, int32_t* out_slot, int32_t* out_miss,
                        bool fill) {
  if (n > c->slots)
    return fail(FTMOE_ERR_UNSUPPORTED, "%d experts do not fit %d slots", n, c->slots);
  std::vector<char> seen(c->E, 0), needed(c->slots, 0);
  for (int i = 0; i < n; ++i) {
    const int e = experts[i];
    if (e < 0 || e >= c->E) return fail(FTMOE_ERR_INVALID_ARG, "expert %d outside [0, %d)", e, c->E);
    if (seen[e]) return fail(FTMOE_ERR_INVALID_ARG, "expert %d listed twice", e);
    seen[e] = 1;
    if (c->expert_slot[e] >= 0) needed[c->expert_slot[e]] = 1;
  }
  // free slots in least-recently-used order (never used first, then by age, then by index)
  std::vector<int> cand;
  for (int sl = 0; sl < c->slots; ++sl)
    if (!needed[sl]) cand.push_back(sl);
  std::stable_sort(cand.begin(), cand.end(), [&](int a, int b) { return c->last_use[a] < c->last_use[b]; });
  size_t next = 0;
  ++c->clock;
  for (int i = 0; i < n; ++i) {
    const int e = experts[i];
    int sl = c->expert_slot[e];
    const bool miss = !resident(c, e);
    if (sl < 0) {
      sl = cand[next++];
      if (c->slot_expert[sl] >= 0) c->expert_slot[c->slot_expert[sl]] = -1;
      c->slot_expert[sl] = e;
      c->expert_slot[e] = sl;
    }
    if (miss) {
      c->filled[sl] = fill ? 1 : 0;
      ++c->misses;
    } else {
      ++c->hits;
    }
    c->last_use[sl] = c->clock;
    if (out_slot) out_slot[i] = sl;
    if (out_miss) out_miss[i] = miss ? 1 : 0;
  }
  return FTMOE_OK;
}

// Copies of pass i on the copy stream: each missing expert's gate_up and down
// arrays, host -> its slot, after the last earlier pass that reads one of the
// slots they overwrite; then the pass's "copied" event.
ftmoe_status cache_copy_pass(ftmoe_cache* c, int i) {
  if (c->copy_e[i].empty()) return FTMOE_OK;
  const hipStream_t cs = c->copy_stream;
  if (c->copy_after[i] >= 0) FT_HIP(hipStreamWaitEvent(cs, c->ev_done[c->copy_after[i]], 0), "copy stream wait");
  const PoolLayout& pl = c->pl;
  if (c->zero_copy == 1) {
    FillArgs fa{};
    const size_t dst_off[kFillArrays] = {pl.gu_codes, pl.gu_scales, pl.gu_ts, pl.dn_codes, pl.dn_scales, pl.dn_ts};
    const size_t per[kFillArrays] = {pl.gu.codes, pl.gu.scales, pl.gu.ts, pl.dn.codes, pl.dn.scales, pl.dn.ts};
    size_t expert_bytes = 0;
    for (int j = 0; j < kFillArrays; ++j) {
      fa.src[j] = c->dev_src[j];
      fa.dst[j] = c->pool + dst_off[j];
      fa.bytes[j] = c->dev_src[j] ? static_cast<uint32_t>(per[j]) : 0u;
      expert_bytes += fa.bytes[j];
    }
    const int n = static_cast<int>(c->copy_e[i].size());
    for (int a = 0; a < n; a += kFillMax) {
      fa.n = std::min(kFillMax, n - a);
      for (int m = 0; m < fa.n; ++m) {
        fa.e[m] = c->copy_e[i][a + m];
        fa.s[m] = c->copy_s[i][a + m];
      }
      FT_HIP(launch_expert_fill(fa, cs), "pool fill launch");
    }
    c->bytes += static_cast<int64_t>(expert_bytes) * n;
    FT_HIP(hipEventRecord(c->ev_copied[i], cs), "copy event");
    return FTMOE_OK;
  }
  auto copy = [&](size_t dst_off, const void* src, size_t bytes) -> hipError_t {
    if (bytes == 0) return hipSuccess;
    c->bytes += static_cast<int64_t>(bytes);
    return hipMemcpyAsync(c->pool + dst_off, src, bytes, hipMemcpyHostToDevice, cs);
  };
  for (size_t m = 0; m < c->copy_e[i].size(); ++m) {
    const size_t e = static_cast<size_t>(c->copy_e[i][m]), sl = static_cast<size_t>(c->copy_s[i][m]);
    const uint8_t* gc = static_cast<const uint8_t*>(c->host_gu.codes);
    const uint8_t* gs = static_cast<const uint8_t*>(c->host_gu.block_scales);
    const uint8_t* gt = reinterpret_cast<const uint8_t*>(c->host_gu.tensor_scales);
    const uint8_t* dc = static_cast<const uint8_t*>(c->host_dn.codes);
    const uint8_t* ds = static_cast<const uint8_t*>(c->host_dn.block_scales);
    const uint8_t* dt = reinterpret_cast<const uint8_t*>(c->host_dn.tensor_scales);
    FT_HIP(copy(pl.gu_codes + sl * pl.gu.codes, gc + e * pl.gu.codes, pl.gu.codes), "expert copy");
    if (pl.gu.scales) FT_HIP(copy(pl.gu_scales + sl * pl.gu.scales, gs + e * pl.gu.scales, pl.gu.scales), "expert copy");
    if (pl.gu.ts) FT_HIP(copy(pl.gu_ts + sl * pl.gu.ts, gt + e * pl.gu.ts, pl.gu.ts), "expert copy");
    FT_HIP(copy(pl.dn_codes + sl * pl.dn.codes, dc + e * pl.dn.codes, pl.dn.codes), "expert copy");
    if (pl.dn.scales) FT_HIP(copy(pl.dn_scales + sl * pl.dn.scales, ds + e * pl.dn.scales, pl.dn.scales), "expert copy");
    if (pl.dn.ts) FT_HIP(copy(pl.dn_ts + sl * pl.dn.ts, dt + e * pl.dn.ts, pl.dn.ts), "expert copy");
  }
  FT_HIP(hipEventRecord(c->ev_copied[i], cs), "copy event");
  return FTMOE_OK;
}

// Grows the pinned host buffer to `words` (after the last call's work, which may read it, is done).
ftmoe_status cache_host_buffer(ftmoe_cache* c, size_t words) {
  if (words <= c->pin_words) return FTMOE_OK;
  if (c->pin) {
    if (c->called) FT_HIP(hipStreamSynchronize(c->stream), "previous stream");
    (void)hipHostFree(c->pin);
    c->pin = nullptr;
    c->pin_words = 0;
  }
  void* p = nullptr;
  FT_HIP(hipHostMalloc(&p, words * 4, hipHostMallocDefault), "pinned host buffer");
  c->pin = static_cast<int32_t*>(p);
  c->pin_words = words;
  return FTMOE_OK;
}

// Whether every host array has a device-visible address (pinned, mapped
// memory) and fits the fill kernel's 32-bit per-expert sizes; else the pool
// is filled by DMA copies.
ftmoe_status cache_probe_zero_copy(ftmoe_cache* c) {
  const void* host[kFillArrays] = {c->host_gu.codes, c->host_gu.block_scales, c->host_gu.tensor_scales,
                                   c->host_dn.codes, c->host_dn.block_scales, c->host_dn.tensor_scales};
  const size_t per[kFillArrays] = {c->pl.gu.codes, c->pl.gu.scales, c->pl.gu.ts,
                                   c->pl.dn.codes, c->pl.dn.scales, c->pl.dn.ts};
  bool ok = true;
  for (int j = 0; j < kFillArrays; ++j) {
    c->dev_src[j] = nullptr;
    if (!host[j] || per[j] == 0) continue;
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(host[j]), 0) != hipSuccess || !d) {
      (void)hipGetLastError();   // not pinned and mapped: clear the error, use DMA copies
      ok = false;
      break;
    }
    if (per[j] % 4 || per[j] > 0xFFFFFFFFu) ok = false;
    c->dev_src[j] = static_cast<const uint8_t*>(d);
  }
  c->zero_copy = ok ? 1 : 0;
  return FTMOE_OK;
}

// Pass hooks: pass 0 starts its own copies; pass i waits for its copies; after
// pass i is enqueued its "done" event is recorded and pass i + 1's copies
// start, so they overlap pass i's kernels unless they evict what it reads.
ftmoe_status cache_before_pass(void* ctx, int i) {
  ftmoe_cache* c = static_cast<ftmoe_cache*>(ctx);
  if (i == 0) FT_TRY(cache_copy_pass(c, 0));
  if (!c->copy_e[i].empty()) FT_HIP(hipStreamWaitEvent(c->stream, c->ev_copied[i], 0), "pass wait");
  return FTMOE_OK;
}

ftmoe_status cache_after_pass(void* ctx, int i) {
  ftmoe_cache* c = static_cast<ftmoe_cache*>(ctx);
  FT_HIP(hipEventRecord(c->ev_done[i], c->stream), "pass event");
  if (i + 1 < static_cast<int>(c->copy_e.size())) FT_TRY(cache_copy_pass(c, i + 1));
  return FTMOE_OK;
}

// Misses per pass when a step's experts do not all fit: half the pool, so
// one pass's copies can land while the previous pass runs.
int cache_group(const ftmoe_cache* c) { return std::max(1, c->slots / 2); }

ftmoe_host::Mat host_mat(const ftmoe_qweight& q) {
  ftmoe_host::Mat m;
  m.fmt = q.fmt;
  m.n = q.n;
  m.k = q.k;
  m.codes = static_cast<const uint8_t*>(q.codes);
  m.scales = static_cast<const uint8_t*>(q.block_scales);
  m.tscale = q.tensor_scales;
  m.rowsc = q.row_scales;
  return m;
}

// Host-computed expert rows: wait for x on the host, compute, and scatter
// the rows into the device path's o buffer (the passes run meanwhile).
ftmoe_status cache_host_rows(void* ctx, void* o, bool fp32) {
  ftmoe_cache* c = static_cast<ftmoe_cache*>(ctx);
  if (c->h_n == 0) return FTMOE_OK;
  const ftmoe_layer& L = c->layer;
  FT_HIP(hipEventSynchronize(c->ev_x), "x copy");
  const auto t0 = std::chrono::steady_clock::now();
  const ftmoe_host::Mat gu = host_mat(c->host_gu), dn = host_mat(c->host_dn);
  if (!ftmoe_host::expert_rows(*c->host_pool, gu, dn, L.hidden, L.inter, L.act == FTMOE_ACT_MXFP8,
                               static_cast<const uint16_t*>(c->hx), c->h_tok.data(), c->h_ex.data(), c->h_n,
                               c->h_out))
    return fail(FTMOE_ERR_UNSUPPORTED, "host expert compute needs AVX2 and FMA");
  const double took = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  c->host_seconds += took;
  if (c->host_adaptive && c->host_predicted > 0)
    c->host_scale = 0.7 * c->host_scale + 0.3 * c->host_scale * took / c->host_predicted;
  void *rows = nullptr, *flat = nullptr;
  FT_HIP(hipHostGetDevicePointer(&rows, c->h_out, 0), "host rows address");
  FT_HIP(hipHostGetDevicePointer(&flat, c->h_flat, 0), "host rows address");
  FT_HIP(launch_host_rows_scatter(static_cast<const float*>(rows), static_cast<const int32_t*>(flat), c->h_n,
                                  L.hidden, fp32 ? static_cast<float*>(o) : nullptr,
                                  fp32 ? nullptr : static_cast<uint16_t*>(o), c->stream),
         "host rows scatter launch");
  return FTMOE_OK;
}

// Pinned host buffer p of at least `bytes` (grown; the caller has made sure no device work reads the old one).
ftmoe_status grow_pinned(void** p, size_t* cap, size_t bytes) {
  if (bytes <= *cap) return FTMOE_OK;
  if (*p) (void)hipHostFree(*p);
  *p = nullptr;
  *cap = 0;
  FT_HIP(hipHostMalloc(p, bytes, hipHostMallocDefault), "pinned host buffer");
  *cap = bytes;
  return FTMOE_OK;
}

// The co-execution split (bandwidth-adaptive): the missing experts, fewest
// routed rows first (then by index), go to the host while that shortens the
// step: q minimises max(sum of host times of the first q, sum of link times
// of the rest), host time = expert_s + rows * row_s, link time = bytes /
// link rate; ties take the smaller q.  Returns q; `missing` is reordered.
int host_split(ftmoe_cache* c, std::vector<int>& missing, const std::vector<int>& rows) {
  c->host_predicted = 0;
  if (!c->host_pool || missing.empty()) return 0;
  std::stable_sort(missing.begin(), missing.end(), [&](int a, int b) { return rows[a] < rows[b]; });
  const double bytes = static_cast<double>(c->pl.gu.codes + c->pl.gu.scales + c->pl.gu.ts + c->pl.dn.codes +
                                           c->pl.dn.scales + c->pl.dn.ts);
  const int m = static_cast<int>(missing.size());
  double link_rest = m * bytes / c->link_bps, host = 0, best = link_rest;
  int q_best = 0;
  double host_best = 0;
  for (int q = 1; q <= m; ++q) {
    host += c->host_scale * (c->host_expert_s + rows[missing[q - 1]] * c->host_row_s);
    link_rest -= bytes / c->link_bps;
    const double t = std::max(host, link_rest);
    if (t < best) {
      best = t;
      q_best = q;
      host_best = host;
    }
  }
  c->host_predicted = host_best;
  return q_best;
}

// The copy stream, per-pass events, the routing event and the pinned
// residency table (host resources of the cache, made once).
int cache_max_passes(const ftmoe_cache* c);
int cache_group(const ftmoe_cache* c);
ftmoe_status cache_host_resources(ftmoe_cache* c) {
  if (c->zero_copy < 0) FT_TRY(cache_probe_zero_copy(c));
  for (hipStream_t* st : {&c->copy_stream, &c->x_stream})
    if (!*st && hipStreamCreateWithFlags(st, hipStreamNonBlocking) != hipSuccess) {
      *st = nullptr;
      return fail(FTMOE_ERR_HIP, "copy stream creation failed");
    }
  if (!c->ev_ids) FT_HIP(hipEventCreateWithFlags(&c->ev_ids, hipEventDisableTiming), "event creation");
  if (!c->ev_x) FT_HIP(hipEventCreateWithFlags(&c->ev_x, hipEventDisableTiming), "event creation");
  if (!c->resid_host) {
    void* p = nullptr;
    FT_HIP(hipHostMalloc(&p, static_cast<size_t>(c->E) * 4, hipHostMallocDefault), "pinned host buffer");
    c->resid_host = static_cast<int32_t*>(p);
  }
  const int np = cache_max_passes(c);
  while (static_cast<int>(c->ev_done.size()) < np) {
    hipEvent_t a = nullptr, b = nullptr;
    FT_HIP(hipEventCreateWithFlags(&a, hipEventDisableTiming), "event creation");
    if (hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
      (void)hipEventDestroy(a);
      return fail(FTMOE_ERR_HIP, "event creation failed");
    }
    c->ev_copied.push_back(a);
    c->ev_done.push_back(b);
  }
  c->tptr.assign(np, nullptr);
  return FTMOE_OK;
}

// Plans the step once its routing is on the host.  spec: the first pass
// (the resident experts, on the device residency table) is already
// enqueued, and the misses get passes 1..; else every pass is planned here,
// pass 0 included.  Passes: the hits, then the misses (after the host's
// share is taken out) in one pass when they fit beside the hits, else in
// groups of half the pool; with per-tensor FP8 activations a single pass.
ftmoe_status cache_plan_step(ftmoe_cache* c, bool spec) {
  const ftmoe_layer* L = &c->layer;
  const int E = c->E, k = c->step_k;
  const size_t n_ids = c->n_ids;
  FT_HIP(hipEventSynchronize(c->ev_ids), "routing copy");
  const int32_t* ids_host = c->pin;
  std::vector<int> rows(E, 0);
  for (size_t i = 0; i < n_ids; ++i) ++rows[ids_host[i]];
  std::vector<int> hit, missing;
  for (int e = 0; e < E; ++e)
    if (rows[e]) (resident(c, e) ? hit : missing).push_back(e);
  // co-execution: some missing experts computed on the host instead of filled
  c->h_n = 0;
  const int q = host_split(c, missing, rows);
  if (q > 0) {
    std::vector<char> on_host(E, 0);
    int nr = 0;
    for (int i = 0; i < q; ++i) {
      on_host[missing[i]] = 1;
      nr += rows[missing[i]];
    }
    missing.erase(missing.begin(), missing.begin() + q);
    std::sort(missing.begin(), missing.end());
    if (static_cast<size_t>(nr) > c->h_rows_cap) {
      size_t cap_f = c->h_rows_cap * 4, cap_o = c->h_rows_cap * 4 * static_cast<size_t>(L->hidden);
      void* pf = c->h_flat;
      void* po = c->h_out;
      FT_TRY(grow_pinned(&pf, &cap_f, static_cast<size_t>(nr) * 4));
      c->h_flat = static_cast<int32_t*>(pf);
      FT_TRY(grow_pinned(&po, &cap_o, static_cast<size_t>(nr) * 4 * L->hidden));
      c->h_out = static_cast<float*>(po);
      c->h_rows_cap = nr;
    }
    c->h_tok.clear();
    c->h_ex.clear();
    for (size_t f = 0; f < n_ids; ++f)
      if (on_host[ids_host[f]]) {
        c->h_flat[c->h_n++] = static_cast<int32_t>(f);
        c->h_tok.push_back(static_cast<int32_t>(f / k));
        c->h_ex.push_back(ids_host[f]);
      }
    c->host_experts += q;
    c->host_rows += nr;
  }
  const int n = static_cast<int>(hit.size() + missing.size());
  std::vector<std::vector<int>> groups;
  if (!spec) {
    if (n > c->slots)
      return fail(FTMOE_ERR_UNSUPPORTED, "per-tensor FP8 activations need all %d experts of the step in %d slots",
                  n, c->slots);
    groups.emplace_back(hit);
    groups[0].insert(groups[0].end(), missing.begin(), missing.end());
  } else {
    groups.push_back(hit);
    const int m = static_cast<int>(missing.size());
    const int g = n <= c->slots ? std::max(1, m) : cache_group(c);
    for (int a = 0; a < m; a += g)
      groups.emplace_back(missing.begin() + a, missing.begin() + std::min(m, a + g));
  }
  const int npass = static_cast<int>(groups.size());
  // plan every pass; a pass's copies wait for the last earlier pass reading a slot they overwrite
  c->copy_e.assign(npass, {});
  c->copy_s.assign(npass, {});
  c->copy_after.assign(npass, -1);
  const int first = spec ? 1 : 0;   // passes whose tables go to the workspace
  int32_t* tab_host = c->pin + n_ids;
  std::fill(tab_host, tab_host + static_cast<size_t>(npass - first) * E, -1);
  std::vector<int> reader(c->slots, -1);
  std::vector<int32_t> sl(c->slots), miss(c->slots);
  for (int i = 0; i < npass; ++i) {
    const int m = static_cast<int>(groups[i].size());
    FT_TRY(cache_plan(c, groups[i].data(), m, sl.data(), miss.data(), true));
    for (int qq = 0; qq < m; ++qq) {
      if (i >= first) tab_host[static_cast<size_t>(i - first) * E + groups[i][qq]] = sl[qq];
      if (miss[qq]) {
        c->copy_e[i].push_back(groups[i][qq]);
        c->copy_s[i].push_back(sl[qq]);
        c->copy_after[i] = std::max(c->copy_after[i], reader[sl[qq]]);
      }
    }
    for (int qq = 0; qq < m; ++qq) reader[sl[qq]] = i;
  }
  if (npass > first)
    FT_HIP(hipMemcpyAsync(c->tables_dev, tab_host, static_cast<size_t>(npass - first) * E * 4,
                          hipMemcpyHostToDevice, c->stream),
           "table copy");
  for (int i = first; i < npass; ++i) c->tptr[i] = c->tables_dev + static_cast<size_t>(i - first) * E;
  c->run.n = npass;
  c->passes += npass;
  return FTMOE_OK;
}

// Hooks of the speculative flow: pass 0 (the resident experts) has no
// copies; its hook plans the rest and starts pass 1's copies.
ftmoe_status cache_spec_before(void* ctx, int i) {
  ftmoe_cache* c = static_cast<ftmoe_cache*>(ctx);
  if (i > 0 && !c->copy_e[i].empty()) FT_HIP(hipStreamWaitEvent(c->stream, c->ev_copied[i], 0), "pass wait");
  return FTMOE_OK;
}

ftmoe_status cache_spec_after(void* ctx, int i) {
  ftmoe_cache* c = static_cast<ftmoe_cache*>(ctx);
  FT_HIP(hipEventRecord(c->ev_done[i], c->stream), "pass event");
  if (i == 0) FT_TRY(cache_plan_step(c, true));
  if (i + 1 < c->run.n) FT_TRY(cache_copy_pass(c, i + 1));
  return FTMOE_OK;
}

// Before the combine: the host rows, then the residency table the next
// step's first pass reads (after every pass of this step on the stream).
ftmoe_status cache_spec_combine(void* ctx, void* o, bool fp32) {
  ftmoe_cache* c = static_cast<ftmoe_cache*>(ctx);
  FT_TRY(cache_host_rows(ctx, o, fp32));
  for (int e = 0; e < c->E; ++e) c->resid_host[e] = resident(c, e) ? c->expert_slot[e] : -1;
  FT_HIP(hipMemcpyAsync(c->pool + c->pl.resid, c->resid_host, static_cast<size_t>(c->E) * 4, hipMemcpyHostToDevice,
                        c->stream),
         "residency table copy");
  return FTMOE_OK;
}

// The most passes a step can need (the resident experts, then the misses in
// groups), and the workspace of ftmoe_cache_forward.
int cache_max_passes(const ftmoe_cache* c) { return 1 + (c->E + cache_group(c) - 1) / cache_group(c); }

size_t cache_ws_bytes(const ftmoe_cache* c, const Plan& p) {
  return up256(p.total) + up256(static_cast<size_t>(cache_max_passes(c)) * c->E * 4);
}

}  // namespace

extern "C" {

ftmoe_status ftmoe_workspace_size(const ftmoe_layer* layer, int32_t T, size_t* bytes) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  FT_TRY(check_tokens(T));
  if (!bytes) return fail(FTMOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_plan(layer, T).total;
  return FTMOE_OK;
}

size_t ftmoe_workspace_bytes(const ftmoe_layer* layer, int32_t T) {
  size_t n = 0;
  return ftmoe_workspace_size(layer, T, &n) == FTMOE_OK ? n : 0;
}

int32_t ftmoe_align_max_padded(int32_t T, int32_t k, int32_t E, int32_t block_m) {
  if (T < 0 || T > kMaxTokens || k < 1 || k > kMaxTopK || E < 1 || E > kMaxExperts || block_m < 1 ||
      block_m > 1024)
    return -1;
  return max_padded(T, k, E, block_m);
}

size_t ftmoe_align_workspace_size(int32_t T, int32_t k, int32_t E, int32_t block_m) {
  if (ftmoe_align_max_padded(T, k, E, block_m) < 0) return 0;
  return align_scratch_bytes(T, k, E, block_m);
}

ftmoe_status ftmoe_route(const ftmoe_layer* layer, const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                         int32_t* topk_ids, float* topk_w, float* shared_gate, void* stream) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  FT_TRY(check_tokens(T));
  if (T == 0) return FTMOE_OK;
  if (!x || !topk_ids || !topk_w) return fail(FTMOE_ERR_INVALID_ARG, "x, topk_ids and topk_w must be non-NULL");
  if (!aligned16(x)) return fail(FTMOE_ERR_INVALID_ARG, "x is not 16-byte aligned");
  if (layer->shared_inter > 0 && !shared_gate)
    return fail(FTMOE_ERR_INVALID_ARG, "the layer has a shared expert: shared_gate must be non-NULL");
  const Plan p = make_plan(layer, T);
  FT_TRY(check_ws(p, ws, ws_bytes));
  return enqueue_route(layer, x, T, p, ws, topk_ids, topk_w, shared_gate, false, false,
                       static_cast<hipStream_t>(stream));
}

ftmoe_status ftmoe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m, int32_t* counts,
                         int32_t* offsets, int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                         void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (ftmoe_align_max_padded(T, k, E, block_m) < 0)
    return fail(FTMOE_ERR_INVALID_ARG, "bad sizes T=%d k=%d E=%d block_m=%d", T, k, E, block_m);
  if (T == 0) return FTMOE_OK;
  if (!topk_ids || !counts || !offsets || !sorted_ids || !block_expert || !num_padded)
    return fail(FTMOE_ERR_INVALID_ARG, "align: every array must be non-NULL");
  const size_t need = align_scratch_bytes(T, k, E, block_m);
  if (ws_bytes < need) return fail(FTMOE_ERR_WORKSPACE, "align needs %zu bytes of workspace", need);
  if (need > 0 && (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u)))
    return fail(FTMOE_ERR_WORKSPACE, "align workspace must be non-NULL and 256-byte aligned");
  return hip_status(launch_align(topk_ids, T, k, E, block_m, counts, offsets, sorted_ids, block_expert, num_padded,
                                 ws, nullptr, 0, static_cast<hipStream_t>(stream)),
                    "align launch");
}

ftmoe_status ftmoe_experts_forward(const ftmoe_layer* layer, const uint16_t* x, int32_t T, const int32_t* topk_ids,
                                   const float* topk_w, const float* shared_gate, void* ws, size_t ws_bytes,
                                   uint16_t* y, void* stream) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  FT_TRY(check_tokens(T));
  if (T == 0) return FTMOE_OK;
  if (!x || !topk_ids || !topk_w || !y)
    return fail(FTMOE_ERR_INVALID_ARG, "x, topk_ids, topk_w and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if (layer->shared_inter > 0 && !shared_gate)
    return fail(FTMOE_ERR_INVALID_ARG, "the layer has a shared expert: shared_gate must be non-NULL");
  const Plan p = make_plan(layer, T);
  FT_TRY(check_ws(p, ws, ws_bytes));
  return enqueue_experts(layer, x, T, topk_ids, topk_w, shared_gate, p, ws, y, false, false,
                         static_cast<hipStream_t>(stream));
}

ftmoe_status ftmoe_forward(const ftmoe_layer* layer, const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                           uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  FT_TRY(check_tokens(T));
  if (T == 0) return FTMOE_OK;
  if (!x || !y) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  const Plan p = make_plan(layer, T);
  FT_TRY(check_ws(p, ws, ws_bytes));
  return enqueue_forward(layer, x, T, p, ws, y, topk_ids_out, topk_w_out, static_cast<hipStream_t>(stream));
}

ftmoe_status ftmoe_forward_noalloc(const ftmoe_layer* layer, const uint16_t* x, int32_t T, uint16_t* y,
                                   int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  FT_TRY(check_tokens(T));
  if (T == 0) return FTMOE_OK;
  if (!x || !y) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  const Plan p = make_plan(layer, T);
  if (p.total > kScratchBytes)
    return fail(FTMOE_ERR_WORKSPACE,
                "%d tokens of this layer need %zu bytes of scratch; the allocation-free forward has %zu (call "
                "ftmoe_forward with a workspace instead)",
                T, p.total, kScratchBytes);
  void* ws = nullptr;
  FT_TRY(device_scratch(&ws));
  // no timing events either (they would be created on first use)
  const bool timing = g_timing;
  g_timing = false;
  const ftmoe_status st = enqueue_forward(layer, x, T, p, ws, y, topk_ids_out, topk_w_out,
                                          static_cast<hipStream_t>(stream));
  g_timing = timing;
  return st;
}

ftmoe_status ftmoe_packed_size(const ftmoe_qweight* w, int32_t role, size_t* bytes) {
  g_last_error.clear();
  if (!w || !bytes) return fail(FTMOE_ERR_INVALID_ARG, "w and bytes must be non-NULL");
  if (role != FTMOE_ROLE_GATE_UP && role != FTMOE_ROLE_DOWN)
    return fail(FTMOE_ERR_INVALID_ARG, "role=%d is not an ftmoe_role", role);
  if (w->fmt != FTMOE_W_MXFP4 && w->fmt != FTMOE_W_NVFP4 && w->fmt != FTMOE_W_FP8_E4M3)
    return fail(w->fmt == FTMOE_W_BF16 ? FTMOE_ERR_UNSUPPORTED : FTMOE_ERR_INVALID_ARG,
                "fmt=%d has no packed layout", w->fmt);
  if (w->num_experts < 1 || w->num_experts > kMaxExperts || w->n < 1 || w->k < 128 || w->k % 128 ||
      w->k > kMaxDim || w->n > 2 * kMaxDim || (role == FTMOE_ROLE_GATE_UP && w->n % 256))
    return fail(FTMOE_ERR_UNSUPPORTED, "matrix set [%d][%d][%d] has no packed layout", w->num_experts, w->n, w->k);
  *bytes = packed_bytes(w->fmt, w->num_experts, w->n, w->k, role == FTMOE_ROLE_GATE_UP);
  return FTMOE_OK;
}

ftmoe_status ftmoe_pack_qweight(const ftmoe_qweight* w, int32_t role, void* packed, size_t packed_bytes_,
                                void* stream) {
  size_t need = 0;
  FT_TRY(ftmoe_packed_size(w, role, &need));
  ftmoe_qweight src = *w;
  src.packed = nullptr;   // the source is the row-major matrices
  FT_TRY(check_qweight(src, "w", src.fmt, src.num_experts, src.n, src.k));
  if (!packed || (reinterpret_cast<uintptr_t>(packed) & 255u))
    return fail(FTMOE_ERR_INVALID_ARG, "packed must be non-NULL and 256-byte aligned");
  if (packed_bytes_ < need)
    return fail(FTMOE_ERR_INVALID_ARG, "packed holds %zu bytes, %zu needed", packed_bytes_, need);
  FT_HIP(launch_pack_weights(to_qw(src), src.num_experts, role == FTMOE_ROLE_GATE_UP, static_cast<uint8_t*>(packed),
                             static_cast<hipStream_t>(stream)),
         "pack launch");
  return FTMOE_OK;
}

ftmoe_status ftmoe_quantize_fp8_per_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* scale, void* ws,
                                           size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (n < 0) return fail(FTMOE_ERR_INVALID_ARG, "n=%lld is negative", static_cast<long long>(n));
  if (n == 0) return FTMOE_OK;
  if (!x || !q || !scale) return fail(FTMOE_ERR_INVALID_ARG, "x, q and scale must be non-NULL");
  if (!aligned16(x) || !aligned16(q)) return fail(FTMOE_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
  if (!ws || ws_bytes < 256 || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(FTMOE_ERR_WORKSPACE, "quantiser needs 256 bytes of 256-byte aligned workspace");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  FT_HIP(launch_zero_u32(amax, 1, s), "zero launch");
  FT_HIP(launch_amax_bf16(x, n, amax, s), "amax launch");
  FT_HIP(launch_quant_fp8(x, n, amax, q, scale, s), "quantise launch");
  return FTMOE_OK;
}

void ftmoe_timing_enable(int32_t on) { g_timing = on != 0; }

int32_t ftmoe_timing_collect(int32_t max_entries, char* names, double* total_ms, int64_t* counts) {
  std::vector<std::string> keys;
  std::vector<double> ms;
  std::vector<int64_t> cnt;
  for (const TimedLaunch& t : g_pending) {
    float m = 0.f;
    hipEventSynchronize(t.b);
    if (hipEventElapsedTime(&m, t.a, t.b) != hipSuccess) m = 0.f;
    size_t i = 0;
    while (i < keys.size() && keys[i] != t.name) ++i;
    if (i == keys.size()) {
      keys.emplace_back(t.name);
      ms.push_back(0.0);
      cnt.push_back(0);
    }
    ms[i] += m;
    cnt[i] += 1;
    hipEventSynchronize(t.d);
    g_event_pool.push_back(t.a);
    g_event_pool.push_back(t.b);
    g_event_pool.push_back(t.c);
    g_event_pool.push_back(t.d);
  }
  g_pending.clear();
  const int32_t n = static_cast<int32_t>(keys.size());
  for (int32_t i = 0; i < n && i < max_entries; ++i) {
    if (names) {
      strncpy(names + 32 * i, keys[i].c_str(), 31);
      names[32 * i + 31] = 0;
    }
    if (total_ms) total_ms[i] = ms[i];
    if (counts) counts[i] = cnt[i];
  }
  return n;
}

const char* ftmoe_status_string(ftmoe_status st) {
  switch (st) {
    case FTMOE_OK: return "FTMOE_OK";
    case FTMOE_ERR_INVALID_ARG: return "FTMOE_ERR_INVALID_ARG";
    case FTMOE_ERR_UNSUPPORTED: return "FTMOE_ERR_UNSUPPORTED";
    case FTMOE_ERR_WORKSPACE: return "FTMOE_ERR_WORKSPACE";
    case FTMOE_ERR_HIP: return "FTMOE_ERR_HIP";
  }
  return "FTMOE_UNKNOWN_STATUS";
}

const char* ftmoe_last_error(void) { return g_last_error.c_str(); }

int32_t ftmoe_version(void) { return 100; }

ftmoe_status ftmoe_cache_pool_size(const ftmoe_layer* layer, int32_t slots, size_t* bytes) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  if (slots < 1 || slots > layer->num_experts)
    return fail(FTMOE_ERR_INVALID_ARG, "slots=%d outside [1, num_experts=%d]", slots, layer->num_experts);
  if (!bytes) return fail(FTMOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = pool_layout(layer->gate_up, layer->down, slots, layer->num_experts).total;
  return FTMOE_OK;
}

ftmoe_status ftmoe_cache_create(const ftmoe_layer* layer, const ftmoe_qweight* host_gate_up,
                                const ftmoe_qweight* host_down, int32_t slots, void* pool, size_t pool_bytes,
                                ftmoe_cache** cache) {
  g_last_error.clear();
  if (!cache || !host_gate_up || !host_down) return fail(FTMOE_ERR_INVALID_ARG, "NULL argument");
  *cache = nullptr;
  FT_TRY(check_layer(layer));
  const int E = layer->num_experts;
  if (slots < 1 || slots > E) return fail(FTMOE_ERR_INVALID_ARG, "slots=%d outside [1, num_experts=%d]", slots, E);
  const int fmt = layer->gate_up.fmt;
  FT_TRY(check_qweight(*host_gate_up, "host_gate_up", fmt, E, 2 * layer->inter, layer->hidden));
  FT_TRY(check_qweight(*host_down, "host_down", fmt, E, layer->hidden, layer->inter));
  if (host_gate_up->packed || host_down->packed)
    return fail(FTMOE_ERR_INVALID_ARG, "host experts have no packed layout");
  const PoolLayout pl = pool_layout(*host_gate_up, *host_down, slots, E);
  if (!pool || (reinterpret_cast<uintptr_t>(pool) & 255u))
    return fail(FTMOE_ERR_INVALID_ARG, "pool must be non-NULL and 256-byte aligned");
  if (pool_bytes < pl.total)
    return fail(FTMOE_ERR_INVALID_ARG, "pool holds %zu bytes, %zu needed", pool_bytes, pl.total);
  ftmoe_cache* c = new (std::nothrow) ftmoe_cache;
  if (!c) return fail(FTMOE_ERR_INVALID_ARG, "out of host memory");
  c->layer = *layer;
  c->host_gu = *host_gate_up;
  c->host_dn = *host_down;
  c->slots = slots;
  c->E = E;
  c->pl = pl;
  c->pool = static_cast<uint8_t*>(pool);
  auto pooled = [&](const ftmoe_qweight& h, size_t codes, size_t scales, size_t ts) {
    ftmoe_qweight q = h;
    q.codes = c->pool + codes;
    q.block_scales = h.block_scales ? c->pool + scales : nullptr;
    q.tensor_scales = h.tensor_scales ? reinterpret_cast<const float*>(c->pool + ts) : nullptr;
    q.packed = nullptr;
    return q;
  };
  c->layer.gate_up = pooled(*host_gate_up, pl.gu_codes, pl.gu_scales, pl.gu_ts);
  c->layer.down = pooled(*host_down, pl.dn_codes, pl.dn_scales, pl.dn_ts);
  c->slot_expert.assign(slots, -1);
  c->expert_slot.assign(E, -1);
  c->last_use.assign(slots, -1);
  c->filled.assign(slots, 0);
  *cache = c;
  return FTMOE_OK;
}

void ftmoe_cache_destroy(ftmoe_cache* cache) { delete cache; }

ftmoe_status ftmoe_cache_plan(ftmoe_cache* cache, const int32_t* experts, int32_t n, int32_t* out_slot,
                              int32_t* out_miss) {
  g_last_error.clear();
  if (!cache || (n > 0 && !experts) || n < 0) return fail(FTMOE_ERR_INVALID_ARG, "bad arguments");
  FT_TRY(cache_plan(cache, experts, n, out_slot, out_miss, false));
  // evicted experts are gone from their slots: the device residency table
  // the next forward's first pass reads is rewritten from the host state
  cache->resid_init = false;
  return FTMOE_OK;
}

ftmoe_status ftmoe_cache_workspace_size(const ftmoe_cache* cache, int32_t T, size_t* bytes) {
  g_last_error.clear();
  if (!cache || !bytes) return fail(FTMOE_ERR_INVALID_ARG, "NULL argument");
  FT_TRY(check_tokens(T));
  *bytes = cache_ws_bytes(cache, make_plan(&cache->layer, T));
  return FTMOE_OK;
}

static ftmoe_status cache_forward_impl(ftmoe_cache* c, const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                                       uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* stream);

ftmoe_status ftmoe_cache_forward(ftmoe_cache* c, const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                                 uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  g_last_error.clear();
  if (!c) return fail(FTMOE_ERR_INVALID_ARG, "cache is NULL");
  const ftmoe_status st = cache_forward_impl(c, x, T, ws, ws_bytes, y, topk_ids_out, topk_w_out, stream);
  if (st == FTMOE_ERR_HIP) {
    // a runtime failure after planning may leave slots marked resident whose fills never ran: forget them all
    // (finishing what was enqueued first, so that no fill lands in a slot after it is reassigned)
    if (c->copy_stream) (void)hipStreamSynchronize(c->copy_stream);
    if (c->x_stream) (void)hipStreamSynchronize(c->x_stream);
    if (c->called) (void)hipStreamSynchronize(c->stream);
    std::fill(c->slot_expert.begin(), c->slot_expert.end(), -1);
    std::fill(c->expert_slot.begin(), c->expert_slot.end(), -1);
    std::fill(c->last_use.begin(), c->last_use.end(), -1);
    std::fill(c->filled.begin(), c->filled.end(), 0);
    c->resid_init = false;   // the device residency table is rewritten on the next call
  }
  return st;
}

static ftmoe_status cache_forward_impl(ftmoe_cache* c, const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                                       uint16_t* y, int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  const ftmoe_layer* L = &c->layer;
  FT_TRY(check_tokens(T));
  if (T == 0) return FTMOE_OK;
  if (!x || !y) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(FTMOE_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  const Plan p = make_plan(L, T);
  const size_t need = cache_ws_bytes(c, p);
  if (ws_bytes < need)
    return fail(FTMOE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, need);
  FT_TRY(check_ws(p, ws, ws_bytes));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the previous call's passes, on another stream, may still read the pool
  if (c->called && c->stream != s) FT_HIP(hipStreamSynchronize(c->stream), "previous stream");
  const int E = c->E, k = L->top_k;
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, p.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, p.w);
  float* sg = at<float>(ws, p.sg);
  const bool fused_align = p.decode && p.small_route;
  const bool gemm_x = !p.small_route && (p.mx_gemm || p.mx_gemm_shared);
  FT_TRY(enqueue_route(L, x, T, p, ws, ids, w, sg, fused_align, gemm_x, s));

  // host resources (made once), the routing ids on their way to the host
  const size_t n_ids = static_cast<size_t>(T) * k;
  FT_TRY(cache_host_buffer(c, n_ids + static_cast<size_t>(cache_max_passes(c)) * E));
  FT_TRY(cache_host_resources(c));
  c->stream = s;
  c->called = true;
  c->n_ids = n_ids;
  c->step_k = k;
  c->step_T = T;
  c->tables_dev = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + up256(p.total));
  FT_HIP(hipMemcpyAsync(c->pin, ids, n_ids * 4, hipMemcpyDeviceToHost, s), "routing copy");
  FT_HIP(hipEventRecord(c->ev_ids, s), "routing copy event");
  c->h_n = 0;
  c->run = Passes{};
  c->run.ctx = c;
  if (L->act == FTMOE_ACT_FP8_PER_TENSOR) {
    // one pass of every expert of the step (the h scale spans them all), planned before it runs
    FT_TRY(cache_plan_step(c, false));
    c->run.before = cache_before_pass;
    c->run.after = cache_after_pass;
  } else {
    // The first pass runs at once on the residency table of the last step:
    // the step's resident experts run while the routing reaches the host;
    // its hook then plans the misses (more passes) and the host rows.
    if (c->host_pool) {
      // x for the host rows, on a stream of its own: neither the first pass
      // nor the pool fills (on the copy stream) queue behind it
      const size_t xb = static_cast<size_t>(T) * L->hidden * 2;
      // the last call's x copy may still be writing the buffer that grows
      if (c->hx && xb > c->hx_bytes) FT_HIP(hipStreamSynchronize(c->x_stream), "x stream");
      FT_TRY(grow_pinned(&c->hx, &c->hx_bytes, xb));
      FT_HIP(hipStreamWaitEvent(c->x_stream, c->ev_ids, 0), "x stream wait");
      FT_HIP(hipMemcpyAsync(c->hx, x, static_cast<size_t>(T) * L->hidden * 2, hipMemcpyDeviceToHost, c->x_stream),
             "x copy");
      FT_HIP(hipEventRecord(c->ev_x, c->x_stream), "x copy event");
    }
    int32_t* resid = reinterpret_cast<int32_t*>(c->pool + c->pl.resid);
    if (!c->resid_init) {
      for (int e = 0; e < E; ++e) c->resid_host[e] = resident(c, e) ? c->expert_slot[e] : -1;
      FT_HIP(hipMemcpyAsync(resid, c->resid_host, static_cast<size_t>(E) * 4, hipMemcpyHostToDevice, s),
             "residency table copy");
      c->resid_init = true;
    }
    c->tptr[0] = resid;
    c->copy_e.assign(1, {});
    c->copy_s.assign(1, {});
    c->copy_after.assign(1, -1);
    c->run.n = 1;
    c->run.before = cache_spec_before;
    c->run.after = cache_spec_after;
    c->run.before_combine = cache_spec_combine;
  }
  c->run.tables = c->tptr.data();
  return enqueue_experts(L, x, T, ids, w, sg, p, ws, y, fused_align, gemm_x, s, c->run);
}

ftmoe_status ftmoe_cache_set_host_compute(ftmoe_cache* c, int32_t threads, double expert_s, double row_s,
                                          double link_bytes_per_s) {
  g_last_error.clear();
  if (!c) return fail(FTMOE_ERR_INVALID_ARG, "cache is NULL");
  if (threads < 0 || threads > 256) return fail(FTMOE_ERR_INVALID_ARG, "threads=%d outside [0, 256]", threads);
  if (threads == 0) {
    c->host_pool.reset();
    return FTMOE_OK;
  }
  if (c->layer.act == FTMOE_ACT_FP8_PER_TENSOR)
    return fail(FTMOE_ERR_UNSUPPORTED, "per-tensor FP8 activations span every expert: no host compute");
  if (!ftmoe_host::cpu_supported()) return fail(FTMOE_ERR_UNSUPPORTED, "host expert compute needs AVX2 and FMA");
  c->host_pool = std::make_unique<ftmoe_host::Pool>(threads);
  c->link_bps = link_bytes_per_s > 0 ? link_bytes_per_s : 50e9;
  c->host_scale = 1;
  c->host_adaptive = !(expert_s > 0 && row_s >= 0);
  if (!c->host_adaptive) {
    c->host_expert_s = expert_s;
    c->host_row_s = row_s;
    return FTMOE_OK;
  }
  // calibration: expert 0 with 1 and with 65 rows of a constant token, best of two each (many rows
  // make the dot products, not the weight decoding, the bound)
  const int H = c->layer.hidden;
  const ftmoe_host::Mat gu = host_mat(c->host_gu), dn = host_mat(c->host_dn);
  std::vector<uint16_t> x(H, 0x3C00);   // bf16 0.0078125
  constexpr int kRows = 65;
  std::vector<int32_t> tok(kRows, 0), ex(kRows, 0);
  std::vector<float> o(static_cast<size_t>(kRows) * H);
  double t[2] = {1e30, 1e30};
  for (int rep = 0; rep < 2; ++rep)
    for (int v = 0; v < 2; ++v) {
      const auto t0 = std::chrono::steady_clock::now();
      ftmoe_host::expert_rows(*c->host_pool, gu, dn, H, c->layer.inter, c->layer.act == FTMOE_ACT_MXFP8, x.data(),
                              tok.data(), ex.data(), v ? kRows : 1, o.data());
      t[v] = std::min(t[v], std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count());
    }
  c->host_row_s = std::max(0.0, (t[1] - t[0]) / (kRows - 1));
  c->host_expert_s = std::max(1e-7, t[0] - c->host_row_s);
  return FTMOE_OK;
}

ftmoe_status ftmoe_cache_host_stats(const ftmoe_cache* c, int64_t* experts, int64_t* rows, double* seconds,
                                    double* expert_s, double* row_s) {
  g_last_error.clear();
  if (!c) return fail(FTMOE_ERR_INVALID_ARG, "cache is NULL");
  if (experts) *experts = c->host_experts;
  if (rows) *rows = c->host_rows;
  if (seconds) *seconds = c->host_seconds;
  if (expert_s) *expert_s = c->host_expert_s * c->host_scale;
  if (row_s) *row_s = c->host_row_s * c->host_scale;
  return FTMOE_OK;
}

ftmoe_status ftmoe_host_expert_rows(const ftmoe_layer* layer, const uint16_t* x, const int32_t* tok,
                                    const int32_t* ex, int32_t n, float* o, int32_t threads) {
  g_last_error.clear();
  FT_TRY(check_layer(layer));
  if (n < 0 || threads < 1 || threads > 256) return fail(FTMOE_ERR_INVALID_ARG, "bad n or threads");
  if (n > 0 && (!x || !tok || !ex || !o)) return fail(FTMOE_ERR_INVALID_ARG, "NULL argument");
  if (layer->act == FTMOE_ACT_FP8_PER_TENSOR)
    return fail(FTMOE_ERR_UNSUPPORTED, "per-tensor FP8 activations span every expert: no host compute");
  for (int i = 0; i < n; ++i)
    if (ex[i] < 0 || ex[i] >= layer->num_experts || tok[i] < 0)
      return fail(FTMOE_ERR_INVALID_ARG, "row %d: expert %d or token %d out of range", i, ex[i], tok[i]);
  const ftmoe_host::Mat gu = host_mat(layer->gate_up), dn = host_mat(layer->down);
  ftmoe_host::Pool pool(threads);
  if (!ftmoe_host::expert_rows(pool, gu, dn, layer->hidden, layer->inter, layer->act == FTMOE_ACT_MXFP8, x, tok, ex,
                               n, o))
    return fail(FTMOE_ERR_UNSUPPORTED, "host expert compute needs AVX2 and FMA");
  return FTMOE_OK;
}

ftmoe_status ftmoe_cache_stats(const ftmoe_cache* cache, int64_t* hits, int64_t* misses, int64_t* bytes_copied,
                               int64_t* passes) {
  g_last_error.clear();
  if (!cache) return fail(FTMOE_ERR_INVALID_ARG, "cache is NULL");
  if (hits) *hits = cache->hits;
  if (misses) *misses = cache->misses;
  if (bytes_copied) *bytes_copied = cache->bytes;
  if (passes) *passes = cache->passes;
  return FTMOE_OK;
}

}  // extern "C"
