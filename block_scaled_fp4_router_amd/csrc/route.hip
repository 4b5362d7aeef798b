// Router: logits l[t,e] = x_t . W_r[e] (fp32 accumulation of exact bf16 x
// and fp32 W_r), then per-token softmax top-k with renormalised weights and
// the shared expert's sigmoid gate.
#include "align_dev.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace ftmoe {

// ---------------------------------------------------------------- GEMV ----
// Few tokens: one wave per router row (row E is the shared-gate vector).
// Each lane walks H in float4 steps and keeps one partial per token.
constexpr int kGemvMaxT = 16;

template <int TMAX>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                          const float* __restrict__ router_w, int E,
                                                          const float* __restrict__ shared_gate_w,
                                                          float* __restrict__ logits) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = E + (shared_gate_w ? 1 : 0);
  if (row >= rows) return;
  const float* wrow = row < E ? router_w + static_cast<size_t>(row) * H : shared_gate_w;
  const int lane = lane_id();
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.f;
  for (int h = lane * 4; h < H; h += kWave * 4) {
    const float4 w = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + static_cast<size_t>(t) * H + h);
        acc[t] = fmaf(bf16_to_f32(xv.x & 0xFFFF), w.x, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv.x >> 16), w.y, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv.y & 0xFFFF), w.z, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv.y >> 16), w.w, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) logits[static_cast<size_t>(t) * (E + 1) + row] = v;
    }
  }
}

// ---------------------------------------------------------------- GEMM ----
// Many tokens: bf16 MFMA with the fp32 router weights split exactly into
// three bf16 terms, w = w1 + w2 + w3 (w1 = bf16(w), w2 = bf16(w - w1),
// w3 = w - w1 - w2, which fits bf16 because each rounding leaves at most 8
// significant bits fewer).  Each product x * w_i of a bf16 x is exact in
// fp32 and the MFMA accumulates in fp32, so the logits keep fp32 accuracy.
// The split is made once per call into three bf16 planes [3][rows][H] (every
// token tile of the GEMM would otherwise convert the same weights again).
// Workgroup: RT tokens x 64 router rows, 4 waves of RT / 2 tokens x 32 rows
// each (RT = 128: two 32 x 32 tiles per wave sharing the weight fragments,
// so every weight fragment read from LDS feeds two MFMAs; RT = 64, for token
// counts that would leave CUs idle, one); K stages of 64 staged through LDS
// (rows of 128 bytes, XOR-swizzled).  The global loads of the next stage are
// issued before the current stage's MFMA work, and several workgroups share
// each CU, so their latency is covered.
constexpr int kRE = 64, kRK = 64, kRThreads = 256;

// Token tile of the router GEMM for T tokens and `rows` router rows: 128
// when that still gives 256 tiles, else 64.
int router_token_tile(int T, int rows) {
  const long long t128 = static_cast<long long>((T + 127) / 128) * ((rows + kRE - 1) / kRE);
  return t128 >= 256 ? 128 : 64;
}

__device__ __forceinline__ int rswz(int r, int q) { return q ^ ((r & 7) ^ ((r >> 3) & 1)); }

__device__ __forceinline__ void split3(float w, uint16_t& a, uint16_t& b, uint16_t& c) {
  a = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(a);
  b = f32_to_bf16(r1);
  c = f32_to_bf16(r1 - bf16_to_f32(b));
}

// planes[m][r][h], m = 0, 1, 2: the three terms of row r (r = E: the shared
// gate vector); one thread per 8 consecutive elements.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ router_w, int E, int H,
                                                           const float* __restrict__ shared_gate_w,
                                                           uint16_t* __restrict__ planes) {
  const int rows = E + (shared_gate_w ? 1 : 0);
  const size_t n8 = static_cast<size_t>(rows) * H / 8;
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const size_t el = 8 * i;
  const int r = static_cast<int>(el / H), h = static_cast<int>(el % H);
  const float* src = (r < E ? router_w + static_cast<size_t>(r) * H : shared_gate_w) + h;
  const float4 v0 = *reinterpret_cast<const float4*>(src);
  const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
  const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t p[3][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint16_t a0, b0, c0, a1, b1, c1;
    split3(f[2 * q], a0, b0, c0);
    split3(f[2 * q + 1], a1, b1, c1);
    p[0][q] = a0 | (static_cast<uint32_t>(a1) << 16);
    p[1][q] = b0 | (static_cast<uint32_t>(b1) << 16);
    p[2][q] = c0 | (static_cast<uint32_t>(c1) << 16);
  }
  const size_t plane = static_cast<size_t>(rows) * H;
#pragma unroll
  for (int m = 0; m < 3; ++m)
    *reinterpret_cast<uint4*>(planes + m * plane + el) = make_uint4(p[m][0], p[m][1], p[m][2], p[m][3]);
}

// With XOUT (MXFP4 experts) the workgroups of the first router-row tile also
// write x in the form the expert GEMMs read, from the x stages they load
// anyway: split E4M3 pairs ([T][2H], per 64 elements 64 hi then 64 lo codes)
// or, with a8, MXFP8 codes ([T][H]), and the E8M0 scales [T][H / 32].  A
// thread stages one 32-block of x per stage (RT = 128) or half of one, the
// other half being in lane ^ 1 (RT = 64).
template <int RT, bool XOUT>
__global__ __launch_bounds__(kRThreads) void router_gemm_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                                const uint16_t* __restrict__ planes, int E,
                                                                int rows, float* __restrict__ logits,
                                                                uint8_t* __restrict__ xout, uint8_t* __restrict__ xsc_out,
                                                                int a8) {
  // blockIdx.z: the K split; split z sums H range [z, z + 1) * H / gridDim.z into logits[z]
  constexpr int MW = RT / 64;    // 32-token tiles per wave
  constexpr int XV = RT / 32;    // x vectors a thread stages per stage
  __shared__ __attribute__((aligned(16))) uint8_t xs[RT * 128];
  __shared__ __attribute__((aligned(16))) uint8_t ws[3][kRE * 128];
  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * kRE;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int wt = (wave & 1) * 32 * MW, we = (wave >> 1) * 32;
  const int j = lane & 31, g = lane >> 5;

  // staging: x row tid / (8 / XV), vectors XV (tid % (8 / XV)) .. + XV - 1;
  // W row tid / 4, vectors 2 (tid % 4) and + 1 of each of the three planes
  const int xr = tid / (8 / XV), xq = (tid % (8 / XV)) * XV;
  const int wr = tid >> 2, wq = (tid & 3) * 2;
  const int t = t0 + xr, e = e0 + wr;
  const uint16_t* xrow = t < T ? x + static_cast<size_t>(t) * H : nullptr;
  const size_t plane = static_cast<size_t>(rows) * H;
  const uint16_t* wrow = e < rows ? planes + static_cast<size_t>(e) * H : nullptr;

  struct Stage {
    uint4 x[XV];
    uint4 w[3][2];
  };
  Stage st;
  auto load = [&](Stage& sg, int k0) {
#pragma unroll
    for (int h = 0; h < XV; ++h)
      sg.x[h] = xrow ? *reinterpret_cast<const uint4*>(xrow + k0 + (xq + h) * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        sg.w[m][h] = wrow ? *reinterpret_cast<const uint4*>(wrow + m * plane + k0 + (wq + h) * 8)
                          : make_uint4(0, 0, 0, 0);
  };
  auto store = [&](const Stage& sg) {
#pragma unroll
    for (int h = 0; h < XV; ++h) *reinterpret_cast<uint4*>(xs + xr * 128 + 16 * rswz(xr, xq + h)) = sg.x[h];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int off = wr * 128 + 16 * rswz(wr, wq + h);
#pragma unroll
      for (int m = 0; m < 3; ++m) *reinterpret_cast<uint4*>(ws[m] + off) = sg.w[m][h];
    }
  };

  const bool split_x = XOUT && blockIdx.y == 0;   // uniform per workgroup
  auto split_stage = [&](const Stage& sg, int k0) {
    const int e0 = k0 + 8 * xq;   // the thread's elements start here; its 32-block is e0 / 32
    if constexpr (XV == 4) {
      if (!xrow) return;
      uint8_t* sc = xsc_out + static_cast<size_t>(t) * (H / 32) + e0 / 32;
      if (a8) {
        mxfp8_block(sg.x, xout + static_cast<size_t>(t) * H + e0, sc);
      } else {
        uint8_t* hi = xout + static_cast<size_t>(t) * (2 * H) + (e0 / 64) * 128 + (e0 % 64);
        mx_split_block(sg.x, hi, hi + 64, sc);
      }
    } else {   // half a block: the block maximum from lane ^ 1 (every lane joins)
      float m = bf16_amax(sg.x);
      m = __builtin_fmaxf(m, __shfl_xor(m, 1, kWave));
      if (!xrow) return;
      uint32_t code;
      if (a8) {
        uint4 q;
        code = mxfp8_half(sg.x, m, q);
        *reinterpret_cast<uint4*>(xout + static_cast<size_t>(t) * H + e0) = q;
      } else {
        uint4 hi, lo;
        code = mx_split_half(sg.x, m, hi, lo);
        uint8_t* dst = xout + static_cast<size_t>(t) * (2 * H) + (e0 / 64) * 128 + (e0 % 64);
        *reinterpret_cast<uint4*>(dst) = hi;
        *reinterpret_cast<uint4*>(dst + 64) = lo;
      }
      if ((xq & 2) == 0) xsc_out[static_cast<size_t>(t) * (H / 32) + e0 / 32] = static_cast<uint8_t>(code);
    }
  };

  f32x16 acc[MW] = {};
  const int kspan = H / static_cast<int>(gridDim.z), kbeg = static_cast<int>(blockIdx.z) * kspan;
  const int ns = kspan / kRK;
  logits += static_cast<size_t>(blockIdx.z) * T * (E + 1);
  if (ns > 0) load(st, kbeg);
  for (int s = 0; s < ns; ++s) {
    __syncthreads();   // the previous stage's reads are done
    store(st);
    if constexpr (XOUT)
      if (split_x) split_stage(st, kbeg + s * kRK);
    __syncthreads();
    if (s + 1 < ns) load(st, kbeg + (s + 1) * kRK);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int q = 2 * ks + g;   // 8 bf16 of K group g of step ks
      const int rb = we + j;
      bf16x8 a[MW];
#pragma unroll
      for (int m = 0; m < MW; ++m) {
        const int ra = wt + 32 * m + j;
        a[m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xs + ra * 128 + 16 * rswz(ra, q)));
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 b =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ws[p] + rb * 128 + 16 * rswz(rb, q)));
#pragma unroll
        for (int m = 0; m < MW; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b, acc[m], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MW; ++m) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = t0 + wt + 32 * m + 8 * (r >> 2) + 4 * g + (r & 3);
      const int ee = e0 + we + j;
      if (tt < T && ee < rows) logits[static_cast<size_t>(tt) * (E + 1) + ee] = acc[m][r];
    }
  }
}

// K splits of the router GEMM: enough workgroups for about four per compute
// unit (the top-k kernel adds the splits in order, so the logits stay
// deterministic).
int router_splits_gemm(int T, int H, int rows) {
  if (T <= kGemvMaxT) return 1;
  const int rt = router_token_tile(T, rows);
  const long long tiles = static_cast<long long>((T + rt - 1) / rt) * ((rows + kRE - 1) / kRE);
  int S = 1;
  while (S < 4 && tiles * S < 1024 && (H / kRK) % (2 * S) == 0) S *= 2;
  return S;
}

size_t router_planes_bytes(int E, int H, bool shared) {
  return 3 * static_cast<size_t>(E + (shared ? 1 : 0)) * H * sizeof(uint16_t);
}

hipError_t launch_router_split(const float* router_w, int E, int H, const float* shared_gate_w, uint16_t* planes,
                               hipStream_t s) {
  const size_t n8 = static_cast<size_t>(E + (shared_gate_w ? 1 : 0)) * H / 8;
  return launch(router_split_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, s, router_w, E, H,
                shared_gate_w, planes);
}

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* router_w, int E,
                                const float* shared_gate_w, const uint16_t* planes, float* logits, uint8_t* xs,
                                uint8_t* xssc, bool a8, hipStream_t s) {
  const int rows = E + (shared_gate_w ? 1 : 0);
  if (T <= kGemvMaxT) {
    dim3 grid((rows + 3) / 4);
    if (T <= 1)
      return launch(router_gemv_kernel<1>, grid, dim3(256), 0, s, x, T, H, router_w, E, shared_gate_w, logits);
    else if (T <= 4)
      return launch(router_gemv_kernel<4>, grid, dim3(256), 0, s, x, T, H, router_w, E, shared_gate_w, logits);
    else
      return launch(router_gemv_kernel<kGemvMaxT>, grid, dim3(256), 0, s, x, T, H, router_w, E, shared_gate_w, logits);
  } else {
    if (!planes) return hipErrorInvalidValue;
    const int rt = router_token_tile(T, rows);
    const dim3 grid((T + rt - 1) / rt, (rows + kRE - 1) / kRE, router_splits_gemm(T, H, rows));
    auto go = [&]<int RT>() {
      if (xs)
        return launch(router_gemm_kernel<RT, true>, grid, dim3(kRThreads), 0, s, x, T, H, planes, E, rows, logits,
                      xs, xssc, a8 ? 1 : 0);
      return launch(router_gemm_kernel<RT, false>, grid, dim3(kRThreads), 0, s, x, T, H, planes, E, rows, logits, xs,
                    xssc, 0);
    };
    return rt == 128 ? go.template operator()<128>() : go.template operator()<64>();
  }
}

// ---------------------------------------------------------------- top-k ---
// One wave per token.  Lane l holds the logits of experts l, l+64, ... (SLOTS
// of them) and sorts them once, descending (equal values: lower expert
// first).  Each of the k rounds is then a wave argmax over the lanes' heads
// (DPP reductions; equal values go to the lower expert index) after which the
// winning lane drops its head.  Weights: softmax over the k selected logits.
constexpr int kTopkMaxPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// v[i] holds the logit of expert lane + 64 i (-inf past E).  On return lane
// j < k holds the j-th selected expert and its renormalised weight.
template <int SLOTS>
__device__ __forceinline__ void wave_topk_softmax(float (&v)[SLOTS], int k, int* sel_id, float* sel_w) {
  const int lane = lane_id();
  int id[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) id[i] = lane + i * kWave;
  // odd-even transposition sort, descending
#pragma unroll
  for (int pass = 0; pass < SLOTS; ++pass) {
#pragma unroll
    for (int i = pass & 1; i + 1 < SLOTS; i += 2) {
      if (better(v[i + 1], id[i + 1], v[i], id[i])) {
        const float tv = v[i];
        v[i] = v[i + 1];
        v[i + 1] = tv;
        const int ti = id[i];
        id[i] = id[i + 1];
        id[i + 1] = ti;
      }
    }
  }
  float sel_v = 0.f;
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv;
    int bi;
    wave_argmax(v[0], id[0], &bv, &bi);
    if (lane == j) {
      sel_v = bv;
      sel_i = bi;
    }
    if ((bi & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i + 1 < SLOTS; ++i) {
        v[i] = v[i + 1];
        id[i] = id[i + 1];
      }
      v[SLOTS - 1] = -__builtin_inff();
    }
  }
  const float m = readlane_f(sel_v, 0);
  const float ex = lane < k ? expf(sel_v - m) : 0.f;
  const float sum = wave_sum_fixed(ex);
  *sel_id = sel_i;
  *sel_w = ex / sum;
}

// Softmax over lanes < k of `l` (a selection-only bias: the selected
// experts' logits without the bias), in a wave.
__device__ __forceinline__ float lanes_softmax(float l, int k) {
  const float m = wave_max_fast(lane_id() < k ? l : -__builtin_inff());
  const float ex = lane_id() < k ? expf(l - m) : 0.f;
  return ex / wave_sum_fixed(ex);
}

template <int SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int nsplit, int T, int E, int k,
                                                   const float* __restrict__ bias, int bias_select, int has_shared,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   float* __restrict__ sgate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const float* row = logits + static_cast<size_t>(t) * (E + 1);
  const size_t split = static_cast<size_t>(T) * (E + 1);
  auto logit = [&](int e) {   // the K splits added in order
    float l = row[e];
    for (int z = 1; z < nsplit; ++z) l += row[z * split + e];
    return l;
  };
  float v[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + i * kWave;
    v[i] = -__builtin_inff();
    if (e < E) v[i] = logit(e) + (bias ? bias[e] : 0.f);
  }
  int sel_i;
  float sel_w;
  wave_topk_softmax<SLOTS>(v, k, &sel_i, &sel_w);
  if (bias && bias_select) sel_w = lanes_softmax(lane < k ? logit(sel_i) : 0.f, k);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = sel_i;
    w[static_cast<size_t>(t) * k + lane] = sel_w;
  }
  if (has_shared && lane == 0) {
    const float g = logit(E);
    sgate[t] = 1.0f / (1.0f + expf(-g));
  }
}

// Calls f.template operator()<SLOTS>() with the smallest SLOTS covering E.
template <class F>
static hipError_t with_slots(int E, F&& f) {
  if (E <= 64) return f.template operator()<1>();
  if (E <= 128) return f.template operator()<2>();
  if (E <= 256) return f.template operator()<4>();
  if (E <= 512) return f.template operator()<8>();
  return f.template operator()<16>();
}

hipError_t launch_topk(const float* logits, int nsplit, int T, int E, int k, const float* bias, bool bias_select,
                       bool has_shared, int32_t* ids, float* w, float* sgate, hipStream_t s) {
  dim3 grid((T + 3) / 4);
  return with_slots(E, [&]<int SL>() {
    return launch(topk_kernel<SL>, grid, dim3(256), 0, s, logits, nsplit, T, E, k, bias, bias_select ? 1 : 0,
                  has_shared ? 1 : 0, ids, w, sgate);
  });
}

// ======================================================= decode router ====
// Few tokens (T <= 16).  The router matrix (E x H fp32, 1-4 MiB) is read by
// many workgroups at once: workgroup (r, s) reads rows 4r..4r+3 over the
// H-slice [256 s, 256 s + 256) -- at most one 16-byte load per lane -- and
// writes partial logits part[t][row][s] (S is rounded up to a multiple of 4;
// slices past H contribute zero).  The fused top-k kernel adds the S slices
// in order, so the logits do not depend on scheduling.  The workgroups of
// row block 0 also write the split E4M3 form of their x slice when asked.
int router_splits(int H) {
  const int s = (H + 255) / 256;
  return (s + 3) / 4 * 4;
}

__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t* __restrict__ x, int T, int H, int S,
                                                             const float* __restrict__ router_w, int E,
                                                             const float* __restrict__ shared_gate_w,
                                                             float* __restrict__ part, uint8_t* __restrict__ xhi,
                                                             uint8_t* __restrict__ xlo, uint8_t* __restrict__ xsc,
                                                             int xsc_pitch) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kDecodeMaxT][256];
  const int rows = E + (shared_gate_w ? 1 : 0);
  const int s = blockIdx.y;
  const int h0 = s * 256;
  const int L = H - h0 < 0 ? 0 : (H - h0 > 256 ? 256 : H - h0);  // a multiple of 128
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
  const bool have_row = row < rows;
  if (have_row && lane * 4 < L) {
    const float* wrow = row < E ? router_w + static_cast<size_t>(row) * H : shared_gate_w;
    wv = *reinterpret_cast<const float4*>(wrow + h0 + lane * 4);
  }
  // Stage the x slice of every token (T x L bf16) in 16-byte pieces.
  for (int i = threadIdx.x; i < T * (L / 8); i += blockDim.x) {
    const int t = i / (L / 8), c = (i % (L / 8)) * 8;
    *reinterpret_cast<uint4*>(&xs[t][c]) = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * H + h0 + c);
  }
  __syncthreads();
  if (xhi && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < T * (L / 32); i += blockDim.x) {
      const int t = i / (L / 32), blk = i % (L / 32);
      uint4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const uint4*>(&xs[t][blk * 32 + q * 8]);
      const size_t o = static_cast<size_t>(t) * H + h0 + blk * 32;
      uint8_t* sc = xsc + static_cast<size_t>(t) * xsc_pitch + (h0 / 32) + blk;
      if (xlo)
        mx_split_block(v, xhi + o, xlo + o, sc);
      else
        mxfp8_block(v, xhi + o, sc);
    }
  }
  if (!have_row) return;
  for (int t = 0; t < T; ++t) {
    float acc = 0.f;
    if (lane * 4 < L) {
      const uint2 xv = *reinterpret_cast<const uint2*>(&xs[t][lane * 4]);
      acc = bf16_to_f32(xv.x & 0xFFFF) * wv.x;
      acc = fmaf(bf16_to_f32(xv.x >> 16), wv.y, acc);
      acc = fmaf(bf16_to_f32(xv.y & 0xFFFF), wv.z, acc);
      acc = fmaf(bf16_to_f32(xv.y >> 16), wv.w, acc);
    }
    const float v = wave_sum_fixed(acc);
    if (lane == 0) part[(static_cast<size_t>(t) * rows + row) * S + s] = v;
  }
}

hipError_t launch_router_partial(const uint16_t* x, int T, int H, const float* router_w, int E,
                                 const float* shared_gate_w, float* part, uint8_t* xhi, uint8_t* xlo, uint8_t* xsc,
                                 int xsc_pitch, hipStream_t s) {
  const int rows = E + (shared_gate_w ? 1 : 0);
  const int S = router_splits(H);
  dim3 grid((rows + 3) / 4, S);
  return launch(router_partial_kernel, grid, dim3(256), 0, s, x, T, H, S, router_w, E, shared_gate_w, part, xhi, xlo,
                xsc, xsc_pitch);
}

// Logit of (token t, row e): the S partials, added in slice order.
template <int SQ>
__device__ __forceinline__ float sum_partials(const float* part, size_t base) {
  float4 v[SQ];
  const float4* p = reinterpret_cast<const float4*>(part + base);
#pragma unroll
  for (int q = 0; q < SQ; ++q) v[q] = p[q];
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < SQ; ++q) acc = ((acc + v[q].x) + v[q].y + v[q].z) + v[q].w;
  return acc;
}

// Fused decode top-k + align: one workgroup of 1024 threads.  Wave t < T sums
// token t's partial logits (slices in order), adds the bias and runs k rounds
// of wave argmax (DPP reductions); then the whole workgroup aligns the T*k
// routed rows into blocks of kDecodeBM (stable counting sort in LDS).
template <int SLOTS, int SQ>
__global__ __launch_bounds__(1024) void topk_align_decode_kernel(
    const float* __restrict__ part, int S, int T, int E, int k, const float* __restrict__ bias, int bias_select,
    int has_shared,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ sgate, int32_t* counts, int32_t* offsets,
    int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded, int P, uint32_t* zero_words, int n_zero) {
  constexpr int kRowWaves = kDecodeMaxT * 16 / kWave;   // waves of routed rows (T * k <= 256)
  constexpr int kFewRows = 32;
  __shared__ __attribute__((aligned(16))) int ids_s[kDecodeMaxT * 16];
  __shared__ int cnt[kAlignMaxE];
  __shared__ int cntw[kRowWaves][kAlignMaxE];   // rows of each expert in each wave of 64 rows
  __shared__ int tmp[32];
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  const int rows = E + (has_shared ? 1 : 0);
  const int nw = (T * k + kWave - 1) / kWave;
  for (int i = tid; i < n_zero; i += blockDim.x) zero_words[i] = 0u;
  // every sorted slot starts as the sentinel (coalesced); the routed rows'
  // slots are overwritten at the end, after several barriers
  for (int i = tid; i < P; i += blockDim.x) sorted_ids[i] = T * k;
  const bool few = T * k <= kFewRows;   // rank by a scan of the earlier rows
  if (few)
    cnt[tid] = 0;
  else
    for (int i = tid; i < nw * kAlignMaxE; i += blockDim.x) cntw[i / kAlignMaxE][i % kAlignMaxE] = 0;
  if (wv < T) {
    const int t = wv;
    float v[SLOTS];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) {
      const int e = lane + i * kWave;
      float acc = -__builtin_inff();
      if (e < E) {
        acc = sum_partials<SQ>(part, (static_cast<size_t>(t) * rows + e) * S);
        if (bias) acc += bias[e];
      }
      v[i] = acc;
    }
    int sel_i;
    float sel_w;
    wave_topk_softmax<SLOTS>(v, k, &sel_i, &sel_w);
    if (bias && bias_select)   // weights from the selected logits without the bias
      sel_w = lanes_softmax(lane < k ? sum_partials<SQ>(part, (static_cast<size_t>(t) * rows + sel_i) * S) : 0.f, k);
    if (lane < k) {
      ids[t * k + lane] = sel_i;
      w[t * k + lane] = sel_w;
      ids_s[t * k + lane] = sel_i;
    }
    if (has_shared && lane == 0) {
      const float g = sum_partials<SQ>(part, (static_cast<size_t>(t) * rows + E) * S);
      sgate[t] = 1.0f / (1.0f + expf(-g));
    }
  }
  if (P == 0) return;  // routing only
  __syncthreads();
  const int n = T * k;
  // Stable rank of row i among the earlier rows of its expert.  Up to
  // kFewRows rows: counts by LDS atomics and the rank by a scan of the
  // earlier rows.  More: wave rw takes rows [64 rw, 64 rw + 64), the lanes
  // holding the same expert are found with one ballot per bit of the id,
  // and the last lane of each group records the wave's count of that
  // expert; rows of earlier waves are counted through those records.
  int my_id = -1, rank_in = 0;
  if (few) {
    if (tid < n) {
      my_id = ids_s[tid];
      atomicAdd(&cnt[my_id], 1);
      for (int j = 0; j < tid; ++j) rank_in += ids_s[j] == my_id;
    }
  } else if (wv < nw) {   // uniform per wave
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    my_id = tid < n ? ids_s[tid] : -1;
    uint64_t peers = __ballot(my_id >= 0);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (my_id >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    rank_in = __popcll(peers & ((uint64_t{1} << lane) - 1));
    if (my_id >= 0 && (peers >> lane) == 1) cntw[wv][my_id] = __popcll(peers);
  }
  __syncthreads();
  int c = 0;
  if (tid < E) {
    if (few)
      c = cnt[tid];
    else
      for (int w = 0; w < nw; ++w) c += cntw[w][tid];
  }
  int off, total;
  finish_layout(tid, E, c, kDecodeBM, n, P, counts, offsets, sorted_ids, block_expert, num_padded, tmp, &off,
                &total, false);
  if (tid < E) cnt[tid] = off;   // segment starts
  __syncthreads();
  if (my_id >= 0) {
    int before = 0;
    if (!few)
      for (int w = 0; w < wv; ++w) before += cntw[w][my_id];
    sorted_ids[cnt[my_id] + before + rank_in] = tid;
  }
}

hipError_t launch_topk_align_decode(const float* part, int S, int T, int E, int k, const float* bias,
                                    bool bias_select, bool has_shared, int32_t* ids, float* w, float* sg, int32_t* counts,
                                    int32_t* offsets, int32_t* sorted_ids, int32_t* block_expert,
                                    int32_t* num_padded, int P, uint32_t* zero_words, int n_zero,
                                    hipStream_t s) {
  return with_slots(E, [&]<int SL>() {
    auto go = [&]<int SQ>() {
      return launch(topk_align_decode_kernel<SL, SQ>, dim3(1), dim3(1024), 0, s, part, S, T, E, k, bias,
                    bias_select ? 1 : 0, has_shared ? 1 : 0, ids, w, sg, counts, offsets, sorted_ids, block_expert,
                    num_padded, P, zero_words, n_zero);
    };
    switch (S / 4) {
      case 1: return go.template operator()<1>();
      case 2: return go.template operator()<2>();
      case 3: return go.template operator()<3>();
      case 4: return go.template operator()<4>();
      case 5: return go.template operator()<5>();
      case 6: return go.template operator()<6>();
      case 7: return go.template operator()<7>();
      case 8: return go.template operator()<8>();
      default: return hipErrorInvalidValue;
    }
  });
}

}  // namespace ftmoe
