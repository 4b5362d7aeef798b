// Host half of CPU-GPU co-execution (see host_experts.hpp).  Weight rows are
// decoded to fp32 once per expert and reused by every row routed to it;
// the dot products run 8 lanes wide with FMA.  Only the functions marked
// FT_AVX2 use AVX2/FMA, and they run only after cpu_supported().
#include "host_experts.hpp"

#include <immintrin.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <numeric>

#include "ftmoe.h"

namespace ftmoe_host {

// ------------------------------------------------------------------ pool ---
Pool::Pool(int threads) {
  for (int i = 1; i < threads; ++i) workers_.emplace_back([this] { work(); });
}

Pool::~Pool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
  }
  cv_.notify_all();
  for (std::thread& t : workers_) t.join();
}

void Pool::run(int n, const std::function<void(int)>& fn) {
  {
    std::lock_guard<std::mutex> lk(mu_);
    fn_ = &fn;
    n_ = n;
    next_.store(0);
    busy_ = static_cast<int>(workers_.size());
    ++gen_;
  }
  cv_.notify_all();
  for (int i; (i = next_.fetch_add(1)) < n;) fn(i);
  std::unique_lock<std::mutex> lk(mu_);
  done_cv_.wait(lk, [&] { return busy_ == 0; });
  fn_ = nullptr;
}

void Pool::work() {
  uint64_t seen = 0;
  std::unique_lock<std::mutex> lk(mu_);
  for (;;) {
    cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
    if (stop_) return;
    seen = gen_;
    const std::function<void(int)>* fn = fn_;
    const int n = n_;
    lk.unlock();
    for (int i; (i = next_.fetch_add(1)) < n;) (*fn)(i);
    lk.lock();
    if (--busy_ == 0) done_cv_.notify_one();
  }
}

bool cpu_supported() { return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma"); }

namespace {

// ---------------------------------------------------------------- codecs ---
// E4M3FN (bias 7, no infinities, 0x7F / 0xFF NaN): value of every byte.
struct E4M3Table {
  float v[256];
  E4M3Table() {
    for (int c = 0; c < 256; ++c) {
      const int e = (c >> 3) & 15, m = c & 7;
      float a = e == 0 ? ldexpf(static_cast<float>(m), -9) : ldexpf(1.f + m / 8.f, e - 7);
      if ((c & 0x7F) == 0x7F) a = NAN;
      v[c] = (c & 0x80) ? -a : a;
    }
  }
};
const E4M3Table kE4M3;

// 2^(s - 127) / 2 for every E8M0 byte (the E2M1 decoder yields twice the value).
struct E8M0HalfTable {
  float v[256];
  E8M0HalfTable() {
    for (int c = 0; c < 256; ++c) v[c] = ldexpf(0.5f, c - 127);
  }
};
const E8M0HalfTable kE8M0Half;

// Nearest E4M3FN value of a (finite) float, ties to even, saturating at 448.
inline float e4m3_nearest(float v) {
  const float a = fabsf(v);
  float q;
  if (a >= 448.f) {
    q = 448.f;
  } else if (a < 0.015625f) {   // below 2^-6 the grid is the subnormal step 2^-9
    q = nearbyintf(a * 512.f) * (1.f / 512.f);
  } else {
    int e;
    frexpf(a, &e);   // a in [2^(e-1), 2^e): three mantissa bits give a step of 2^(e-4)
    const float step = ldexpf(1.f, e - 4);
    q = nearbyintf(a / step) * step;
  }
  return copysignf(q, v);
}

// One MXFP8 block (OCP Microscaling v1.0, E4M3 elements): v[0..32) replaced
// by its dequantised values 2^X * e4m3(v / 2^X), X = floor(log2 amax) - 8
// (at least -127).
inline void mxfp8_block(float* v) {
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int X = -127;
  if (amax > 0.f) {
    int e;
    frexpf(amax, &e);
    X = std::max(e - 1 - 8, -127);
  }
  for (int i = 0; i < 32; ++i) v[i] = ldexpf(e4m3_nearest(ldexpf(v[i], -X)), X);
}

inline float bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return f;
}

inline float bf16_bits(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

#define FT_AVX2 __attribute__((target("avx2,fma")))

// 32 E2M1 codes (16 bytes, element 2i in the low nibble) as 2x their value,
// int8, in element order.
FT_AVX2 inline void e2m1x2_32(const uint8_t* p, __m128i& a, __m128i& b) {
  const __m128i m = _mm_set1_epi8(0x0F);
  const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i*>(p));
  const __m128i lo = _mm_and_si128(v, m), hi = _mm_and_si128(_mm_srli_epi16(v, 4), m);
  const __m128i lut = _mm_setr_epi8(0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12);
  a = _mm_shuffle_epi8(lut, _mm_unpacklo_epi8(lo, hi));
  b = _mm_shuffle_epi8(lut, _mm_unpackhi_epi8(lo, hi));
}

FT_AVX2 inline __m256 i8x8_to_ps(__m128i v) { return _mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v)); }

// Row `row` of expert e decoded to fp32 without its fp32 multiplier (the
// block scales included).
FT_AVX2 void decode_row(const Mat& w, int e, int row, float* out) {
  const int K = w.k;
  const size_t r = static_cast<size_t>(e) * w.n + row;
  switch (w.fmt) {
    case FTMOE_W_MXFP4: {
      const uint8_t* c = w.codes + r * (K / 2);
      const uint8_t* s = w.scales + r * (K / 32);
      for (int b = 0; b < K / 32; ++b) {
        __m128i x0, x1;
        e2m1x2_32(c + 16 * b, x0, x1);
        const __m256 sc = _mm256_set1_ps(kE8M0Half.v[s[b]]);
        float* o = out + 32 * b;
        _mm256_storeu_ps(o, _mm256_mul_ps(i8x8_to_ps(x0), sc));
        _mm256_storeu_ps(o + 8, _mm256_mul_ps(i8x8_to_ps(_mm_srli_si128(x0, 8)), sc));
        _mm256_storeu_ps(o + 16, _mm256_mul_ps(i8x8_to_ps(x1), sc));
        _mm256_storeu_ps(o + 24, _mm256_mul_ps(i8x8_to_ps(_mm_srli_si128(x1, 8)), sc));
      }
      break;
    }
    case FTMOE_W_NVFP4: {
      const uint8_t* c = w.codes + r * (K / 2);
      const uint8_t* s = w.scales + r * (K / 16);
      for (int b = 0; b < K / 32; ++b) {
        __m128i x0, x1;
        e2m1x2_32(c + 16 * b, x0, x1);
        const __m256 s0 = _mm256_set1_ps(0.5f * kE4M3.v[s[2 * b]]);
        const __m256 s1 = _mm256_set1_ps(0.5f * kE4M3.v[s[2 * b + 1]]);
        float* o = out + 32 * b;
        _mm256_storeu_ps(o, _mm256_mul_ps(i8x8_to_ps(x0), s0));
        _mm256_storeu_ps(o + 8, _mm256_mul_ps(i8x8_to_ps(_mm_srli_si128(x0, 8)), s0));
        _mm256_storeu_ps(o + 16, _mm256_mul_ps(i8x8_to_ps(x1), s1));
        _mm256_storeu_ps(o + 24, _mm256_mul_ps(i8x8_to_ps(_mm_srli_si128(x1, 8)), s1));
      }
      break;
    }
    case FTMOE_W_FP8_E4M3: {
      const uint8_t* c = w.codes + r * K;
      for (int i = 0; i < K; ++i) out[i] = kE4M3.v[c[i]];
      break;
    }
    default: {   // BF16
      const uint16_t* c = reinterpret_cast<const uint16_t*>(w.codes) + r * K;
      for (int i = 0; i < K; i += 8) {
        const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i*>(c + i));
        _mm256_storeu_ps(out + i, _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(v), 16)));
      }
    }
  }
}

inline float multiplier(const Mat& w, int e, int row) {
  if (w.fmt != FTMOE_W_NVFP4 && w.fmt != FTMOE_W_FP8_E4M3) return 1.f;
  return w.rowsc ? w.tscale[static_cast<size_t>(e) * w.n + row] : w.tscale[e];
}

// a . b summed as dot4 sums each of its rows (two 8-lane accumulators over
// steps of 16, then the same horizontal order), so a row's result does not
// depend on how many rows share the weight row.
FT_AVX2 float dot(const float* a, const float* b, int K) {
  __m256 s = _mm256_setzero_ps(), t = s;
  for (int i = 0; i < K; i += 16) {
    s = _mm256_fmadd_ps(_mm256_loadu_ps(a + i), _mm256_loadu_ps(b + i), s);
    t = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 8), _mm256_loadu_ps(b + i + 8), t);
  }
  const __m256 v = _mm256_add_ps(s, t);
  __m128 h = _mm_add_ps(_mm256_castps256_ps128(v), _mm256_extractf128_ps(v, 1));
  h = _mm_add_ps(h, _mm_movehl_ps(h, h));
  h = _mm_add_ss(h, _mm_movehdup_ps(h));
  return _mm_cvtss_f32(h);
}

// Four dot products of one row a with rows b0..b3 (the row a is loaded once per four).
FT_AVX2 void dot4(const float* a, const float* b0, const float* b1, const float* b2, const float* b3, int K,
                  float* out) {
  __m256 s0 = _mm256_setzero_ps(), s1 = s0, s2 = s0, s3 = s0, t0 = s0, t1 = s0, t2 = s0, t3 = s0;
  for (int i = 0; i < K; i += 16) {
    const __m256 w0 = _mm256_loadu_ps(a + i), w1 = _mm256_loadu_ps(a + i + 8);
    s0 = _mm256_fmadd_ps(w0, _mm256_loadu_ps(b0 + i), s0);
    s1 = _mm256_fmadd_ps(w0, _mm256_loadu_ps(b1 + i), s1);
    s2 = _mm256_fmadd_ps(w0, _mm256_loadu_ps(b2 + i), s2);
    s3 = _mm256_fmadd_ps(w0, _mm256_loadu_ps(b3 + i), s3);
    t0 = _mm256_fmadd_ps(w1, _mm256_loadu_ps(b0 + i + 8), t0);
    t1 = _mm256_fmadd_ps(w1, _mm256_loadu_ps(b1 + i + 8), t1);
    t2 = _mm256_fmadd_ps(w1, _mm256_loadu_ps(b2 + i + 8), t2);
    t3 = _mm256_fmadd_ps(w1, _mm256_loadu_ps(b3 + i + 8), t3);
  }
  const __m256 v[4] = {_mm256_add_ps(s0, t0), _mm256_add_ps(s1, t1), _mm256_add_ps(s2, t2), _mm256_add_ps(s3, t3)};
  for (int r = 0; r < 4; ++r) {
    __m128 h = _mm_add_ps(_mm256_castps256_ps128(v[r]), _mm256_extractf128_ps(v[r], 1));
    h = _mm_add_ps(h, _mm_movehl_ps(h, h));
    h = _mm_add_ss(h, _mm_movehdup_ps(h));
    out[r] = _mm_cvtss_f32(h);
  }
}

// out[r] = a . rows[r], r < nr, rows `stride` floats apart.
void dot_rows(const float* a, const float* rows, size_t stride, int nr, int K, float* out) {
  int r = 0;
  for (; r + 4 <= nr; r += 4)
    dot4(a, rows + r * stride, rows + (r + 1) * stride, rows + (r + 2) * stride, rows + (r + 3) * stride, K,
         out + r);
  for (; r < nr; ++r) out[r] = dot(a, rows + r * stride, K);
}

constexpr int kMaxK = 4096;
constexpr int kMaxRowsStep = 64;   // rows per dot_rows call (the per-thread result buffers)
constexpr int kChunk = 32;   // h elements (gate/up row pairs) or output columns per work item

}  // namespace

bool expert_rows(Pool& pool, const Mat& gu, const Mat& dn, int H, int I, bool mx8, const uint16_t* x,
                 const int32_t* tok, const int32_t* ex, int n, float* o) {
  if (!cpu_supported() || H > kMaxK || I > kMaxK || H % kChunk || I % kChunk) return false;
  if (n <= 0) return true;
  // rows grouped by expert (stable), one job per expert
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return ex[a] < ex[b]; });
  std::vector<int> job_start;
  for (int i = 0; i < n; ++i)
    if (i == 0 || ex[order[i]] != ex[order[i - 1]]) job_start.push_back(i);
  const int njobs = static_cast<int>(job_start.size());
  job_start.push_back(n);

  // activations in fp32, in grouped order (MXFP8 layers: quantised per 32-block)
  std::vector<float> xs(static_cast<size_t>(n) * H), hs(static_cast<size_t>(n) * I);
  pool.run(n, [&](int i) {
    const uint16_t* src = x + static_cast<size_t>(tok[order[i]]) * H;
    float* dst = xs.data() + static_cast<size_t>(i) * H;
    for (int c = 0; c < H; ++c) dst[c] = bf16_bits(src[c]);
    if (mx8)
      for (int c = 0; c < H; c += 32) mxfp8_block(dst + c);
  });

  // gate_up + SwiGLU: item = (job, 32 consecutive h elements)
  const int ia = I / kChunk;
  pool.run(njobs * ia, [&](int item) {
    const int j = item / ia, i0 = (item % ia) * kChunk;
    const int e = ex[order[job_start[j]]], r0 = job_start[j], nr = job_start[j + 1] - r0;
    alignas(32) float wg[kMaxK], wu[kMaxK];
    float g[kMaxRowsStep], u[kMaxRowsStep];
    for (int i = i0; i < i0 + kChunk; ++i) {
      decode_row(gu, e, i, wg);
      decode_row(gu, e, I + i, wu);
      const float mg = multiplier(gu, e, i), mu = multiplier(gu, e, I + i);
      for (int ra = 0; ra < nr; ra += kMaxRowsStep) {
        const int m = std::min(kMaxRowsStep, nr - ra);
        const float* xr = xs.data() + static_cast<size_t>(r0 + ra) * H;
        dot_rows(wg, xr, H, m, H, g);
        dot_rows(wu, xr, H, m, H, u);
        for (int r = 0; r < m; ++r) {
          const float gv = g[r] * mg;
          hs[static_cast<size_t>(r0 + ra + r) * I + i] = gv / (1.f + expf(-gv)) * (u[r] * mu);
        }
      }
    }
    for (int r = 0; r < nr; ++r) {
      float* h = hs.data() + static_cast<size_t>(r0 + r) * I + i0;
      if (mx8)
        mxfp8_block(h);
      else
        for (int q = 0; q < kChunk; ++q) h[q] = bf16_round(h[q]);
    }
  });

  // down: item = (job, 32 output columns)
  const int ib = H / kChunk;
  pool.run(njobs * ib, [&](int item) {
    const int j = item / ib, c0 = (item % ib) * kChunk;
    const int e = ex[order[job_start[j]]], r0 = job_start[j], nr = job_start[j + 1] - r0;
    alignas(32) float wd[kMaxK];
    float d[kMaxRowsStep];
    for (int c = c0; c < c0 + kChunk; ++c) {
      decode_row(dn, e, c, wd);
      const float mult = multiplier(dn, e, c);
      for (int ra = 0; ra < nr; ra += kMaxRowsStep) {
        const int m = std::min(kMaxRowsStep, nr - ra);
        dot_rows(wd, hs.data() + static_cast<size_t>(r0 + ra) * I, I, m, I, d);
        for (int r = 0; r < m; ++r) o[static_cast<size_t>(order[r0 + ra + r]) * H + c] = d[r] * mult;
      }
    }
  });
  return true;
}

}  // namespace ftmoe_host
