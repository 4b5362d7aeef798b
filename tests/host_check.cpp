// Host-code check program for the sanitizer builds (AddressSanitizer with
// UndefinedBehaviorSanitizer, and ThreadSanitizer) of the ftmoe library's
// host code: argument validation of every entry point, the expert-slot
// pool's residency planner, and the threaded host expert kernels of CPU-GPU
// co-execution with its calibration.  Nothing here touches a GPU: device
// pointers are placeholders that validation never dereferences, and the pool
// is only planned, never filled.  Exits non-zero on the first failed check
// (the sanitizers abort on their own findings).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "ftmoe.h"

namespace {

int g_failures = 0;

#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_failures;                                                       \
    }                                                                     \
  } while (0)

void* fake() { return reinterpret_cast<void*>(static_cast<uintptr_t>(1) << 20); }

// Host arrays of one small layer in a format (random codes and scales).
struct HostSet {
  std::vector<uint8_t> codes, scales;
  std::vector<float> ts;
  ftmoe_qweight q{};
};

HostSet make_set(int fmt, int E, int n, int k, std::mt19937& rng) {
  HostSet h;
  const size_t nk = static_cast<size_t>(E) * n * k;
  std::uniform_int_distribution<int> byte(0, 255);
  if (fmt == FTMOE_W_MXFP4 || fmt == FTMOE_W_NVFP4) {
    h.codes.resize(nk / 2);
    h.scales.resize(nk / (fmt == FTMOE_W_MXFP4 ? 32 : 16));
    for (auto& c : h.codes) c = static_cast<uint8_t>(byte(rng));
    // scales near 1 so the sums stay finite (E8M0 around 127; E4M3 in [0x30, 0x40))
    for (auto& s : h.scales) s = static_cast<uint8_t>(fmt == FTMOE_W_MXFP4 ? 120 + byte(rng) % 8 : 0x30 + byte(rng) % 16);
  } else if (fmt == FTMOE_W_FP8_E4M3) {
    h.codes.resize(nk);
    for (auto& c : h.codes) {
      c = static_cast<uint8_t>(byte(rng));
      if ((c & 0x7F) == 0x7F) c = 0;
    }
  } else {
    h.codes.resize(2 * nk);
    for (size_t i = 0; i < nk; ++i) {   // bf16 values of moderate size
      const uint16_t b = static_cast<uint16_t>(0x3C00 + byte(rng) % 0x300) | static_cast<uint16_t>((byte(rng) & 1) << 15);
      std::memcpy(&h.codes[2 * i], &b, 2);
    }
  }
  if (fmt == FTMOE_W_NVFP4 || fmt == FTMOE_W_FP8_E4M3) h.ts.assign(E, 1.0f / 64.0f);
  h.q.fmt = fmt;
  h.q.num_experts = E;
  h.q.n = n;
  h.q.k = k;
  h.q.codes = h.codes.data();
  h.q.block_scales = h.scales.empty() ? nullptr : h.scales.data();
  h.q.tensor_scales = h.ts.empty() ? nullptr : h.ts.data();
  return h;
}

ftmoe_layer layer_of(int fmt, int act, int H, int I, int E, int k, const ftmoe_qweight& gu, const ftmoe_qweight& dn) {
  ftmoe_layer L{};
  L.hidden = H;
  L.inter = I;
  L.num_experts = E;
  L.top_k = k;
  L.act = act;
  L.path = FTMOE_PATH_AUTO;
  L.router_w = static_cast<const float*>(fake());
  L.gate_up = gu;
  L.down = dn;
  (void)fmt;
  return L;
}

void check_validation() {
  std::mt19937 rng(1);
  HostSet gu = make_set(FTMOE_W_MXFP4, 8, 256, 256, rng), dn = make_set(FTMOE_W_MXFP4, 8, 256, 128, rng);
  ftmoe_layer L = layer_of(FTMOE_W_MXFP4, FTMOE_ACT_BF16, 256, 128, 8, 2, gu.q, dn.q);
  size_t n = 0;
  CHECK(ftmoe_workspace_size(&L, 16, &n) == FTMOE_OK && n > 0);
  CHECK(ftmoe_workspace_bytes(&L, 16) == n);
  CHECK(ftmoe_workspace_bytes(nullptr, 16) == 0);
  CHECK(ftmoe_workspace_bytes(&L, -3) == 0);
  CHECK(std::strlen(ftmoe_last_error()) > 0);
  ftmoe_layer bad = L;
  bad.hidden = 100;
  CHECK(ftmoe_workspace_size(&bad, 16, &n) == FTMOE_ERR_UNSUPPORTED);
  bad = L;
  bad.top_k = 0;
  CHECK(ftmoe_workspace_size(&bad, 16, &n) == FTMOE_ERR_UNSUPPORTED);
  bad = L;
  bad.act = 7;
  CHECK(ftmoe_workspace_size(&bad, 16, &n) == FTMOE_ERR_INVALID_ARG);
  bad = L;
  bad.gate_up.k = 128;
  CHECK(ftmoe_workspace_size(&bad, 16, &n) != FTMOE_OK);
  // entry points refuse before enqueueing anything
  CHECK(ftmoe_forward(&L, nullptr, 4, fake(), 1 << 20, static_cast<uint16_t*>(fake()), nullptr, nullptr, nullptr) ==
        FTMOE_ERR_INVALID_ARG);
  CHECK(ftmoe_forward(&L, static_cast<uint16_t*>(fake()), 4, fake(), 16, static_cast<uint16_t*>(fake()), nullptr,
                      nullptr, nullptr) == FTMOE_ERR_WORKSPACE);
  CHECK(ftmoe_forward_noalloc(&L, static_cast<uint16_t*>(fake()), 1 << 20, static_cast<uint16_t*>(fake()), nullptr,
                              nullptr, nullptr) == FTMOE_ERR_WORKSPACE);
  CHECK(ftmoe_route(&L, static_cast<uint16_t*>(fake()), -1, fake(), 1 << 20, static_cast<int32_t*>(fake()),
                    static_cast<float*>(fake()), nullptr, nullptr) == FTMOE_ERR_INVALID_ARG);
  CHECK(ftmoe_align(static_cast<int32_t*>(fake()), 4, 2, 8, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                    nullptr) == FTMOE_ERR_INVALID_ARG);
  CHECK(ftmoe_align_max_padded(4, 17, 32, 16) == -1);
  CHECK(ftmoe_align_max_padded(16, 2, 8, 16) > 0);
  for (int st = 0; st <= 5; ++st) CHECK(ftmoe_status_string(static_cast<ftmoe_status>(st)) != nullptr);
}

// The residency planner: random step sequences, distinct slots within a
// step, counters that add up, refusals that change nothing.
void check_cache_planner() {
  std::mt19937 rng(2);
  for (int round = 0; round < 4; ++round) {
    const int E = 16 + 8 * round, slots = 4 + round;
    HostSet gu = make_set(FTMOE_W_MXFP4, E, 256, 256, rng), dn = make_set(FTMOE_W_MXFP4, E, 256, 128, rng);
    ftmoe_layer L = layer_of(FTMOE_W_MXFP4, FTMOE_ACT_BF16, 256, 128, E, 2, gu.q, dn.q);
    size_t pool = 0;
    CHECK(ftmoe_cache_pool_size(&L, slots, &pool) == FTMOE_OK && pool > 0);
    ftmoe_cache* c = nullptr;
    CHECK(ftmoe_cache_create(&L, &gu.q, &dn.q, slots, fake(), pool, &c) == FTMOE_OK && c);
    if (!c) return;
    int64_t plans = 0;
    for (int step = 0; step < 200; ++step) {
      std::vector<int32_t> e(E);
      for (int i = 0; i < E; ++i) e[i] = i;
      std::shuffle(e.begin(), e.end(), rng);
      const int n = 1 + static_cast<int>(rng() % slots);
      e.resize(n);
      std::vector<int32_t> sl(n), miss(n);
      CHECK(ftmoe_cache_plan(c, e.data(), n, sl.data(), miss.data()) == FTMOE_OK);
      std::vector<int> seen(slots, 0);
      for (int i = 0; i < n; ++i) {
        CHECK(sl[i] >= 0 && sl[i] < slots);
        if (sl[i] >= 0 && sl[i] < slots) CHECK(++seen[sl[i]] == 1);
      }
      plans += n;
    }
    int64_t hits = -1, misses = -1, bytes = -1, passes = -1;
    CHECK(ftmoe_cache_stats(c, &hits, &misses, &bytes, &passes) == FTMOE_OK);
    CHECK(hits + misses == plans && bytes == 0 && passes == 0);
    std::vector<int32_t> too_many(slots + 1);
    for (int i = 0; i <= slots; ++i) too_many[i] = i;
    CHECK(ftmoe_cache_plan(c, too_many.data(), slots + 1, nullptr, nullptr) == FTMOE_ERR_UNSUPPORTED);
    const int32_t twice[2] = {1, 1}, outside[1] = {E};
    CHECK(ftmoe_cache_plan(c, twice, 2, nullptr, nullptr) == FTMOE_ERR_INVALID_ARG);
    CHECK(ftmoe_cache_plan(c, outside, 1, nullptr, nullptr) == FTMOE_ERR_INVALID_ARG);
    size_t ws = 0;
    CHECK(ftmoe_cache_workspace_size(c, 8, &ws) == FTMOE_OK && ws > 0);
    ftmoe_cache_destroy(c);
  }
}

// Host expert rows: the same rows give the same bits whatever the number of
// threads (one summation order per row), for every format; and the pool's
// host compute calibration creates, uses and tears down its threads.
void check_host_experts() {
  struct Fmt {
    int fmt, act;
  } fmts[] = {{FTMOE_W_MXFP4, FTMOE_ACT_BF16},
              {FTMOE_W_MXFP4, FTMOE_ACT_MXFP8},
              {FTMOE_W_NVFP4, FTMOE_ACT_BF16},
              {FTMOE_W_FP8_E4M3, FTMOE_ACT_BF16},
              {FTMOE_W_BF16, FTMOE_ACT_BF16}};
  std::mt19937 rng(3);
  const int H = 256, I = 128, E = 6, T = 9, n = 23;
  std::vector<uint16_t> x(static_cast<size_t>(T) * H);
  for (auto& v : x) v = static_cast<uint16_t>(0x3E00 + rng() % 0x200) | static_cast<uint16_t>((rng() & 1) << 15);
  std::vector<int32_t> tok(n), ex(n);
  for (int i = 0; i < n; ++i) {
    tok[i] = static_cast<int32_t>(rng() % T);
    ex[i] = static_cast<int32_t>(rng() % E);
  }
  for (const Fmt& f : fmts) {
    HostSet gu = make_set(f.fmt, E, 2 * I, H, rng), dn = make_set(f.fmt, E, H, I, rng);
    ftmoe_layer L = layer_of(f.fmt, f.act, H, I, E, 2, gu.q, dn.q);
    std::vector<float> ref(static_cast<size_t>(n) * H), o(static_cast<size_t>(n) * H);
    const ftmoe_status st = ftmoe_host_expert_rows(&L, x.data(), tok.data(), ex.data(), n, ref.data(), 1);
    if (st == FTMOE_ERR_UNSUPPORTED) {   // a CPU without AVX2 / FMA: nothing more to check here
      std::fprintf(stderr, "host expert kernels unsupported on this CPU\n");
      return;
    }
    CHECK(st == FTMOE_OK);
    for (int threads : {2, 3, 8, 16}) {
      for (int rep = 0; rep < 3; ++rep) {
        std::fill(o.begin(), o.end(), -1.0f);
        CHECK(ftmoe_host_expert_rows(&L, x.data(), tok.data(), ex.data(), n, o.data(), threads) == FTMOE_OK);
        CHECK(std::memcmp(o.data(), ref.data(), o.size() * sizeof(float)) == 0);
      }
    }
    bool finite = true;
    for (float v : ref) finite = finite && std::isfinite(v);
    CHECK(finite);
    const int32_t bad_ex[1] = {E};
    CHECK(ftmoe_host_expert_rows(&L, x.data(), tok.data(), bad_ex, 1, o.data(), 2) == FTMOE_ERR_INVALID_ARG);
    // calibration on a pool: threads made, the cost model measured, threads joined
    size_t pool = 0;
    CHECK(ftmoe_cache_pool_size(&L, 3, &pool) == FTMOE_OK);
    ftmoe_cache* c = nullptr;
    CHECK(ftmoe_cache_create(&L, &gu.q, &dn.q, 3, fake(), pool, &c) == FTMOE_OK && c);
    if (!c) continue;
    for (int threads : {4, 1, 7}) {
      CHECK(ftmoe_cache_set_host_compute(c, threads, 0.0, -1.0, 0.0) == FTMOE_OK);
      double es = 0, rs = -1;
      CHECK(ftmoe_cache_host_stats(c, nullptr, nullptr, nullptr, &es, &rs) == FTMOE_OK);
      CHECK(es > 0 && rs >= 0);
    }
    CHECK(ftmoe_cache_set_host_compute(c, 0, 0.0, 0.0, 0.0) == FTMOE_OK);
    ftmoe_cache_destroy(c);
  }
}

}  // namespace

int main() {
  check_validation();
  check_cache_planner();
  check_host_experts();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
