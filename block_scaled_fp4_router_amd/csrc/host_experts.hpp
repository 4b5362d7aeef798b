// Host half of CPU-GPU co-execution: routed SwiGLU experts computed on the
// host cores from the matrices where they live in host memory (the FreeToken
// README, "About": its runtime splits MoE work between the host CPU and the
// GPU).  Plain C++ (AVX2/FMA), no HIP; the device side only scatters the
// rows this produces into its own output buffer.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace ftmoe_host {

// One stacked matrix set [E][N][K] in host memory, in the layout and
// formats of the device path (fmt: an ftmoe_wfmt).
struct Mat {
  int fmt = 0;
  int n = 0, k = 0;
  const uint8_t* codes = nullptr;
  const uint8_t* scales = nullptr;
  const float* tscale = nullptr;
  int rowsc = 0;
};

// A fixed set of worker threads that run one parallel-for at a time (the
// calling thread works too).
class Pool {
 public:
  explicit Pool(int threads);
  ~Pool();
  int size() const { return static_cast<int>(workers_.size()) + 1; }
  // Calls fn(i) for every i in [0, n), spread over the threads; returns when all are done.
  void run(int n, const std::function<void(int)>& fn);

 private:
  void work();
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int)>* fn_ = nullptr;
  int n_ = 0;
  std::atomic<int> next_{0};
  int busy_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

// Expert outputs for rows: row r is token tok[r] of x [*][H] (bf16 bits)
// through expert ex[r]; o [n][H] fp32 = W_down h with h = silu(W_gate x) *
// (W_up x), h rounded to bf16 (mx8 = false) or each 32-block of h and of x
// quantised to MXFP8 (mx8 = true), as the device path does.  Rows of one
// expert share each decoded weight row.  False if the CPU lacks AVX2/FMA.
bool expert_rows(Pool& pool, const Mat& gu, const Mat& dn, int H, int I, bool mx8, const uint16_t* x,
                 const int32_t* tok, const int32_t* ex, int n, float* o);

bool cpu_supported();

}  // namespace ftmoe_host
