// The CPU tier: int4 experts kept in host memory and computed on the host's cores while the
// device group runs (host code only).
//
// Source: "cuda: COLI_GROUP_ASYNC=1 - overlap the CPU expert rows with the GPU groups at decode",
// section "What": the device groups are issued first, the CPU computes its expert rows while the
// GPU works, then a take phase accumulates both.
#pragma once

#include <condition_variable>
#include <functional>
#include <mutex>
#include <stdint.h>
#include <thread>
#include <vector>

namespace i4moe {

// One int4 tensor in the host format of i4moe_upload_expert_tensor (offset nibbles, low nibble
// first, O * ceil(C/gs) or O scales), owned by the library.
struct HostTensor {
  int O = 0, C = 0, gs = 0, ng = 1;
  std::vector<uint8_t> packed;  // O * C/2
  std::vector<float> scales;    // O * ng
};

struct HostExpert {
  HostTensor gate, up, down;  // I x D, I x D, D x I
};

// Fixed worker threads.  run(n, fn) splits [0, n) into one contiguous range per thread (the same
// split every time for the same n and thread count) and returns when all ranges are done; each
// index is handled by exactly one thread, so per-index results never depend on timing.
class HostPool {
 public:
  explicit HostPool(int threads);
  ~HostPool();
  HostPool(const HostPool &) = delete;
  HostPool &operator=(const HostPool &) = delete;
  int threads() const { return (int)workers_.size() + 1; }
  void run(long n, const std::function<void(long begin, long end)> &fn);

 private:
  void work(int id);
  std::vector<std::thread> workers_;
  std::mutex m_;
  std::condition_variable go_, done_;
  const std::function<void(long, long)> *fn_ = nullptr;
  long n_ = 0;
  unsigned gen_ = 0;
  int pending_ = 0;
  bool stop_ = false;
};

// One job at a time on a thread of its own: post(fn) hands fn over and returns at once, wait()
// returns when it has finished.
class HostHelper {
 public:
  HostHelper();
  ~HostHelper();
  HostHelper(const HostHelper &) = delete;
  HostHelper &operator=(const HostHelper &) = delete;
  void post(std::function<void()> fn);
  void wait();

 private:
  std::thread t_;
  std::mutex m_;
  std::condition_variable cv_;
  std::function<void()> job_;
  bool busy_ = false, stop_ = false;
};

// One host row: (token, expert, weight).
struct HostRow {
  int token;
  const HostExpert *e;
  float w;
};

// For the rows (in route order), in float32:
//   P[t][d] += sum over the rows r of token t, in order, of w_r * y_r[d],
//   y_r = down . (silu(gate . x_t) * (up . x_t))
// x: S x D float32 rows, P: S x D float32 (accumulated into).  Each weight row's dot product is
// summed group by group (a group's products summed, then scaled): in column order, or, on a host
// with AVX2 and FMA, 32 columns at a time in four 8-wide partial sums added in a fixed order.
void host_rows_forward(HostPool &pool, const std::vector<HostRow> &rows, const float *x, int D, int I, float *P);

}  // namespace i4moe
