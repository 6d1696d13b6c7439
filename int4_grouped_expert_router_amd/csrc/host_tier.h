// The CPU tier: int4 experts kept in host memory and computed on the host's cores while the
// device group runs (host code only).
//
// Source: "cuda: COLI_GROUP_ASYNC=1 - overlap the CPU expert rows with the GPU groups at decode",
// section "What": the device groups are issued first, the CPU computes its expert rows while the
// GPU works, then a take phase accumulates both.
#pragma once

#include <atomic>
#include <condition_variable>
#include <exception>
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
// index is handled by exactly one thread, so per-index results never depend on timing.  An
// exception thrown by a range is rethrown by run() on the calling thread once every range is done.  Between
// runs a worker polls for the next one for about kSpinMicros before it sleeps, so the phases of
// one computation follow each other without a wake-up through the kernel.
class HostPool {
 public:
  explicit HostPool(int threads);
  ~HostPool();
  HostPool(const HostPool &) = delete;
  HostPool &operator=(const HostPool &) = delete;
  int threads() const { return (int)workers_.size() + 1; }
  void run(long n, const std::function<void(long begin, long end)> &fn);
  // Sleeping workers start polling again (for kSpinMicros), so a run that follows within that
  // time finds them awake: call it ahead of a run whose inputs are still on their way.
  void warm();
  static constexpr int kSpinMicros = 200;

 private:
  void work(int id);
  std::vector<std::thread> workers_;
  std::mutex m_;
  std::condition_variable go_;
  const std::function<void(long, long)> *fn_ = nullptr;
  long n_ = 0;
  std::atomic<unsigned> gen_{0}, wake_{0};
  std::atomic<int> pending_{0}, sleepers_{0};
  std::atomic<bool> stop_{false};
  std::exception_ptr error_;  // the first exception a worker's range threw in the current run
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

// For the rows (in route order):
//   P[t][d] += sum over the rows r of token t, in order, of w_r * y_r[d],
//   y_r = down . (silu(gate . x_t) * (up . x_t))
// x: S x D float32 rows, P: S x D float32 (accumulated into).  Two ways to a weight row's dot
// product, each deterministic:
//  * integer (hosts with AVX-512 VNNI, when every tensor is per-row or its group size a multiple
//    of 64): the activation row (x_t, or one row of h) in 24-bit fixed point with its own
//    power-of-two exponent, as three int8 digits; each group's sum an exact integer, times its
//    scale (groups of 64 columns: in float32 lane sums, even and odd groups apart; otherwise in
//    double), the lanes added in double, rounded to float32 at the end;
//  * float32 (otherwise, or with I4MOE_HOST_INT=0 in the environment): each group's products
//    summed, then scaled: in column order, or, on a host with AVX2 and FMA, 32 columns at a time
//    in four 8-wide partial sums added in a fixed order.
// SiLU, the gated product and the weighted sum are float32 either way.
void host_rows_forward(HostPool &pool, const std::vector<HostRow> &rows, const float *x, int D, int I, float *P);

// Whether this host can take the integer path.
bool host_int_path_available();

}  // namespace i4moe
