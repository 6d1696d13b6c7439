// The CPU tier's arithmetic and worker pool (host code; see host_tier.h).
#include "host_tier.h"

#include <cmath>

namespace i4moe {

HostPool::HostPool(int threads) {
  for (int i = 1; i < threads; ++i) workers_.emplace_back([this, i] { work(i); });
}

HostPool::~HostPool() {
  {
    std::lock_guard<std::mutex> lk(m_);
    stop_ = true;
  }
  go_.notify_all();
  for (auto &t : workers_) t.join();
}

void HostPool::work(int id) {
  unsigned seen = 0;
  for (;;) {
    const std::function<void(long, long)> *fn;
    long n;
    {
      std::unique_lock<std::mutex> lk(m_);
      go_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (stop_) return;
      seen = gen_;
      fn = fn_;
      n = n_;
    }
    const long T = threads();
    (*fn)(n * id / T, n * (id + 1) / T);
    {
      std::lock_guard<std::mutex> lk(m_);
      if (--pending_ == 0) done_.notify_one();
    }
  }
}

void HostPool::run(long n, const std::function<void(long, long)> &fn) {
  if (n <= 0) return;
  if (workers_.empty()) {
    fn(0, n);
    return;
  }
  {
    std::lock_guard<std::mutex> lk(m_);
    fn_ = &fn;
    n_ = n;
    pending_ = (int)workers_.size();
    ++gen_;
  }
  go_.notify_all();
  fn(0, n / threads());  // the calling thread takes range 0
  std::unique_lock<std::mutex> lk(m_);
  done_.wait(lk, [&] { return pending_ == 0; });
}

namespace {

// sum over the columns [c0, c1) of row `row` (c0 even) of (q - 8) * x[c], in column order
inline float nibble_dot(const uint8_t *row, const float *x, int c0, int c1) {
  float s = 0.f;
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    const uint8_t b = row[c >> 1];
    s += (float)((int)(b & 15) - 8) * x[c];
    s += (float)((int)(b >> 4) - 8) * x[c + 1];
  }
  if (c < c1) s += (float)((int)(row[c >> 1] & 15) - 8) * x[c];
  return s;
}

// One output row of an int4 tensor against x: per-row, the scale times the whole sum; group-wise,
// each group's sum times its scale, added group by group (the last group may be narrower).
inline float row_dot(const HostTensor &T, int o, const float *x) {
  const uint8_t *row = T.packed.data() + (size_t)o * (T.C / 2);
  if (T.ng == 1) return T.scales[o] * nibble_dot(row, x, 0, T.C);
  const float *s = T.scales.data() + (size_t)o * T.ng;
  float acc = 0.f;
  for (int g = 0; g < T.ng; ++g) {
    const int c0 = g * T.gs, c1 = c0 + T.gs < T.C ? c0 + T.gs : T.C;
    acc += s[g] * nibble_dot(row, x, c0, c1);
  }
  return acc;
}

}  // namespace

void host_rows_forward(HostPool &pool, const std::vector<HostRow> &rows, const float *x, int D, int I, float *P) {
  const long n = (long)rows.size();
  if (n == 0) return;
  std::vector<float> h((size_t)n * I), y((size_t)n * D);
  // gate and up, SiLU-gated product: one (row, output) pair per index
  pool.run(n * I, [&](long b, long e) {
    for (long k = b; k < e; ++k) {
      const HostRow &r = rows[k / I];
      const int o = (int)(k % I);
      const float *xt = x + (size_t)r.token * D;
      const float g = row_dot(r.e->gate, o, xt);
      const float u = row_dot(r.e->up, o, xt);
      h[k] = g / (1.f + std::exp(-g)) * u;
    }
  });
  // down
  pool.run(n * D, [&](long b, long e) {
    for (long k = b; k < e; ++k) {
      const HostRow &r = rows[k / D];
      y[k] = row_dot(r.e->down, (int)(k % D), h.data() + (size_t)(k / D) * I);
    }
  });
  // the weighted sum per token, rows in order: one column per index
  pool.run(D, [&](long b, long e) {
    for (long d = b; d < e; ++d)
      for (long k = 0; k < n; ++k) {
        float &p = P[(size_t)rows[k].token * D + d];
        p = std::fma(rows[k].w, y[(size_t)k * D + d], p);
      }
  });
}

}  // namespace i4moe
