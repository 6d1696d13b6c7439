// The CPU tier's arithmetic and worker pool (host code; see host_tier.h).
#include "host_tier.h"

#include <immintrin.h>

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

HostHelper::HostHelper() {
  t_ = std::thread([this] {
    for (;;) {
      std::function<void()> job;
      {
        std::unique_lock<std::mutex> lk(m_);
        cv_.wait(lk, [&] { return stop_ || (busy_ && job_); });
        if (stop_) return;
        job = std::move(job_);
        job_ = nullptr;
      }
      job();
      {
        std::lock_guard<std::mutex> lk(m_);
        busy_ = false;
      }
      cv_.notify_all();
    }
  });
}

HostHelper::~HostHelper() {
  {
    std::lock_guard<std::mutex> lk(m_);
    stop_ = true;
  }
  cv_.notify_all();
  t_.join();
}

void HostHelper::post(std::function<void()> fn) {
  {
    std::lock_guard<std::mutex> lk(m_);
    job_ = std::move(fn);
    busy_ = true;
  }
  cv_.notify_all();
}

void HostHelper::wait() {
  std::unique_lock<std::mutex> lk(m_);
  cv_.wait(lk, [&] { return !busy_; });
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

// The same sum with AVX2 and FMA, 32 columns (16 bytes) per step in four 8-wide partial sums
// (added in a fixed order at the end), then the scalar loop for the columns left over.  Used when
// the host CPU has both; the order of additions differs from the scalar loop, never between runs.
__attribute__((target("avx2,fma"))) float nibble_dot_avx2(const uint8_t *row, const float *x, int c0, int c1) {
  __m256 a0 = _mm256_setzero_ps(), a1 = _mm256_setzero_ps(), a2 = _mm256_setzero_ps(), a3 = _mm256_setzero_ps();
  const __m128i low = _mm_set1_epi8(0x0F), eight = _mm_set1_epi8(8);
  int c = c0;
  for (; c + 32 <= c1; c += 32) {
    const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i *>(row + (c >> 1)));
    const __m128i lo = _mm_and_si128(b, low);                     // even columns
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(b, 4), low);  // odd columns
    const __m128i v0 = _mm_sub_epi8(_mm_unpacklo_epi8(lo, hi), eight);  // columns c .. c+15
    const __m128i v1 = _mm_sub_epi8(_mm_unpackhi_epi8(lo, hi), eight);  // columns c+16 .. c+31
    a0 = _mm256_fmadd_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v0)), _mm256_loadu_ps(x + c), a0);
    a1 = _mm256_fmadd_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v0, 8))), _mm256_loadu_ps(x + c + 8), a1);
    a2 = _mm256_fmadd_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(v1)), _mm256_loadu_ps(x + c + 16), a2);
    a3 = _mm256_fmadd_ps(_mm256_cvtepi32_ps(_mm256_cvtepi8_epi32(_mm_srli_si128(v1, 8))), _mm256_loadu_ps(x + c + 24), a3);
  }
  const __m256 a = _mm256_add_ps(_mm256_add_ps(a0, a1), _mm256_add_ps(a2, a3));
  alignas(32) float t[8];
  _mm256_store_ps(t, a);
  float s = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
  return s + (c < c1 ? nibble_dot(row, x, c, c1) : 0.f);
}

const bool kAvx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");

inline float span_dot(const uint8_t *row, const float *x, int c0, int c1) {
  return kAvx2 ? nibble_dot_avx2(row, x, c0, c1) : nibble_dot(row, x, c0, c1);
}

// One output row of an int4 tensor against x: per-row, the scale times the whole sum; group-wise,
// each group's sum times its scale, added group by group (the last group may be narrower).
inline float row_dot(const HostTensor &T, int o, const float *x) {
  const uint8_t *row = T.packed.data() + (size_t)o * (T.C / 2);
  if (T.ng == 1) return T.scales[o] * span_dot(row, x, 0, T.C);
  const float *s = T.scales.data() + (size_t)o * T.ng;
  float acc = 0.f;
  for (int g = 0; g < T.ng; ++g) {
    const int c0 = g * T.gs, c1 = c0 + T.gs < T.C ? c0 + T.gs : T.C;
    acc += s[g] * span_dot(row, x, c0, c1);
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
