// The CPU tier's arithmetic and worker pool (host code; see host_tier.h).
#include "host_tier.h"

#include <immintrin.h>

#include <chrono>
#include <cmath>
#include <cstdlib>
#include <cstring>

namespace i4moe {

HostPool::HostPool(int threads) {
  try {
    for (int i = 1; i < threads; ++i) workers_.emplace_back([this, i] { work(i); });
  } catch (...) {  // a thread that could not start: stop and join the ones that did
    {
      std::lock_guard<std::mutex> lk(m_);
      stop_.store(true);
    }
    go_.notify_all();
    for (auto &t : workers_) t.join();
    throw;
  }
}

HostPool::~HostPool() {
  {
    std::lock_guard<std::mutex> lk(m_);
    stop_.store(true);
  }
  go_.notify_all();
  for (auto &t : workers_) t.join();
}

void HostPool::work(int id) {
  unsigned seen = 0;
  for (;;) {
    // poll for a new run, then sleep: a worker counts itself in sleepers_ before it looks at
    // gen_ (and wake_) under the lock, and run() (warm()) bumps gen_ (wake_) before it looks at
    // sleepers_, so either the worker sees the change or it is woken; a warm() wake-up polls
    // for another kSpinMicros
    auto until = std::chrono::steady_clock::now() + std::chrono::microseconds(kSpinMicros);
    unsigned g;
    for (int i = 0;; ++i) {
      g = gen_.load();
      if (g != seen || stop_.load()) break;
      _mm_pause();
      if ((i & 255) == 255 && std::chrono::steady_clock::now() > until) {
        std::unique_lock<std::mutex> lk(m_);
        sleepers_.fetch_add(1);
        const unsigned w = wake_.load();
        go_.wait(lk, [&] { return stop_.load() || gen_.load() != seen || wake_.load() != w; });
        sleepers_.fetch_sub(1);
        until = std::chrono::steady_clock::now() + std::chrono::microseconds(kSpinMicros);
      }
    }
    if (stop_.load()) return;
    seen = g;
    const long T = threads();
    const long n = n_;
    try {
      (*fn_)(n * id / T, n * (id + 1) / T);
    } catch (...) {  // handed to run(), which rethrows it on the calling thread
      std::lock_guard<std::mutex> lk(m_);
      if (!error_) error_ = std::current_exception();
    }
    pending_.fetch_sub(1);
  }
}

void HostPool::warm() {
  wake_.fetch_add(1);  // before sleepers_ is read, as in run()
  if (sleepers_.load() > 0) {
    std::lock_guard<std::mutex> lk(m_);
    go_.notify_all();
  }
}

void HostPool::run(long n, const std::function<void(long, long)> &fn) {
  if (n <= 0) return;
  if (workers_.empty()) {
    fn(0, n);
    return;
  }
  fn_ = &fn;
  n_ = n;
  error_ = nullptr;
  pending_.store((int)workers_.size());
  gen_.fetch_add(1);  // publishes fn_ and n_ (sequentially consistent)
  if (sleepers_.load() > 0) {
    std::lock_guard<std::mutex> lk(m_);
    go_.notify_all();
  }
  std::exception_ptr mine;
  try {
    fn(0, n / threads());  // the calling thread takes range 0
  } catch (...) {
    mine = std::current_exception();
  }
  while (pending_.load() != 0) _mm_pause();
  if (mine) std::rethrow_exception(mine);
  if (error_) std::rethrow_exception(error_);
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

// ---- Integer path: int8 dot products of fixed-point activations (AVX-512 VNNI) -------------
//
// An activation row v of C columns in fixed point: X[c] = rint(v[c] 2^E), E chosen from the
// row's largest magnitude m (E = 148 - the biased exponent of m, so |X| <= 2^22), written as
// three balanced base-256 digits X = d0 + 256 d1 + 65536 d2 (each in [-128, 127]).  A weight
// nibble q stands for q - 8, so a row's group sum is
//   sum_c (q_c - 8) X_c = sum_n 256^n (sum_c q_c d_n[c] - 8 sum_c d_n[c]),
// every term an exact integer: vpdpbusd multiplies the unsigned nibbles by the signed digits,
// four products per int32 lane, and the second sum is the lanes' start value.  A 64-column
// block is 32 weight bytes: the low nibbles hold its even columns, the high nibbles its odd
// ones; int32 lane L of a block takes the columns 8 L .. 8 L + 7.  The digit rows are stored
// in superblocks of two blocks (the 64 weight bytes of one 512-bit load): for each digit, the
// even columns' digits of both blocks (2 x 32 bytes), then their odd columns' digits, so one
// 512-bit operand covers two blocks and one 256-bit operand one block.  The start values are
// laid out the same way: per superblock and digit, 8 lanes of each block.

constexpr int kBlockCols = 64;
constexpr int kPlanes = 3;
constexpr int kSuperBytes = 2 * kPlanes * kBlockCols;  // digit bytes per superblock
constexpr int kLanes = 8;                              // int32 lanes of a 256-bit register
constexpr int kLaneInts = kPlanes * kLanes;            // start values per block

struct DigitRow {
  int E = 0, nb = 0;         // nb blocks, stored as (nb + 1) / 2 superblocks
  std::vector<int8_t> dig;   // per superblock and digit: 64 even-column, then 64 odd-column digits
  std::vector<int32_t> neg;  // per superblock and digit: 2 x 8 lanes of -8 x (the lane's eight digits)
  std::vector<int32_t> pre;  // (nb + 1) x 3 x 8: the sums of each block's start values over the blocks before
};

// Offsets of block b's pieces: digit n's even (odd = 1: odd) columns, in bytes of dig, and its
// start values, in ints of neg.
inline size_t dig_at(int b, int n, int odd) {
  return (size_t)(b >> 1) * kSuperBytes + n * 2 * kBlockCols + odd * kBlockCols + (b & 1) * 32;
}
inline size_t neg_at(int b, int n) { return ((size_t)(b >> 1) * kPlanes + n) * 2 * kLanes + (b & 1) * kLanes; }

#define I4MOE_VNNI __attribute__((target("avx512f,avx512bw,avx512vl,avx512vnni,avx2,fma")))

// The digit row of v (C columns), vectorised over a block at a time.
I4MOE_VNNI void make_digit_row(const float *v, int C, DigitRow &r) {
  r.nb = (C + kBlockCols - 1) / kBlockCols;
  const int nsb = (r.nb + 1) / 2;
  r.dig.assign((size_t)nsb * kSuperBytes, 0);  // a missing second block of the last superblock stays zero
  r.neg.assign((size_t)nsb * 2 * kLaneInts, 0);
  r.pre.resize((size_t)(r.nb + 1) * kLaneInts);
  __m512 mx = _mm512_setzero_ps();
  for (int c = 0; c < C; c += 16) {
    const __mmask16 k = C - c >= 16 ? (__mmask16)0xffff : (__mmask16)((1u << (C - c)) - 1u);
    mx = _mm512_max_ps(mx, _mm512_abs_ps(_mm512_maskz_loadu_ps(k, v + c)));
  }
  const float m = _mm512_reduce_max_ps(mx);
  uint32_t mb;
  std::memcpy(&mb, &m, 4);
  r.E = 148 - (int)(mb >> 23);
  const __m512d scale = _mm512_set1_pd(std::ldexp(1.0, r.E));  // v 2^E is exact in double
  // columns 0, 2, .., 14 then 1, 3, .., 15 of 16
  const __m512i evens_odds = _mm512_setr_epi32(0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15);
  const __m512i bias = _mm512_set1_epi32(0x808080);
  const __m256i ones = _mm256_set1_epi8(1);
  int8_t *dig = r.dig.data();
  for (int b = 0; b < r.nb; ++b) {
    for (int i = 0; i < 4; ++i) {  // 16 columns at a time
      const int c = b * kBlockCols + 16 * i;
      const __mmask16 k = c >= C ? (__mmask16)0 : C - c >= 16 ? (__mmask16)0xffff : (__mmask16)((1u << (C - c)) - 1u);
      const __m512 f = _mm512_maskz_loadu_ps(k, v + (c < C ? c : 0));
      const __m256i x0 = _mm512_cvtpd_epi32(_mm512_mul_pd(_mm512_cvtps_pd(_mm512_castps512_ps256(f)), scale));
      const __m256i x1 = _mm512_cvtpd_epi32(
          _mm512_mul_pd(_mm512_cvtps_pd(_mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(f), 1))), scale));
      const __m512i X = _mm512_inserti64x4(_mm512_castsi256_si512(x0), x1, 1);  // round to nearest even
      const __m512i u = _mm512_permutexvar_epi32(evens_odds, _mm512_xor_si512(_mm512_add_epi32(X, bias), bias));
      for (int n = 0; n < kPlanes; ++n) {
        const __m128i d = _mm512_cvtepi32_epi8(_mm512_srli_epi32(u, 8 * n));  // 8 even, then 8 odd digits
        _mm_storel_epi64(reinterpret_cast<__m128i *>(dig + dig_at(b, n, 0) + 8 * i), d);
        _mm_storel_epi64(reinterpret_cast<__m128i *>(dig + dig_at(b, n, 1) + 8 * i), _mm_srli_si128(d, 8));
      }
    }
    for (int n = 0; n < kPlanes; ++n) {
      const __m256i e = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(dig + dig_at(b, n, 0)));
      const __m256i o = _mm256_loadu_si256(reinterpret_cast<const __m256i *>(dig + dig_at(b, n, 1)));
      const __m256i sum = _mm256_dpbusd_epi32(_mm256_dpbusd_epi32(_mm256_setzero_si256(), ones, e), ones, o);
      _mm256_storeu_si256(reinterpret_cast<__m256i *>(r.neg.data() + neg_at(b, n)),
                          _mm256_sub_epi32(_mm256_setzero_si256(), _mm256_slli_epi32(sum, 3)));
    }
  }
  std::fill(r.pre.begin(), r.pre.begin() + kLaneInts, 0);
  for (int b = 0; b < r.nb; ++b)
    for (int n = 0; n < kPlanes; ++n)
      for (int l = 0; l < kLanes; ++l)
        r.pre[((size_t)(b + 1) * kPlanes + n) * kLanes + l] =
            r.pre[((size_t)b * kPlanes + n) * kLanes + l] + r.neg[neg_at(b, n) + l];
}

// The integer path takes tensors whose groups are whole blocks (per-row, or gs a multiple of 64).
inline bool vnni_fits(const HostTensor &T) { return T.ng == 1 || T.gs % kBlockCols == 0; }

I4MOE_VNNI inline __m256i ld256(const void *p) { return _mm256_loadu_si256(reinterpret_cast<const __m256i *>(p)); }

// The 32 weight bytes of block b of a row of rb bytes (zero past the row's end).
I4MOE_VNNI inline __m256i weight_block(const uint8_t *row, int b, int rb) {
  const int rest = rb - 32 * b;
  return rest >= 32 ? _mm256_loadu_si256(reinterpret_cast<const __m256i *>(row + 32 * b))
                    : _mm256_maskz_loadu_epi8((__mmask32)((1u << rest) - 1u), row + 32 * b);
}

// Lanes a0 + 256 a1 + 65536 a2 in int32 (exact when the group is at most 256 columns wide:
// |lane| <= 32 x 8 x 2^22 = 2^30), times sc into the double lane sums.
I4MOE_VNNI inline void join_narrow(__m256i a0, __m256i a1, __m256i a2, double sc, __m256d &s0, __m256d &s1) {
  const __m256i j = _mm256_add_epi32(_mm256_add_epi32(a0, _mm256_slli_epi32(a1, 8)), _mm256_slli_epi32(a2, 16));
  const __m256d k = _mm256_set1_pd(sc);
  s0 = _mm256_fmadd_pd(_mm256_cvtepi32_pd(_mm256_castsi256_si128(j)), k, s0);
  s1 = _mm256_fmadd_pd(_mm256_cvtepi32_pd(_mm256_extracti128_si256(j, 1)), k, s1);
}

// The same join in double (any width: each digit sum is exact in int32 up to the column cap).
I4MOE_VNNI inline void join_wide(__m256i a0, __m256i a1, __m256i a2, double sc, __m256d &s0, __m256d &s1) {
  const __m256d k1 = _mm256_set1_pd(256.0), k2 = _mm256_set1_pd(65536.0), k = _mm256_set1_pd(sc);
  const __m256d lo = _mm256_fmadd_pd(_mm256_cvtepi32_pd(_mm256_castsi256_si128(a2)), k2,
                                     _mm256_fmadd_pd(_mm256_cvtepi32_pd(_mm256_castsi256_si128(a1)), k1,
                                                     _mm256_cvtepi32_pd(_mm256_castsi256_si128(a0))));
  const __m256d hi = _mm256_fmadd_pd(_mm256_cvtepi32_pd(_mm256_extracti128_si256(a2, 1)), k2,
                                     _mm256_fmadd_pd(_mm256_cvtepi32_pd(_mm256_extracti128_si256(a1, 1)), k1,
                                                     _mm256_cvtepi32_pd(_mm256_extracti128_si256(a0, 1))));
  s0 = _mm256_fmadd_pd(lo, k, s0);
  s1 = _mm256_fmadd_pd(hi, k, s1);
}

// One 64-column block of a g64 row against NR digit rows: the exact lanes of its group,
// rounded to float32, times the group's scale sc, into the float32 lane sums e.
template <int NR>
I4MOE_VNNI inline void g64_block(const uint8_t *row, int b, int rb, float sc, const int8_t *const (&dig)[NR],
                                 const int32_t *const (&neg)[NR], __m256 (&e)[NR]) {
  const __m256i low = _mm256_set1_epi8(0x0F);
  const __m256i w = weight_block(row, b, rb);
  const __m256i lo = _mm256_and_si256(w, low), hi = _mm256_and_si256(_mm256_srli_epi16(w, 4), low);
  const __m256 k = _mm256_set1_ps(sc);
  for (int r = 0; r < NR; ++r) {
    const __m256i a0 = _mm256_dpbusd_epi32(
        _mm256_dpbusd_epi32(ld256(neg[r] + neg_at(b, 0)), lo, ld256(dig[r] + dig_at(b, 0, 0))), hi,
        ld256(dig[r] + dig_at(b, 0, 1)));
    const __m256i a1 = _mm256_dpbusd_epi32(
        _mm256_dpbusd_epi32(ld256(neg[r] + neg_at(b, 1)), lo, ld256(dig[r] + dig_at(b, 1, 0))), hi,
        ld256(dig[r] + dig_at(b, 1, 1)));
    const __m256i a2 = _mm256_dpbusd_epi32(
        _mm256_dpbusd_epi32(ld256(neg[r] + neg_at(b, 2)), lo, ld256(dig[r] + dig_at(b, 2, 0))), hi,
        ld256(dig[r] + dig_at(b, 2, 1)));
    const __m256i j = _mm256_add_epi32(_mm256_add_epi32(a0, _mm256_slli_epi32(a1, 8)), _mm256_slli_epi32(a2, 16));
    e[r] = _mm256_fmadd_ps(_mm256_cvtepi32_ps(j), k, e[r]);
  }
}

// One output row of T against NR digit rows x[r] (each weight block loaded once for all of
// them), 256 bits at a time: per row, each group's exact integer lanes, times the group's scale,
// into lane sums (double; float32 for groups of 64 columns, even and odd blocks apart); the
// eight lanes added in a fixed order in double, times 2^-E.  Row r's result takes the same steps
// whatever NR is, so it does not depend on which rows share the call.
template <int NR>
I4MOE_VNNI inline void row_dots_256(const HostTensor &T, int o, const DigitRow *const *x, double *res) {
  const uint8_t *row = T.packed.data() + (size_t)o * (T.C / 2);
  const float *s = T.scales.data() + (size_t)o * T.ng;
  const int rb = T.C / 2, nb = x[0]->nb;
  const __m256i low = _mm256_set1_epi8(0x0F);
  const int8_t *dig[NR];
  const int32_t *neg[NR];
  const __m256i *pre[NR];
  __m256d s0[NR], s1[NR];
  for (int r = 0; r < NR; ++r) {
    dig[r] = x[r]->dig.data();
    neg[r] = x[r]->neg.data();
    pre[r] = reinterpret_cast<const __m256i *>(x[r]->pre.data());
    s0[r] = s1[r] = _mm256_setzero_pd();
  }
  if (T.ng == 1) {
    // one group over the row: per row six accumulators (digit x even/odd) carried across blocks
    __m256i a0[NR], a1[NR], a2[NR], b0[NR], b1[NR], b2[NR];
    for (int r = 0; r < NR; ++r) a0[r] = a1[r] = a2[r] = b0[r] = b1[r] = b2[r] = _mm256_setzero_si256();
    for (int b = 0; b < nb; ++b) {
      const __m256i w = weight_block(row, b, rb);
      const __m256i lo = _mm256_and_si256(w, low), hi = _mm256_and_si256(_mm256_srli_epi16(w, 4), low);
      for (int r = 0; r < NR; ++r) {
        a0[r] = _mm256_dpbusd_epi32(a0[r], lo, ld256(dig[r] + dig_at(b, 0, 0)));
        b0[r] = _mm256_dpbusd_epi32(b0[r], hi, ld256(dig[r] + dig_at(b, 0, 1)));
        a1[r] = _mm256_dpbusd_epi32(a1[r], lo, ld256(dig[r] + dig_at(b, 1, 0)));
        b1[r] = _mm256_dpbusd_epi32(b1[r], hi, ld256(dig[r] + dig_at(b, 1, 1)));
        a2[r] = _mm256_dpbusd_epi32(a2[r], lo, ld256(dig[r] + dig_at(b, 2, 0)));
        b2[r] = _mm256_dpbusd_epi32(b2[r], hi, ld256(dig[r] + dig_at(b, 2, 1)));
      }
    }
    for (int r = 0; r < NR; ++r) {
      const __m256i *p = pre[r] + kPlanes * nb;  // all blocks' start values
      join_wide(_mm256_add_epi32(_mm256_add_epi32(a0[r], b0[r]), _mm256_loadu_si256(p + 0)),
                _mm256_add_epi32(_mm256_add_epi32(a1[r], b1[r]), _mm256_loadu_si256(p + 1)),
                _mm256_add_epi32(_mm256_add_epi32(a2[r], b2[r]), _mm256_loadu_si256(p + 2)), (double)s[0], s0[r],
                s1[r]);
    }
  } else if (T.gs == kBlockCols) {
    // one block per group: each block's exact lanes rounded to float32, times its scale, into
    // float32 lane sums kept apart for the even and the odd blocks (the two halves of the
    // 512-bit form), joined lane by lane at the end
    __m256 e0[NR], e1[NR];
    for (int r = 0; r < NR; ++r) e0[r] = e1[r] = _mm256_setzero_ps();
    int b = 0;
    for (; b + 1 < nb; b += 2) {
      g64_block<NR>(row, b, rb, s[b], dig, neg, e0);
      g64_block<NR>(row, b + 1, rb, s[b + 1], dig, neg, e1);
    }
    if (b < nb) g64_block<NR>(row, b, rb, s[b], dig, neg, e0);
    for (int r = 0; r < NR; ++r) {
      const __m256 t = _mm256_add_ps(e0[r], e1[r]);
      s0[r] = _mm256_cvtps_pd(_mm256_castps256_ps128(t));
      s1[r] = _mm256_cvtps_pd(_mm256_extractf128_ps(t, 1));
    }
  } else {
    // groups of several blocks (the last one may be narrower)
    const int gb = T.gs / kBlockCols;
    for (int g = 0, g0 = 0; g0 < nb; ++g, g0 += gb) {
      const int g1 = g0 + gb < nb ? g0 + gb : nb;
      __m256i a0[NR], a1[NR], a2[NR];
      for (int r = 0; r < NR; ++r) {
        a0[r] = _mm256_sub_epi32(_mm256_loadu_si256(pre[r] + kPlanes * g1 + 0), _mm256_loadu_si256(pre[r] + kPlanes * g0 + 0));
        a1[r] = _mm256_sub_epi32(_mm256_loadu_si256(pre[r] + kPlanes * g1 + 1), _mm256_loadu_si256(pre[r] + kPlanes * g0 + 1));
        a2[r] = _mm256_sub_epi32(_mm256_loadu_si256(pre[r] + kPlanes * g1 + 2), _mm256_loadu_si256(pre[r] + kPlanes * g0 + 2));
      }
      for (int b = g0; b < g1; ++b) {
        const __m256i w = weight_block(row, b, rb);
        const __m256i lo = _mm256_and_si256(w, low), hi = _mm256_and_si256(_mm256_srli_epi16(w, 4), low);
        for (int r = 0; r < NR; ++r) {
          a0[r] = _mm256_dpbusd_epi32(_mm256_dpbusd_epi32(a0[r], lo, ld256(dig[r] + dig_at(b, 0, 0))), hi,
                                      ld256(dig[r] + dig_at(b, 0, 1)));
          a1[r] = _mm256_dpbusd_epi32(_mm256_dpbusd_epi32(a1[r], lo, ld256(dig[r] + dig_at(b, 1, 0))), hi,
                                      ld256(dig[r] + dig_at(b, 1, 1)));
          a2[r] = _mm256_dpbusd_epi32(_mm256_dpbusd_epi32(a2[r], lo, ld256(dig[r] + dig_at(b, 2, 0))), hi,
                                      ld256(dig[r] + dig_at(b, 2, 1)));
        }
      }
      for (int r = 0; r < NR; ++r) {
        if (gb <= 4)
          join_narrow(a0[r], a1[r], a2[r], (double)s[g], s0[r], s1[r]);
        else
          join_wide(a0[r], a1[r], a2[r], (double)s[g], s0[r], s1[r]);
      }
    }
  }
  for (int r = 0; r < NR; ++r) {
    alignas(32) double t[8];
    _mm256_store_pd(t, s0[r]);
    _mm256_store_pd(t + 4, s1[r]);
    const double total = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    res[r] = std::ldexp(total, -x[r]->E);
  }
}

inline const __m512i *at512(const void *p) { return reinterpret_cast<const __m512i *>(p); }

// The 64 weight bytes of superblock sb of a row of rb bytes (zero past the row's end).
I4MOE_VNNI inline __m512i weight_super(const uint8_t *row, int sb, int rb) {
  const int rest = rb - 64 * sb;
  return rest >= 64 ? _mm512_loadu_si512(row + 64 * sb)
                    : _mm512_maskz_loadu_epi8((__mmask64)((1ull << rest) - 1ull), row + 64 * sb);
}

// The two blocks' lanes of a 512-bit accumulator added lane by lane (exact in int32).
I4MOE_VNNI inline __m256i fold(__m512i a) {
  return _mm256_add_epi32(_mm512_castsi512_si256(a), _mm512_extracti64x4_epi64(a, 1));
}

// The same dot products as row_dots_256, two blocks per 512-bit instruction, for per-row tensors
// and group sizes 64 and multiples of 128 (a group never splits a superblock).  Every integer
// lane sum is exact and every double operation happens in the same order as in row_dots_256
// (a 64-column group's two blocks join one after the other), so the results are the same bits.
template <int NR>
I4MOE_VNNI inline void row_dots_512(const HostTensor &T, int o, const DigitRow *const *x, double *res) {
  const uint8_t *row = T.packed.data() + (size_t)o * (T.C / 2);
  const float *s = T.scales.data() + (size_t)o * T.ng;
  const int rb = T.C / 2, nb = x[0]->nb, nsb = (nb + 1) / 2;
  const __m512i low = _mm512_set1_epi8(0x0F);
  const int8_t *dig[NR];
  const int32_t *neg[NR];
  const __m256i *pre[NR];
  __m256d s0[NR], s1[NR];
  for (int r = 0; r < NR; ++r) {
    dig[r] = x[r]->dig.data();
    neg[r] = x[r]->neg.data();
    pre[r] = reinterpret_cast<const __m256i *>(x[r]->pre.data());
    s0[r] = s1[r] = _mm256_setzero_pd();
  }
  if (T.ng == 1) {
    __m512i a0[NR], a1[NR], a2[NR], b0[NR], b1[NR], b2[NR];
    for (int r = 0; r < NR; ++r) a0[r] = a1[r] = a2[r] = b0[r] = b1[r] = b2[r] = _mm512_setzero_si512();
    for (int sb = 0; sb < nsb; ++sb) {
      const __m512i w = weight_super(row, sb, rb);
      const __m512i lo = _mm512_and_si512(w, low), hi = _mm512_and_si512(_mm512_srli_epi16(w, 4), low);
      for (int r = 0; r < NR; ++r) {
        const int8_t *d = dig[r] + (size_t)sb * kSuperBytes;
        a0[r] = _mm512_dpbusd_epi32(a0[r], lo, _mm512_loadu_si512(d + 0));
        b0[r] = _mm512_dpbusd_epi32(b0[r], hi, _mm512_loadu_si512(d + 64));
        a1[r] = _mm512_dpbusd_epi32(a1[r], lo, _mm512_loadu_si512(d + 128));
        b1[r] = _mm512_dpbusd_epi32(b1[r], hi, _mm512_loadu_si512(d + 192));
        a2[r] = _mm512_dpbusd_epi32(a2[r], lo, _mm512_loadu_si512(d + 256));
        b2[r] = _mm512_dpbusd_epi32(b2[r], hi, _mm512_loadu_si512(d + 320));
      }
    }
    for (int r = 0; r < NR; ++r) {
      const __m256i *p = pre[r] + kPlanes * nb;
      join_wide(_mm256_add_epi32(_mm256_add_epi32(fold(a0[r]), fold(b0[r])), _mm256_loadu_si256(p + 0)),
                _mm256_add_epi32(_mm256_add_epi32(fold(a1[r]), fold(b1[r])), _mm256_loadu_si256(p + 1)),
                _mm256_add_epi32(_mm256_add_epi32(fold(a2[r]), fold(b2[r])), _mm256_loadu_si256(p + 2)), (double)s[0],
                s0[r], s1[r]);
    }
  } else if (T.gs == kBlockCols) {
    // lanes 0-7: the even block's lanes, 8-15: the odd block's, each with its own scale (the
    // 256-bit form's two float32 sums)
    __m512 e[NR];
    for (int r = 0; r < NR; ++r) e[r] = _mm512_setzero_ps();
    const __m512i halves = _mm512_setr_epi32(0, 0, 0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1, 1, 1, 1);
    for (int sb = 0; sb < nsb; ++sb) {
      const __m512i w = weight_super(row, sb, rb);
      const __m512i lo = _mm512_and_si512(w, low), hi = _mm512_and_si512(_mm512_srli_epi16(w, 4), low);
      const bool both = 2 * sb + 1 < nb;
      const __m512 sc = _mm512_permutexvar_ps(
          halves, _mm512_castps128_ps512(_mm_setr_ps(s[2 * sb], both ? s[2 * sb + 1] : 0.f, 0.f, 0.f)));
      for (int r = 0; r < NR; ++r) {
        const int8_t *d = dig[r] + (size_t)sb * kSuperBytes;
        const int32_t *z = neg[r] + (size_t)sb * 2 * kLaneInts;
        const __m512i a0 =
            _mm512_dpbusd_epi32(_mm512_dpbusd_epi32(_mm512_loadu_si512(z + 0), lo, _mm512_loadu_si512(d + 0)), hi,
                                _mm512_loadu_si512(d + 64));
        const __m512i a1 =
            _mm512_dpbusd_epi32(_mm512_dpbusd_epi32(_mm512_loadu_si512(z + 16), lo, _mm512_loadu_si512(d + 128)), hi,
                                _mm512_loadu_si512(d + 192));
        const __m512i a2 =
            _mm512_dpbusd_epi32(_mm512_dpbusd_epi32(_mm512_loadu_si512(z + 32), lo, _mm512_loadu_si512(d + 256)), hi,
                                _mm512_loadu_si512(d + 320));
        const __m512i j = _mm512_add_epi32(_mm512_add_epi32(a0, _mm512_slli_epi32(a1, 8)), _mm512_slli_epi32(a2, 16));
        const __m512 jf = _mm512_cvtepi32_ps(j);
        e[r] = both ? _mm512_fmadd_ps(jf, sc, e[r]) : _mm512_mask3_fmadd_ps(jf, sc, e[r], (__mmask16)0x00ff);
      }
    }
    for (int r = 0; r < NR; ++r) {
      const __m256 t = _mm256_add_ps(_mm512_castps512_ps256(e[r]),
                                     _mm256_castpd_ps(_mm512_extractf64x4_pd(_mm512_castps_pd(e[r]), 1)));
      s0[r] = _mm256_cvtps_pd(_mm256_castps256_ps128(t));
      s1[r] = _mm256_cvtps_pd(_mm256_extractf128_ps(t, 1));
    }
  } else {
    // groups of gs / 128 superblocks (the last one may be narrower)
    const int gsb = T.gs / (2 * kBlockCols), gb = T.gs / kBlockCols;
    for (int g = 0, g0 = 0; g0 < nsb; ++g, g0 += gsb) {
      const int g1 = g0 + gsb < nsb ? g0 + gsb : nsb;
      const int b0 = 2 * g0, b1 = 2 * g1 < nb ? 2 * g1 : nb;
      __m512i a0[NR], a1[NR], a2[NR];
      for (int r = 0; r < NR; ++r) a0[r] = a1[r] = a2[r] = _mm512_setzero_si512();
      for (int sb = g0; sb < g1; ++sb) {
        const __m512i w = weight_super(row, sb, rb);
        const __m512i lo = _mm512_and_si512(w, low), hi = _mm512_and_si512(_mm512_srli_epi16(w, 4), low);
        for (int r = 0; r < NR; ++r) {
          const int8_t *d = dig[r] + (size_t)sb * kSuperBytes;
          a0[r] = _mm512_dpbusd_epi32(_mm512_dpbusd_epi32(a0[r], lo, _mm512_loadu_si512(d + 0)), hi,
                                      _mm512_loadu_si512(d + 64));
          a1[r] = _mm512_dpbusd_epi32(_mm512_dpbusd_epi32(a1[r], lo, _mm512_loadu_si512(d + 128)), hi,
                                      _mm512_loadu_si512(d + 192));
          a2[r] = _mm512_dpbusd_epi32(_mm512_dpbusd_epi32(a2[r], lo, _mm512_loadu_si512(d + 256)), hi,
                                      _mm512_loadu_si512(d + 320));
        }
      }
      for (int r = 0; r < NR; ++r) {
        const __m256i c0 = _mm256_sub_epi32(_mm256_loadu_si256(pre[r] + kPlanes * b1 + 0), _mm256_loadu_si256(pre[r] + kPlanes * b0 + 0));
        const __m256i c1 = _mm256_sub_epi32(_mm256_loadu_si256(pre[r] + kPlanes * b1 + 1), _mm256_loadu_si256(pre[r] + kPlanes * b0 + 1));
        const __m256i c2 = _mm256_sub_epi32(_mm256_loadu_si256(pre[r] + kPlanes * b1 + 2), _mm256_loadu_si256(pre[r] + kPlanes * b0 + 2));
        const __m256i A0 = _mm256_add_epi32(c0, fold(a0[r])), A1 = _mm256_add_epi32(c1, fold(a1[r])),
                      A2 = _mm256_add_epi32(c2, fold(a2[r]));
        if (gb <= 4)
          join_narrow(A0, A1, A2, (double)s[g], s0[r], s1[r]);
        else
          join_wide(A0, A1, A2, (double)s[g], s0[r], s1[r]);
      }
    }
  }
  for (int r = 0; r < NR; ++r) {
    alignas(32) double t[8];
    _mm256_store_pd(t, s0[r]);
    _mm256_store_pd(t + 4, s1[r]);
    const double total = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    res[r] = std::ldexp(total, -x[r]->E);
  }
}

// The tensors the 512-bit form takes: groups never split a superblock.
inline bool fits_512(const HostTensor &T) { return T.ng == 1 || T.gs == kBlockCols || T.gs % (2 * kBlockCols) == 0; }

template <int NR>
I4MOE_VNNI inline void row_dots_vnni(const HostTensor &T, int o, const DigitRow *const *x, double *res, bool wide) {
  if (wide && fits_512(T))
    row_dots_512<NR>(T, o, x, res);
  else
    row_dots_256<NR>(T, o, x, res);
}

// The host rows of one expert, in route order.
struct HostEntry {
  const HostExpert *e;
  std::vector<int> rows;
};

constexpr int kMaxShare = 4;  // activation rows that share one pass over a weight row

// Gate, up and the SiLU-gated product of output o for the entry's rows rk[0 .. NR).
template <int NR>
I4MOE_VNNI void gate_up_rows(const HostEntry &en, const int *rk, int o, const std::vector<HostRow> &rows,
                             const std::vector<DigitRow> &xd, int I, float *h, bool wide) {
  const DigitRow *xs[NR];
  for (int r = 0; r < NR; ++r) xs[r] = &xd[rows[rk[r]].token];
  double g[NR], u[NR];
  row_dots_vnni<NR>(en.e->gate, o, xs, g, wide);
  row_dots_vnni<NR>(en.e->up, o, xs, u, wide);
  for (int r = 0; r < NR; ++r) {
    const float gf = (float)g[r], uf = (float)u[r];
    h[(size_t)rk[r] * I + o] = gf / (1.f + std::exp(-gf)) * uf;
  }
}

// Output d of the down projection for the entry's rows rk[0 .. NR).
template <int NR>
I4MOE_VNNI void down_rows(const HostEntry &en, const int *rk, int d, const std::vector<DigitRow> &hd, int D, float *y,
                          bool wide) {
  const DigitRow *hs[NR];
  for (int r = 0; r < NR; ++r) hs[r] = &hd[rk[r]];
  double v[NR];
  row_dots_vnni<NR>(en.e->down, d, hs, v, wide);
  for (int r = 0; r < NR; ++r) y[(size_t)rk[r] * D + d] = (float)v[r];
}

// Calls f(rk, nr) for the entry's rows in chunks of at most kMaxShare, in order.
template <class F>
inline void for_chunks(const HostEntry &en, F &&f) {
  const int n = (int)en.rows.size();
  for (int i = 0; i < n; i += kMaxShare) f(en.rows.data() + i, n - i < kMaxShare ? n - i : kMaxShare);
}

I4MOE_VNNI void gate_up_entry(const HostEntry &en, int o, const std::vector<HostRow> &rows,
                              const std::vector<DigitRow> &xd, int I, float *h, bool wide) {
  for_chunks(en, [&](const int *rk, int nr) {
    switch (nr) {
      case 1: gate_up_rows<1>(en, rk, o, rows, xd, I, h, wide); break;
      case 2: gate_up_rows<2>(en, rk, o, rows, xd, I, h, wide); break;
      case 3: gate_up_rows<3>(en, rk, o, rows, xd, I, h, wide); break;
      default: gate_up_rows<4>(en, rk, o, rows, xd, I, h, wide); break;
    }
  });
}

I4MOE_VNNI void down_entry(const HostEntry &en, int d, const std::vector<DigitRow> &hd, int D, float *y, bool wide) {
  for_chunks(en, [&](const int *rk, int nr) {
    switch (nr) {
      case 1: down_rows<1>(en, rk, d, hd, D, y, wide); break;
      case 2: down_rows<2>(en, rk, d, hd, D, y, wide); break;
      case 3: down_rows<3>(en, rk, d, hd, D, y, wide); break;
      default: down_rows<4>(en, rk, d, hd, D, y, wide); break;
    }
  });
}

// Work units: output o of entry i is rows(i) units, entries one after another (cum[i] units
// before entry i).  A worker's range [b, e) takes the outputs whose first unit lies in it, so
// the split follows the work and each output is computed by exactly one worker.
template <class F>
inline void for_outputs(const std::vector<HostEntry> &ent, const std::vector<long> &cum, int n_out, long b, long e,
                        F &&f) {
  size_t i = 0;
  while (i + 1 < ent.size() && cum[i + 1] <= b) ++i;
  for (; i < ent.size() && cum[i] < e; ++i) {
    const long R = (long)ent[i].rows.size();
    long o = b > cum[i] ? (b - cum[i] + R - 1) / R : 0;
    for (; o < n_out && cum[i] + o * R < e; ++o) f(ent[i], (int)o);
  }
}

const bool kVnni = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                   __builtin_cpu_supports("avx512vl") && __builtin_cpu_supports("avx512vnni") && kAvx2;

}  // namespace

bool host_int_path_available() {
  const char *env = std::getenv("I4MOE_HOST_INT");
  return kVnni && !(env && env[0] == '0' && env[1] == 0);
}

// I4MOE_HOST_INT=256 keeps the integer path at 256 bits.
static bool host_int_512() {
  const char *env = std::getenv("I4MOE_HOST_INT");
  return !(env && std::strcmp(env, "256") == 0);
}

void host_rows_forward(HostPool &pool, const std::vector<HostRow> &rows, const float *x, int D, int I, float *P) {
  const long n = (long)rows.size();
  if (n == 0) return;
  bool use_int = host_int_path_available();
  for (const HostRow &r : rows) use_int = use_int && vnni_fits(r.e->gate) && vnni_fits(r.e->up) && vnni_fits(r.e->down);
  std::vector<float> h((size_t)n * I), y((size_t)n * D);
  if (use_int) {
    const bool wide = host_int_512();
    // the rows grouped by expert (first appearance order), so that a weight row is read once
    // for all the rows of its expert
    std::vector<HostEntry> ent;
    for (long k = 0; k < n; ++k) {
      size_t i = 0;
      while (i < ent.size() && ent[i].e != rows[k].e) ++i;
      if (i == ent.size()) ent.push_back(HostEntry{rows[k].e, {}});
      ent[i].rows.push_back((int)k);
    }
    std::vector<long> cum_i(ent.size() + 1, 0), cum_d(ent.size() + 1, 0);
    for (size_t i = 0; i < ent.size(); ++i) {
      cum_i[i + 1] = cum_i[i] + (long)ent[i].rows.size() * I;
      cum_d[i + 1] = cum_d[i] + (long)ent[i].rows.size() * D;
    }
    // the digit rows of the tokens' x, then gate and up with the SiLU-gated product
    int S = 0;
    for (const HostRow &r : rows) S = r.token + 1 > S ? r.token + 1 : S;
    std::vector<char> used(S, 0);
    for (const HostRow &r : rows) used[r.token] = 1;
    std::vector<DigitRow> xd(S), hd(n);
    pool.run(S, [&](long b, long e) {
      for (long t = b; t < e; ++t)
        if (used[t]) make_digit_row(x + (size_t)t * D, D, xd[t]);
    });
    pool.run(cum_i.back(), [&](long b, long e) {
      for_outputs(ent, cum_i, I, b, e,
                  [&](const HostEntry &en, int o) { gate_up_entry(en, o, rows, xd, I, h.data(), wide); });
    });
    // the digit rows of h, then down
    pool.run(n, [&](long b, long e) {
      for (long k = b; k < e; ++k) make_digit_row(h.data() + (size_t)k * I, I, hd[k]);
    });
    pool.run(cum_d.back(), [&](long b, long e) {
      for_outputs(ent, cum_d, D, b, e, [&](const HostEntry &en, int d) { down_entry(en, d, hd, D, y.data(), wide); });
    });
  } else {
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
  }
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
