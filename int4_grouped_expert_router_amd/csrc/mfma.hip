// Grouped W4A16 projections on the matrix cores (gfx950) for experts with many rows in one issue
// (prefill, large batches): the variant the TC_W4A16 gating commit and the GPU-resident-pipeline
// commit of "Commit history of c/backend_cuda.cu" describe, where an expert with at least ~16
// rows in the group runs on tensor cores and smaller row counts keep the GEMV kernels.
//
// Arithmetic: exact integer products, as in the vector kernels.  Every activation row a (x, or h
// for the down projection) is written once per issue as 24-bit fixed point with one
// power-of-two scale per row, X_c = rint(a_c 2^E) with max |a_c| 2^E < 2^22, split into three
// balanced base-256 digits d_n in -128..127 (X = d_0 + 256 d_1 + 65536 d_2): three int8 "digit
// rows".  A weight nibble q (signed, -8..7) becomes the int8 16 q by masking it into the high half
// of its byte, so one v_mfma_i32_16x16x64_i8 per digit gives sum_k 16 q_k d_{n,k} over 64
// columns exactly in int32.  The three digit sums of every 64 columns are joined into a float
// and scaled (a group-wise tensor's group scale, group sizes being multiples of 64; a per-row
// tensor's row scale after the last step).  The result is (join) 2^-E / 16.
//
// Tiling: a workgroup of eight waves owns 64 weight rows x every 16-row token tile of one entry
// (an expert's group rows) x one slice of the columns; wave (w, h) takes weight tile w (16 rows)
// against token tiles 2 h and 2 h + 1, so each SIMD holds two waves of the stage.  The slices
// spread an entry over about two workgroups per CU.  Each stage (two steps of 64 columns: the
// weight rows and the digit rows) is loaded by the whole workgroup with 16-byte loads into LDS
// while the previous stage computes.  A slice's partial sums go to memory and a second launch
// adds the slices in slice order.  MFMA operands: A = 16 activation rows x 64 columns (lane l:
// row l % 16, bytes of columns 16 (l / 16) .. +15 of the step), B = 64 columns x 16 weight rows
// (lane l: weight row l % 16, the same columns), so the 4 result dwords of lane l are rows
// 4 (l / 16) + v of the activation tile against weight row l % 16: one lane holds one weight
// row, and the row's scale is one value per lane.  Inside every 16 columns the bytes run in the
// order the nibble masks produce them (0 2 4 6 1 3 5 7, then 8 .. 15 likewise); the digit rows
// are written in that order.
#include <hip/hip_ext.h>

#include "common.h"

namespace i4moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDigits = 3;
constexpr int kNontemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

// ---- Digit rows ----------------------------------------------------------------------------

// A row's exponent from the bits of its largest |a|: max |a| 2^E < 2^22 (a zero row: E = 148,
// zero digits).
__device__ __forceinline__ int row_exponent_bits(uint32_t m) { return 148 - (int)(m >> 23); }

// The three digit chunks of columns 16 b .. 16 b + 15 of a row (values v, zeros past its end)
// whose exponent is E, in the byte order of the weight operand, into the row's digit rows at dst
// (C64 bytes per digit).
__device__ __forceinline__ void store_digit_chunk(const float (&v)[16], int E, int8_t *dst, int C64, int b) {
  uint32_t d[kDigits][4] = {};
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    // byte p of the chunk holds column 16 b + col(p): within each half, even columns first
    const int h = p >> 3, r = p & 7;
    const int col = 8 * h + (r < 4 ? 2 * r : 2 * (r - 4) + 1);
    const int X = (int)__builtin_rintf(__builtin_ldexpf(v[col], E));
    const uint32_t u = ((uint32_t)X + 0x808080u) ^ 0x808080u;  // balanced digits as int8
#pragma unroll
    for (int n = 0; n < kDigits; ++n) d[n][p >> 2] |= ((u >> (8 * n)) & 0xffu) << (8 * (p & 3));
  }
#pragma unroll
  for (int n = 0; n < kDigits; ++n)
    *reinterpret_cast<u32x4 *>(dst + (size_t)n * C64 + 16 * b) = u32x4{d[n][0], d[n][1], d[n][2], d[n][3]};
}

// The largest of the workgroup's values (all threads; holds a workgroup barrier).
template <int NW>
__device__ __forceinline__ uint32_t block_max(uint32_t m, uint32_t (&s_max)[NW]) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = s_max[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) m = max(m, s_max[k]);
  return m;
}

// One workgroup per activation row: E from the row's largest |a|, then each thread's 16
// columns written as three 16-byte digit chunks in the byte order of the weight operand.
constexpr int kDigBlock = 1024;  // threads per activation row

__global__ __launch_bounds__(kDigBlock) void k_digits8(DigitArgs a) {
  __shared__ uint32_t s_max[kDigBlock / kWave];
  const int row = blockIdx.x;
  const int C = a.C;
  const size_t off = (size_t)row * a.act_ld;
  const uint16_t *xb = static_cast<const uint16_t *>(a.act) + off;
  const float *xf = static_cast<const float *>(a.act) + off;
  // 16 columns per thread and step: whole aligned 4-byte words (C and the row offset are even,
  // rows are 4-byte aligned), clamped into the row, zero past C
  auto load16 = [&](int b, float (&v)[16]) {
    const int c0 = 16 * b;
    if (a.bf16) {
      const uint32_t *w = reinterpret_cast<const uint32_t *>(xb);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = c0 + 2 * k;
        const uint32_t u = w[c < C ? c / 2 : 0];
        v[2 * k] = c < C ? __uint_as_float(u << 16) : 0.f;
        v[2 * k + 1] = c < C ? __uint_as_float(u & 0xffff0000u) : 0.f;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int c = c0 + k;
        const float x = xf[c < C ? c : 0];
        v[k] = c < C ? x : 0.f;
      }
    }
  };
  // one 16-column chunk per thread (C64 / 16 <= kMaxCols / 16 <= kDigBlock), loaded once
  static_assert(kMaxCols / 16 <= kDigBlock, "one chunk per thread");
  const int b = threadIdx.x;
  const bool has = b < a.C64 / 16;
  float v[16];
  load16(has ? b : 0, v);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) m = max(m, has ? __float_as_uint(v[k]) & 0x7fffffffu : 0u);
  const int E = row_exponent_bits(block_max(m, s_max));
  if (threadIdx.x == 0) a.E[row] = E;
  if (has) store_digit_chunk(v, E, a.dig + (size_t)row * kDigits * a.C64, a.C64, b);
}

// ---- Matrix-core projection ----------------------------------------------------------------

// The int8 operand of 16 weight nibbles (two dwords, columns in nibble order): each nibble q
// masked into the high half of its byte is the int8 16 q.
__device__ __forceinline__ v4i weight_operand(uint32_t w0, uint32_t w1) {
  return v4i{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u), (int)((w1 << 4) & 0xF0F0F0F0u),
             (int)(w1 & 0xF0F0F0F0u)};
}


// The slot-th entry of the group with at least mfma_min rows: its first row and row count
// (size 0: no such entry).  Wave-level; every lane gets the result.
__device__ __forceinline__ void big_entry(const GroupBuf *grp, int mfma_min, int slot, int lane, int &start, int &size) {
  const CGroupBuf G = (CGroupBuf)grp;
  const int ne = G->g.n_entries;
  const int r0 = lane < ne ? grp->g.entry_row0[lane] : 0;
  const int r1 = lane < ne ? grp->g.entry_row0[lane + 1] : 0;  // entry_row0[ne] = n_rows
  const bool big = lane < ne && r1 - r0 >= mfma_min;
  const unsigned long long bigs = __ballot(big);
  const unsigned long long pick = __ballot(big && __popcll(bigs & ((1ull << lane) - 1ull)) == slot);
  if (pick == 0) {
    start = size = 0;
    return;
  }
  const int j = __ffsll((long long)pick) - 1;
  start = __builtin_amdgcn_readlane(r0, j);
  size = __builtin_amdgcn_readlane(r1, j) - start;
}

// LDS stage: kCh steps of 64 columns.  Weight rows of 32 bytes per step, digit rows of 64 bytes
// per step and digit; rows padded so that the 16 rows one MFMA operand reads fall in distinct
// banks.
constexpr int kMW = 4;                       // weight tiles per workgroup (16 rows each)
constexpr int kMHalves = 2;                  // waves per weight tile: token tiles 0-1 and 2-3
constexpr int kMThreads = kMW * kMHalves * kWave;
constexpr int kMRows = 16 * kMW;             // weight rows per workgroup
constexpr int kCh = 2;                       // steps per stage
constexpr int kWRow = kCh * 32 + 8;          // LDS bytes per weight row
constexpr int kXRow = kDigits * kCh * 64 + 16;  // LDS bytes per activation row (3 digits)
constexpr int kXLoads = 64 * kDigits * kCh * 64 / 16 / kMThreads;  // 16-byte loads per thread
static_assert(kMRows * kCh * 32 / 16 * 2 == kMThreads, "one 16-byte weight load per thread (two tensors)");
static_assert(kXLoads * kMThreads * 16 == 64 * kDigits * kCh * 64, "digit rows split evenly");

template <int NT>
constexpr int stage_bytes() {
  return NT * kMRows * kWRow + 64 * kXRow + NT * kMRows * kCh * 4;
}
template <int NT>
constexpr size_t mfma_lds_bytes() {
  return 2 * (size_t)stage_bytes<NT>();
}

struct MLoads {
  u32x4 w;  // tensor tid / 256 (when there is one)
  u32x4 x[kXLoads];
  float sc;
};

// Matrix-core projection of one entry's rows: a workgroup owns kMRows weight rows x all token
// tiles of the entry x one slice of the columns; wave w owns weight tile w.  Each stage is loaded
// by the whole workgroup with 16-byte loads (a weight row's kCh x 32 bytes, a digit row's
// kCh x 64 bytes) while the previous stage computes.  The partial sums of the slice go to
// a.part[slice][n][slot][m][o]; k_mfma_h (dual) or k_mfma_reduce (down) adds the slices in order.
// ACC: every tensor of the launch is per-row, so each digit's sums accumulate in int32 over the
// whole slice (at most 2^20 per step, 2^27 over kMaxCols columns) and are joined once at the end.
template <int NT, bool ACC>
__global__ __launch_bounds__(kMThreads) void k_mfma(MfmaArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t s_lds[];
  __shared__ int s_drow[64];
  const int tid = threadIdx.x, lane = tid & 63;
  // wave: weight tile w, token tiles 2 th and 2 th + 1
  const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & (kMW - 1));
  const int th = __builtin_amdgcn_readfirstlane(tid >> 8);
  // blocks: (slot, weight block, column slice), slice fastest; one XCD takes a contiguous run,
  // so the slices of a weight block share an L2 for the digit rows
  const int L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (L >= a.tiles) return;
  const int ks = L % a.ksplit;
  const int wb = (L / a.ksplit) % a.weight_tiles;
  const int slot = L / (a.ksplit * a.weight_tiles);
  int start, size;
  big_entry(a.grp, a.mfma_min, slot, lane, start, size);
  if (size == 0) return;
  const int TT = (size + 15) >> 4;
  const CGroupBuf G = (CGroupBuf)a.grp;
  TensorDesc T[NT];
  bool grp[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const TensorDesc I4MOE_AS4 &d = G->rows[start].t[NT == 2 ? n : 2];
    T[n].q = d.q;
    T[n].s = d.s;
    T[n].row_bytes = d.row_bytes;
    T[n].gs = d.gs;
    T[n].ng = d.ng;
    grp[n] = T[n].ng > 1;
  }
  if (tid < 64) s_drow[tid] = tid < size ? (a.dual ? a.grp->rows[start + tid].token : start + tid) : -1;
  __syncthreads();

  const int O = a.O, o0 = kMRows * wb;
  const int KS = a.C64 / 64;
  const int k0 = (ks * KS) / a.ksplit, k1 = ((ks + 1) * KS) / a.ksplit;  // this slice's steps
  constexpr int kFar = 0x40000000;
  __amdgpu_buffer_rsrc_t wr[NT], sr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    wr[n] = rsrc(T[n].q, O * T[n].row_bytes + 64);
    sr[n] = rsrc(T[n].s, O * T[n].ng * 4);
  }
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.dig, a.dig_rows * kDigits * a.C64);
  // this thread's loads: tensor wn = tid / 256, weight row (tid % 256) / 4, 16-byte chunk tid % 4;
  // digit loads j: activation row m, digit d, chunk c of the stage's 128 bytes; one scale
  // (thread < NT x 128)
  const int wn = tid >> 8, wrow = (tid & 255) >> 2, wch = tid & 3;
  const bool w_ok = wn < NT && o0 + wrow < O;
  int xbase[kXLoads], xlds[kXLoads];
#pragma unroll
  for (int j = 0; j < kXLoads; ++j) {
    const int idx = tid + j * kMThreads;
    const int m = idx / (kDigits * kCh * 4), rem = idx % (kDigits * kCh * 4);
    const int d = rem / (kCh * 4), c = rem % (kCh * 4);
    const int dr = s_drow[m];
    xbase[j] = dr >= 0 ? (dr * kDigits + d) * a.C64 + 16 * c : kFar;
    xlds[j] = m * kXRow + d * (kCh * 64) + 16 * c;
  }
  // scale loads: tensor sn (wave-uniform: 128 threads per tensor), row srow, step sc_c of the stage
  const int sn = __builtin_amdgcn_readfirstlane(tid / (kMRows * kCh));
  const int srow = (tid / kCh) % kMRows, sc_c = tid % kCh;
  const int sn_c = sn < NT ? sn : 0;
  const bool s_ok = sn < NT && o0 + srow < O;
  auto load = [&](MLoads &r, int s0) {  // the stage starting at step s0
    {
      // a stage may reach up to 48 bytes past a row's padded end: the next row's first bytes (or
      // the tensor's 64-byte tail slack), multiplied by zero digits (columns C and up) or unused
      const bool second = NT == 2 && (wn & 1);  // no indexing of T by a runtime value (keeps it in registers)
      const int rb = second ? T[1 % NT].row_bytes : T[0].row_bytes;
      const int off = w_ok ? (o0 + wrow) * rb + 32 * s0 + 16 * wch : kFar;
      r.w = __builtin_amdgcn_raw_buffer_load_b128(second ? wr[1 % NT] : wr[0], off, 0, kNontemporal);
    }
#pragma unroll
    for (int j = 0; j < kXLoads; ++j)
      r.x[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, xbase[j] < kFar ? xbase[j] + 64 * s0 : kFar, 0, 0);
    if constexpr (!ACC) {
      const int gs = NT == 2 ? (sn_c ? T[1 % NT].gs : T[0].gs) : T[0].gs;
      const int ng = NT == 2 ? (sn_c ? T[1 % NT].ng : T[0].ng) : T[0].ng;
      const bool gg = ng > 1;
      const int g = gg ? (64 * (s0 + sc_c)) / gs : 0;
      const int soff = s_ok ? 4 * ((o0 + srow) * ng + g) : kFar;
      const __amdgpu_buffer_rsrc_t srs = NT == 2 ? (sn_c ? sr[1 % NT] : sr[0]) : sr[0];
      r.sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, soff, 0, 0));
    }
  };
  auto store = [&](const MLoads &r, int stage) {
    uint8_t *base = s_lds + stage * stage_bytes<NT>();
    if (wn < NT) *reinterpret_cast<u32x4 *>(base + wn * kMRows * kWRow + wrow * kWRow + 16 * wch) = r.w;
    uint8_t *xb = base + NT * kMRows * kWRow;
#pragma unroll
    for (int j = 0; j < kXLoads; ++j) *reinterpret_cast<u32x4 *>(xb + xlds[j]) = r.x[j];
    float *scb = reinterpret_cast<float *>(xb + 64 * kXRow);
    if (!ACC && sn < NT) scb[(sn * kMRows + srow) * kCh + sc_c] = r.sc;
  };

  // Every step's three digit products start from zero and are joined into F at once: the
  // step's scale (group-wise) or 1 (per-row, its row scale applied after the last step).  Low
  // digits first in int32 (|r| <= 2^20 per step, so r1 * 256 + r0 is exact), then one float.
  float F[2][NT][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 4; ++v) F[tt][n][v] = 0.f;
  // ACC: the digit sums of the slice, digit d of tensor n and token tile tt
  v4i I[ACC ? 2 : 1][NT][kDigits];
#pragma unroll
  for (int tt = 0; tt < (ACC ? 2 : 1); ++tt)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int d = 0; d < kDigits; ++d) I[tt][n][d] = v4i{0, 0, 0, 0};
  const int li = lane & 15, q = lane >> 4;
  // a per-row tensor's scale: one value per lane (its weight row)
  float srow_s[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int orow = o0 + 16 * w + li;
    srow_s[n] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(sr[n], (!grp[n] && orow < O) ? 4 * orow : kFar, 0, 0));
  }
  auto compute = [&](int stage, int nsteps, int s0) {
    const uint8_t *base = s_lds + stage * stage_bytes<NT>();
    const uint8_t *xb = base + NT * kMRows * kWRow;
    const float *scb = reinterpret_cast<const float *>(xb + 64 * kXRow);
#pragma unroll
    for (int cs = 0; cs < kCh; ++cs) {
      if (cs >= nsteps) break;
      v4i B[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x2 u = *reinterpret_cast<const u32x2 *>(base + n * kMRows * kWRow + (16 * w + li) * kWRow + cs * 32 + 8 * q);
        B[n] = weight_operand(u.x, u.y);
      }
      float sc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) sc[n] = (!ACC && grp[n]) ? scb[(n * kMRows + 16 * w + li) * kCh + cs] : 1.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if (2 * th + tt < TT) {
          v4i A[kDigits];
#pragma unroll
          for (int d = 0; d < kDigits; ++d)
            A[d] = *reinterpret_cast<const v4i *>(xb + (16 * (2 * th + tt) + li) * kXRow + d * (kCh * 64) + cs * 64 +
                                                  16 * q);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            if constexpr (ACC) {
#pragma unroll
              for (int d = 0; d < kDigits; ++d)
                I[tt][n][d] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[d], B[n], I[tt][n][d], 0, 0, 0);
            } else {
              v4i r[kDigits];
#pragma unroll
              for (int d = 0; d < kDigits; ++d)
                r[d] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[d], B[n], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int lo = (r[1][v] << 8) + r[0][v];
                F[tt][n][v] = fmaf(fmaf((float)r[2][v], 65536.f, (float)lo), sc[n], F[tt][n][v]);
              }
            }
          }
        }
      }
    }
  };

  // stages over this slice: load stage i + 1 while stage i computes
  MLoads r;
  if (k0 < k1) {
    load(r, k0);
    store(r, 0);
  }
  __syncthreads();
  int stage = 0;
  for (int s0 = k0; s0 < k1; s0 += kCh) {
    const bool more = s0 + kCh < k1;
    if (more) load(r, s0 + kCh);
    compute(stage, min(kCh, k1 - s0), s0);
    if (more) store(r, stage ^ 1);
    __syncthreads();
    stage ^= 1;
  }
  if constexpr (ACC) {
    // the slice's digit sums joined once (exactly, in double), one rounding to f32
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          F[tt][n][v] = (float)(((double)I[tt][n][2][v] * 65536.0 + (double)I[tt][n][1][v] * 256.0) +
                                (double)I[tt][n][0][v]);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
    if (ACC || !grp[n])
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) F[tt][n][v] *= srow_s[n];
  // partial sums of this slice: lane (li, q), element v = activation row 16 (2 th + tt) + 4 q + v,
  // weight row o0 + 16 w + li
  const int o = o0 + 16 * w + li;
  if (o < O) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = 16 * (2 * th + tt) + 4 * q + v;
          if (m < size)
            a.part[((((size_t)ks * NT + n) * a.slots + slot) * 64 + m) * O + o] = F[tt][n][v];
        }
  }
}

// Sum over the slices ks < ksplit (<= KB) of p[ks * stride], in slice order.  The KB loads are
// unconditional (slice indices clamped into the partials) so that all of them are in flight
// together; the slices past ksplit add +0, which leaves the sum's bits unchanged (a sum that
// starts at +0 is never -0).
constexpr int kMaxSlices = 32;
constexpr int kMfmaOneWgRows = 24;
template <int KB>
__device__ __forceinline__ float slice_sum(const float *p, size_t stride, int ksplit) {
  float v[KB];
#pragma unroll
  for (int k = 0; k < KB; ++k) v[k] = p[min(k, ksplit - 1) * stride];
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < KB; ++k) acc += k < ksplit ? v[k] : 0.f;
  return acc;
}

// The down projection's slice reduction: the slices' partial sums in slice order, then
// 2^(-E-4), into the entry's rows of y.  Grid: (column blocks of 256, activation row m < 64, slot).
template <int KB>
__global__ __launch_bounds__(kBlock) void k_mfma_reduce(MfmaArgs a) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.y, slot = blockIdx.z;
  int start, size;
  big_entry(a.grp, a.mfma_min, slot, lane, start, size);
  if (m >= size) return;
  const int o = blockIdx.x * kBlock + threadIdx.x;
  if (o >= a.O) return;
  const int rg = start + m;
  const float acc = slice_sum<KB>(a.part + ((size_t)slot * 64 + m) * a.O + o, (size_t)a.slots * 64 * a.O, a.ksplit);
  a.out[(size_t)rg * a.out_ld + o] = __builtin_ldexpf(acc, -a.E[rg] - 4);
}

// The dual projection's slice reduction fused with the digit rows of h, one workgroup per row m
// of a matrix-core entry: the slices' partial sums in slice order, 2^(-E-4) and SiLU(gate) x up
// into the entry's row of h, then the row's exponent from
// its largest |h| and its three digit rows (the arithmetic of k_digits8 on that row of h),
// indexed by group row, for the down projection.  Grid: (row m < 64, slot).
template <int KB>
__global__ __launch_bounds__(kDigBlock) void k_mfma_h(MfmaArgs a) {
  __shared__ float s_h[kMaxCols];
  __shared__ uint32_t s_max[kDigBlock / kWave];
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x, slot = blockIdx.y;
  int start, size;
  big_entry(a.grp, a.mfma_min, slot, lane, start, size);
  if (m >= size) return;
  const int O = a.O, O64 = (O + 63) & ~63;
  const int rg = start + m;
  const int E = a.E[a.grp->rows[rg].token];
  uint32_t mx = 0;
  for (int o = threadIdx.x; o < O64; o += kDigBlock) {
    float res = 0.f;
    if (o < O) {
      // gate and up partials of every slice in flight together (clamped slices add +0, as in
      // slice_sum)
      const size_t stride = (size_t)2 * a.slots * 64 * O;  // one slice
      const float *p0 = a.part + ((size_t)slot * 64 + m) * O + o;
      const float *p1 = p0 + (size_t)a.slots * 64 * O;
      float vg[KB], vu[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const size_t off = min(k, a.ksplit - 1) * stride;
        vg[k] = p0[off];
        vu[k] = p1[off];
      }
      float sum[2] = {0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        sum[0] += k < a.ksplit ? vg[k] : 0.f;
        sum[1] += k < a.ksplit ? vu[k] : 0.f;
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) sum[n] = __builtin_ldexpf(sum[n], -E - 4);
      res = sum[0] / (1.f + expf(-sum[0])) * sum[1];
      a.out[(size_t)rg * a.out_ld + o] = res;
    }
    s_h[o] = res;
    mx = max(mx, __float_as_uint(res) & 0x7fffffffu);
  }
  const int Eh = row_exponent_bits(block_max(mx, s_max));  // its barrier also publishes s_h
  if (threadIdx.x == 0) a.E_out[rg] = Eh;
  int8_t *dst = a.dig_out + (size_t)rg * kDigits * O64;
  for (int b = threadIdx.x; b < O64 / 16; b += kDigBlock) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = s_h[16 * b + k];
    store_digit_chunk(v, Eh, dst, O64, b);
  }
}

}  // namespace

hipError_t launch_digits8(const DigitArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (a.rows < 1 || a.rows > kRows || a.C < 1 || a.C64 % 64 != 0 || a.C64 < a.C || a.C64 > kMaxCols)
    return hipErrorInvalidValue;
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_digits8, dim3(a.rows), dim3(kDigBlock), 0, st, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_digits8, dim3(a.rows), dim3(kDigBlock), 0, st, a);
  return hipGetLastError();
}

size_t mfma_part_floats(int NT, int O, int slots, int ksplit) { return (size_t)ksplit * NT * slots * 64 * O; }

int mfma_ksplit(int O, int C64, int slots, int n_cu, int rows) {
  const int blocks = slots * ((O + kMRows - 1) / kMRows);
  const int KS = C64 / 64;
  // about two workgroups per CU; one for entries of 24 rows or more, whose stages carry two or
  // more token tiles (measured on the crossover shape: two per CU faster up to 20 rows, one from
  // 24 rows, 7-13% at 24-64 rows)
  const int per_cu = rows >= kMfmaOneWgRows ? 1 : 2;
  int k = (per_cu * n_cu + blocks - 1) / blocks;
  const int kmax = KS / (2 * kCh) > 0 ? KS / (2 * kCh) : 1;  // at least two stages per slice
  k = k < 1 ? 1 : (k > kmax ? kmax : k);
  return k > kMaxSlices ? kMaxSlices : k;
}

hipError_t launch_mfma(int NT, MfmaArgs a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if ((NT != 1 && NT != 2) || a.mfma_min < 1 || a.C64 % 64 != 0 || a.C64 > kMaxCols || a.dig_rows < 1 ||
      a.dig_rows > kRows || a.slots < 1 || a.slots > kRows || a.ksplit < 1 || a.ksplit > kMaxSlices || !a.part)
    return hipErrorInvalidValue;
  a.weight_tiles = (a.O + kMRows - 1) / kMRows;
  a.tiles = a.slots * a.weight_tiles * a.ksplit;
  const int blocks = (a.tiles + 7) / 8 * 8;
  static const void *const km[2][2] = {
      {reinterpret_cast<const void *>(&k_mfma<1, false>), reinterpret_cast<const void *>(&k_mfma<1, true>)},
      {reinterpret_cast<const void *>(&k_mfma<2, false>), reinterpret_cast<const void *>(&k_mfma<2, true>)}};
  const int acc = a.row_acc ? 1 : 0;
  const void *k = km[NT - 1][acc];
  const size_t lds = NT == 2 ? mfma_lds_bytes<2>() : mfma_lds_bytes<1>();
  static bool raised[2][2][kMaxDevices] = {};
  hipError_t e = raise_lds_once(k, (int)lds, raised[NT - 1][acc]);
  if (e != hipSuccess) return e;
  void *params[] = {&a};
  e = (t0) ? hipExtLaunchKernel(k, dim3(blocks), dim3(kMThreads), params, lds, st, t0, nullptr, 0)
           : hipLaunchKernel(k, dim3(blocks), dim3(kMThreads), params, lds, st);
  if (e != hipSuccess) return e;
  // the reduction, with as many slice loads in flight as the smallest power of two >= ksplit
  const int kb = a.ksplit <= 4 ? 0 : a.ksplit <= 8 ? 1 : a.ksplit <= 16 ? 2 : 3;
  if (NT == 2) {
    // the dual's reduction also writes the digit rows of h for the down projection
    if (!a.dig_out || !a.E_out || a.O > kMaxCols) return hipErrorInvalidValue;
    static const void *const kh[4] = {reinterpret_cast<const void *>(&k_mfma_h<4>),
                                      reinterpret_cast<const void *>(&k_mfma_h<8>),
                                      reinterpret_cast<const void *>(&k_mfma_h<16>),
                                      reinterpret_cast<const void *>(&k_mfma_h<32>)};
    const dim3 hg(64, a.slots);
    e = (t1) ? hipExtLaunchKernel(kh[kb], hg, dim3(kDigBlock), params, 0, st, nullptr, t1, 0)
             : hipLaunchKernel(kh[kb], hg, dim3(kDigBlock), params, 0, st);
  } else {
    static const void *const kr[4] = {reinterpret_cast<const void *>(&k_mfma_reduce<4>),
                                      reinterpret_cast<const void *>(&k_mfma_reduce<8>),
                                      reinterpret_cast<const void *>(&k_mfma_reduce<16>),
                                      reinterpret_cast<const void *>(&k_mfma_reduce<32>)};
    const dim3 rg((a.O + kBlock - 1) / kBlock, 64, a.slots);
    e = (t1) ? hipExtLaunchKernel(kr[kb], rg, dim3(kBlock), params, 0, st, nullptr, t1, 0)
             : hipLaunchKernel(kr[kb], rg, dim3(kBlock), params, 0, st);
  }
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace i4moe
