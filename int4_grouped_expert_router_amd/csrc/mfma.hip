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
// columns exactly in int32.  A group-wise tensor's three digit sums are joined into a float and
// scaled after every 64 columns (group sizes are multiples of 64); a per-row tensor keeps its
// integer sums to the end.  The result is (join) 2^-E / 16.
//
// Tiling: a workgroup owns 32 output rows x 16 rows of one entry (an expert's group rows, its
// token tile); its waves (up to 8, each with at least 8 steps of 64 columns) split the columns,
// and their partial results meet in LDS, summed in wave order.  Each wave keeps two steps of
// loads in flight.  MFMA operands: A = 16 activation rows x 64 columns (lane l: row l % 16, bytes of
// columns 16 (l / 16) .. +15 of the step), B = 64 columns x 16 weight rows (lane l: weight row
// l % 16, the same columns), so the 4 result dwords of lane l are rows 4 (l / 16) + v of the
// activation tile against weight row l % 16: one lane holds one weight row, and the row's scale
// is one value per lane.  Inside every 16 columns the bytes run in the order the nibble masks
// produce them (0 2 4 6 1 3 5 7, then 8 .. 15 likewise); the digit rows are written in that order.
#include <hip/hip_ext.h>

#include "common.h"

namespace i4moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDigits = 3;
constexpr int kMfmaWaves = 8;
constexpr int kNontemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

// ---- Digit rows ----------------------------------------------------------------------------

// One workgroup per activation row: E from the row's largest |a|, then 16 columns per thread
// and step, written as three 16-byte digit chunks in the byte order of the weight operand.
__global__ __launch_bounds__(kBlock) void k_digits8(DigitArgs a) {
  __shared__ uint32_t s_max[kBlock / kWave];
  const int row = blockIdx.x;
  if (a.grp && row >= ((CGroupBuf)a.grp)->g.n_rows) return;  // rows past the group: not used
  const int C = a.C;
  const size_t off = (size_t)row * a.act_ld;
  const uint16_t *xb = static_cast<const uint16_t *>(a.act) + off;
  const float *xf = static_cast<const float *>(a.act) + off;
  auto val = [&](int c) -> float {
    if (c >= C) return 0.f;
    return a.bf16 ? __uint_as_float((uint32_t)xb[c] << 16) : xf[c];
  };
  uint32_t m = 0;
  for (int c = threadIdx.x; c < C; c += kBlock) m = max(m, __float_as_uint(val(c)) & 0x7fffffffu);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int E = 148 - (int)(m >> 23);  // max |a| 2^E < 2^22 (a zero row: E = 148, zero digits)
  if (threadIdx.x == 0) a.E[row] = E;
  int8_t *dst = a.dig + (size_t)row * kDigits * a.C64;
  for (int b = threadIdx.x; b < a.C64 / 16; b += kBlock) {
    uint32_t d[kDigits][4] = {};
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      // byte p of the chunk holds column 16 b + col(p): within each half, even columns first
      const int h = p >> 3, r = p & 7;
      const int col = 16 * b + 8 * h + (r < 4 ? 2 * r : 2 * (r - 4) + 1);
      const int X = (int)__builtin_rintf(__builtin_ldexpf(val(col), E));
      const uint32_t u = ((uint32_t)X + 0x808080u) ^ 0x808080u;  // balanced digits as int8
#pragma unroll
      for (int n = 0; n < kDigits; ++n) d[n][p >> 2] |= ((u >> (8 * n)) & 0xffu) << (8 * (p & 3));
    }
#pragma unroll
    for (int n = 0; n < kDigits; ++n)
      *reinterpret_cast<u32x4 *>(dst + (size_t)n * a.C64 + 16 * b) = u32x4{d[n][0], d[n][1], d[n][2], d[n][3]};
  }
}

// ---- Matrix-core projection ----------------------------------------------------------------

// The int8 operand of 16 weight nibbles (two dwords, columns in nibble order): each nibble q
// masked into the high half of its byte is the int8 16 q.
__device__ __forceinline__ v4i weight_operand(uint32_t w0, uint32_t w1) {
  return v4i{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u), (int)((w1 << 4) & 0xF0F0F0F0u),
             (int)(w1 & 0xF0F0F0F0u)};
}

// sum_n acc[n] 256^n per element as a float (exact digit sums; two roundings).
__device__ __forceinline__ float join3(const v4i (&acc)[kDigits], int v) {
  return fmaf((float)acc[2][v], 65536.f, fmaf((float)acc[1][v], 256.f, (float)acc[0][v]));
}

constexpr int kWT = 2;  // weight tiles (16 rows each) per wave

constexpr int kWaveGroups = 16;  // scale groups of one wave's columns: at most 16 steps of 64

template <int NT>
struct MStep {
  uint32_t w[kWT][NT][2];
  v4i x[kDigits];
};

template <int NT>
__global__ __launch_bounds__(kMfmaWaves * kWave) void k_mfma(MfmaArgs a) {
  __shared__ float s_part[kMfmaWaves][kWT][NT][kWave * 4];
  __shared__ float s_scale[kMfmaWaves][kWT][NT][16][kWaveGroups];  // each wave's group scales
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KW = blockDim.x >> 6;  // waves splitting the columns
  // Logical tiles (entry slot, weight tile pair, token tile), token tile fastest; the blocks of
  // one XCD (block index mod 8) take one contiguous run of them, so the token tiles of a weight
  // tile re-read its weights from the same L2.
  const int L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (L >= a.tiles) return;
  const int tt = L % a.token_tiles;
  const int wt = (L / a.token_tiles) % a.weight_tiles;
  const int slot = L / (a.token_tiles * a.weight_tiles);

  // the slot-th entry with at least mfma_min rows
  const CGroupBuf G = (CGroupBuf)a.grp;
  const int ne = G->g.n_entries;
  const int r0 = lane < ne ? a.grp->g.entry_row0[lane] : 0;
  const int r1 = lane < ne ? a.grp->g.entry_row0[lane + 1] : 0;  // entry_row0[ne] = n_rows
  const bool big = lane < ne && r1 - r0 >= a.mfma_min;
  const unsigned long long bigs = __ballot(big);
  const unsigned long long pick = __ballot(big && __popcll(bigs & ((1ull << lane) - 1ull)) == slot);
  if (pick == 0) return;
  const int j = __ffsll((long long)pick) - 1;
  const int start = __builtin_amdgcn_readlane(r0, j);
  const int size = __builtin_amdgcn_readlane(r1, j) - start;
  if (16 * tt >= size) return;

  TensorDesc T[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const TensorDesc I4MOE_AS4 &d = G->rows[start].t[NT == 2 ? n : 2];
    T[n].q = d.q;
    T[n].s = d.s;
    T[n].row_bytes = d.row_bytes;
    T[n].gs = d.gs;
    T[n].ng = d.ng;
  }
  const int O = a.O;
  const int li = lane & 15, q = lane >> 4;

  // A operand rows: lane row li of the token tile; rows past the entry read zeros
  const int arow_g = min(start + 16 * tt + li, kRows - 1);
  const bool a_ok = 16 * tt + li < size;
  const int drow = a_ok ? (a.dual ? a.grp->rows[arow_g].token : arow_g) : 0;
  const __amdgpu_buffer_rsrc_t xr = rsrc(a.dig, a.dig_rows * kDigits * a.C64);
  const int xoff0 = a_ok ? drow * kDigits * a.C64 + 16 * q : -1;  // -1: no row

  // B operands: weight rows 16 (kWT wt + t) + li of each tensor; rows past O read zeros
  int orow[kWT];
  bool o_ok[kWT];
#pragma unroll
  for (int t = 0; t < kWT; ++t) {
    orow[t] = 16 * (kWT * wt + t) + li;
    o_ok[t] = orow[t] < O;
  }
  __amdgpu_buffer_rsrc_t wr[NT], sr[NT];
  bool grp[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    wr[n] = rsrc(T[n].q, O * T[n].row_bytes);
    sr[n] = rsrc(T[n].s, O * T[n].ng * 4);
    grp[n] = T[n].ng > 1;
  }

  const int KS = a.C64 / 64;
  const int s0 = (w * KS) / KW, s1 = ((w + 1) * KS) / KW;
  // Per-lane base offsets, fixed for the whole loop; a step adds a wave-uniform term, so the
  // loads carry no conditions (a row past O, or an activation row past the entry, gets a base
  // beyond its buffer and reads zeros).  A weight step reaching past a row's padded bytes reads
  // the next row's first bytes, but those columns (C and up) have zero digits; loads of steps
  // past this wave's range are issued and never used.
  constexpr int kFar = 0x40000000;
  int wbase[kWT][NT];
#pragma unroll
  for (int t = 0; t < kWT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      wbase[t][n] = o_ok[t] ? orow[t] * T[n].row_bytes + 8 * q : kFar;
    }
  // The group scales of this wave's columns, staged in the wave's own LDS region once (a step
  // then reads its scale there instead of issuing a load per row): lane (row li, quarter q) loads
  // groups g0 + 4q .. g0 + 4q + 3 of its row (past the row's scales: unused values).
  int g0[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) g0[n] = grp[n] ? (64 * s0) / T[n].gs : 0;
#pragma unroll
  for (int t = 0; t < kWT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int off = (o_ok[t] && grp[n]) ? 4 * (orow[t] * T[n].ng + g0[n] + 4 * q) : kFar;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(sr[n], off, 0, 0);
      *reinterpret_cast<u32x4 *>(&s_scale[w][t][n][li][4 * q]) = v;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int xbase = xoff0 >= 0 ? xoff0 : kFar;
  auto load = [&](MStep<NT> &st, int s) {
#pragma unroll
    for (int t = 0; t < kWT; ++t)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(wr[n], wbase[t][n] + 32 * s, 0, kNontemporal);
        st.w[t][n][0] = u.x;
        st.w[t][n][1] = u.y;
      }
#pragma unroll
    for (int d = 0; d < kDigits; ++d)
      st.x[d] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, xbase + d * a.C64 + 64 * s, 0, 0));
  };

  v4i acc[kWT][NT][kDigits];
  float F[kWT][NT][4];
  float srow[kWT][NT];  // a per-row tensor's row scale
#pragma unroll
  for (int t = 0; t < kWT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      srow[t][n] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(sr[n], o_ok[t] && !grp[n] ? 4 * orow[t] : 0x7ffffff0, 0, 0));
#pragma unroll
      for (int d = 0; d < kDigits; ++d) acc[t][n][d] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < 4; ++v) F[t][n][v] = 0.f;
    }
  auto compute = [&](const MStep<NT> &st, int s) {
#pragma unroll
    for (int t = 0; t < kWT; ++t)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const v4i B = weight_operand(st.w[t][n][0], st.w[t][n][1]);
#pragma unroll
        for (int d = 0; d < kDigits; ++d)
          acc[t][n][d] = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.x[d], B, acc[t][n][d], 0, 0, 0);
        if (grp[n]) {
          const float sc = s_scale[w][t][n][li][(64 * s) / T[n].gs - g0[n]];
#pragma unroll
          for (int v = 0; v < 4; ++v) F[t][n][v] = fmaf(join3(acc[t][n], v), sc, F[t][n][v]);
#pragma unroll
          for (int d = 0; d < kDigits; ++d) acc[t][n][d] = v4i{0, 0, 0, 0};
        }
      }
  };
  // two steps in flight: each step's registers are refilled with the step after next as soon as
  // it is consumed; the loop runs in pairs
  MStep<NT> b0, b1;
  load(b0, s0);
  load(b1, s0 + 1);
  for (int s = s0; s < s1; s += 2) {
    compute(b0, s);
    load(b0, s + 2);
    if (s + 1 < s1) compute(b1, s + 1);  // an odd last step
    load(b1, s + 3);
  }
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int t = 0; t < kWT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n)
      if (!grp[n])
#pragma unroll
        for (int v = 0; v < 4; ++v) F[t][n][v] = join3(acc[t][n], v) * srow[t][n];

#pragma unroll
  for (int t = 0; t < kWT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int v = 0; v < 4; ++v) s_part[w][t][n][lane * 4 + v] = F[t][n][v];
  __syncthreads();
  // one output per thread: weight tile t, lane l2 = i / 4 of the result layout, v = i % 4
  for (int i = threadIdx.x; i < kWT * kWave * 4; i += blockDim.x) {
    const int t = i / (kWave * 4), e = i % (kWave * 4);
    const int l2 = e >> 2, v = e & 3;
    const int m = 4 * (l2 >> 4) + v;               // row of the token tile
    const int o = 16 * (kWT * wt + t) + (l2 & 15);  // weight row
    if (16 * tt + m < size && o < O) {
      const int rg = start + 16 * tt + m;
      const int dr = a.dual ? a.grp->rows[rg].token : rg;
      const int E = a.E[dr];
      float sum[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        float acc_w = 0.f;
        for (int k = 0; k < KW; ++k) acc_w += s_part[k][t][n][e];
        sum[n] = __builtin_ldexpf(acc_w, -E - 4);
      }
      float res = sum[0];
      if constexpr (NT == 2) res = sum[0] / (1.f + expf(-sum[0])) * sum[1];
      a.out[(size_t)rg * a.out_ld + o] = res;
    }
  }
}

}  // namespace

hipError_t launch_digits8(const DigitArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (a.rows < 1 || a.rows > kRows || a.C < 1 || a.C64 % 64 != 0 || a.C64 < a.C || a.C64 > kMaxCols)
    return hipErrorInvalidValue;
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_digits8, dim3(a.rows), dim3(kBlock), 0, st, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_digits8, dim3(a.rows), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_mfma(int NT, MfmaArgs a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if ((NT != 1 && NT != 2) || a.mfma_min < 1 || a.C64 % 64 != 0 || a.C64 > kMaxCols || a.dig_rows < 1 ||
      a.dig_rows > kRows || a.slots < 0 || a.slots > kRows || a.token_tiles < 1 || a.token_tiles > kRows / 16)
    return hipErrorInvalidValue;
  a.weight_tiles = (a.O + 16 * kWT - 1) / (16 * kWT);
  a.tiles = a.slots * a.weight_tiles * a.token_tiles;
  if (a.tiles < 1) return hipSuccess;
  // waves splitting the columns: at least 8 steps of 64 columns each, at most kMfmaWaves
  const int KS = a.C64 / 64;
  int kw = KS / 8;
  kw = kw < 1 ? 1 : (kw > kMfmaWaves ? kMfmaWaves : kw);
  const int blocks = (a.tiles + 7) / 8 * 8;
  const void *k = NT == 2 ? reinterpret_cast<const void *>(&k_mfma<2>) : reinterpret_cast<const void *>(&k_mfma<1>);
  void *params[] = {&a};
  const hipError_t e = (t0 || t1) ? hipExtLaunchKernel(k, dim3(blocks), dim3(kw * kWave), params, 0, st, t0, t1, 0)
                                  : hipLaunchKernel(k, dim3(blocks), dim3(kw * kWave), params, 0, st);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace i4moe
