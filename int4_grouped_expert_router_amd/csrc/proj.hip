// Grouped W4A16 projections for decode (gfx950, wave64, no MFMA: at S<=4 every int4 weight
// feeds one to four products, so the launch is bound by the HBM weight stream).
//
//   dual : h[row][o] = silu(G_e[o,:] . x_t) * (U_e[o,:] . x_t)     (gate/up fused, SiLU fused)
//   down : y[row][o] = Dn_e[o,:] . h[row]
//
// for every group row (expert e, token t) and output row o.  Sources: the grouped
// dual/silu/down decode path of the TC_W4A16 gating commit and the group-wise kernels of the
// g4 commit ("Commit history of c/backend_cuda.cu"): nibbles are converted offset->signed at
// upload, the per-group scale is applied inside the accumulation, gs = 0 is per-row, and
// per-row and group-wise tensors run in one launch.
//
// Arithmetic: integer dot products.  The weights sit on the device as signed nibbles (q - 8 in
// two's complement, converted at upload).  The activation row a (x, or h for the down
// projection) is written as 24-bit fixed point with one power-of-two scale per row:
// X_c = rint(a_c * 2^E), with E chosen so that max |a_c| * 2^E < 2^22, and X_c is split into six
// balanced base-16 digits (each in -8..7, X = sum_n d_n 16^n).  Digit n of eight consecutive
// columns packs into one dword in the weight's own nibble order (a "digit plane"), so
// v_dot8_i32_i4 of a weight dword and a plane dword is sum_k (q_k - 8) d_{n,k}, exactly, and six
// of them give sum_k (q_k - 8) X_k: six instructions per eight weights, no unpacking.  Each
// lane adds its digit sums in integers, joins them into one float (one rounding), applies the
// row or group scale, and the lanes are summed in a fixed DPP order; the row's 2^-E comes out
// after that sum.  The only approximation is the rounding of a to 22-23 significant bits
// relative to the row's largest |a| (relative error <= 2^-22 of that largest value per element).
//
// Work decomposition.  One wavefront owns a tile of consecutive output rows of one group row.
// A row is covered by P passes of the whole wave; in pass p lane l owns V consecutive weight
// dwords (8V columns) starting at dword p*64*V + l*V, fetched with one V-dword load, so every
// pass of the wave reads 256*V contiguous bytes.  The workgroup stages the activation row's
// digit planes in LDS once; every pass reads the lane's planes (six V-dword LDS reads, shared
// by the step's rows and tensors).
//
// Kernels here:
//   k_proj<V, P, NT, GEN, SEL>   the dual (NT = 2) and long-row down (NT = 1) projections;
//                                SEL runs a one-token expert selection first (select.h)
//   k_rows16<P>                  down projection of short rows, 16 lanes per row
//   k_down_take<P>               down projection of short rows fused with the take (one token,
//                                one issue): the weighted, fixed-order sum of the rows is added to
//                                the residual in the same launch
#include <hip/hip_ext.h>

#include "select.h"

namespace i4moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPlanes = 6;                 // base-16 digits of the 24-bit fixed-point activations
constexpr uint32_t kDigitBias = 0x888888u; // sum_n 8 * 16^n: shifts every digit into 0..15

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over the 64 lanes in a fixed order; the total lands in lane 63 and is returned
// wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141, 0xF>(v);  // row_half_mirror
  v += dpp<0x140, 0xF>(v);  // row_mirror
  v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Largest value over the 64 lanes, returned wave-uniform (lanes a step does not reach keep
// their own value, and max with 0 leaves it unchanged).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1, 0xF>(v));
  v = max(v, dpp_u<0x4E, 0xF>(v));
  v = max(v, dpp_u<0x141, 0xF>(v));
  v = max(v, dpp_u<0x140, 0xF>(v));
  v = max(v, dpp_u<0x142, 0xA>(v));
  v = max(v, dpp_u<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ---- Activation digit planes --------------------------------------------------------------

// |a| as bits: for non-negative floats the integer order is the float order.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7fffffffu; }

// E for a row whose largest |a| has the bit pattern m: |a| < 2^(e - 126) for the biased exponent
// e = m >> 23, so max |a| * 2^E < 2^22 with E = 148 - e (a zero row gets E = 148 and all-zero
// digits).
__device__ __forceinline__ int row_exponent(uint32_t m) { return 148 - (int)(m >> 23); }

// The six digits of X = rint(a * 2^E), |X| <= 2^22, packed in nibbles 0..5: adding the bias turns
// the balanced digits d_n into d_n + 8 in 0..15, and the xor turns those into the digits' 4-bit
// two's-complement codes.
__device__ __forceinline__ uint32_t digits24(float a, int E) {
  const int X = (int)__builtin_rintf(__builtin_ldexpf(a, E));
  return ((uint32_t)X + kDigitBias) ^ kDigitBias;
}

// 8 x 8 nibble transpose: on return nibble k of z[n] is what nibble n of z[k] was.  Three block
// swaps: 4 x 4 blocks (bytes 2-3 of z[k] with bytes 0-1 of z[k+4]), 2 x 2 blocks inside those
// (byte pairs of z[k] and z[k+2]), then single nibbles (high nibbles of z[k] with low nibbles of
// z[k+1]).
__device__ __forceinline__ void nibble_transpose8(uint32_t (&z)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t a = z[k], b = z[k + 4];
    z[k] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    z[k + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = (i & 1) + 4 * (i >> 1);  // 0, 1, 4, 5
    const uint32_t a = z[k], b = z[k + 2];
    z[k] = __builtin_amdgcn_perm(b, a, 0x06020400u);
    z[k + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
  }
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    const uint32_t t = ((z[k] >> 4) ^ z[k + 1]) & 0x0F0F0F0Fu;
    z[k + 1] ^= t;
    z[k] ^= t << 4;
  }
}

// One digit-plane position: the eight columns 8j .. 8j+7 of the row, in a thread's registers.
// Loads are 4-byte (f32 columns, or bf16 column pairs), clamped into the row and unconditional,
// so their count never depends on the data; columns past C read as zero.
__device__ __forceinline__ void load_position(float (&v)[8], const void *act, int bf16, size_t row_off, int j,
                                              int positions, int C) {
  const bool ok = j < positions;
  if (bf16) {
    const uint32_t *row = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(act) + row_off);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 8 * j + 2 * k;  // C is even: a pair is whole or past the row
      const bool in = ok && c < C;
      const uint32_t u = row[in ? c / 2 : 0];
      v[2 * k] = in ? __uint_as_float(u << 16) : 0.f;
      v[2 * k + 1] = in ? __uint_as_float(u & 0xffff0000u) : 0.f;
    }
  } else {
    const float *row = static_cast<const float *>(act) + row_off;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = 8 * j + k;
      const bool in = ok && c < C;
      const float x = row[in ? c : 0];
      v[k] = in ? x : 0.f;
    }
  }
}

// The planes of one position from its eight values.
__device__ __forceinline__ void position_planes(uint32_t (&z)[8], const float (&v)[8], int E) {
#pragma unroll
  for (int k = 0; k < 8; ++k) z[k] = digits24(v[k], E);
  nibble_transpose8(z);
}

// Workgroup staging of one activation row as digit planes: planes[n * positions + j] holds digit
// n of columns 8j .. 8j+7 (zero past the row).  `v` holds the thread's positions
// j = threadIdx.x + m * kBlock, loaded earlier (load_position).  All threads of the workgroup
// call it; two barriers.  Returns E.
template <int NPOS>
__device__ __forceinline__ int stage_planes(uint32_t *planes, int positions, const float (&v)[NPOS][8],
                                            uint32_t *s_max) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NPOS; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, abs_bits(v[i][k]));
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int E = row_exponent(m);
#pragma unroll
  for (int i = 0; i < NPOS; ++i) {
    const int j = threadIdx.x + i * kBlock;
    if (j < positions) {
      uint32_t z[8];
      position_planes(z, v[i], E);
#pragma unroll
      for (int n = 0; n < kPlanes; ++n) planes[n * positions + j] = z[n];
    }
  }
  __syncthreads();
  return E;
}

// The lane's planes of one span: V dwords at position d0 of each plane.
template <int V>
__device__ __forceinline__ void read_planes(uint32_t (&X)[kPlanes][V], const uint32_t *planes, int positions, int d0) {
#pragma unroll
  for (int n = 0; n < kPlanes; ++n) {
    const uint32_t *p = planes + n * positions + d0;
    if constexpr (V == 4) {
      const u32x4 q = *reinterpret_cast<const u32x4 *>(p);
      X[n][0] = q.x; X[n][1] = q.y; X[n][2] = q.z; X[n][3] = q.w;
    } else if constexpr (V == 2) {
      const u32x2 q = *reinterpret_cast<const u32x2 *>(p);
      X[n][0] = q.x; X[n][1] = q.y;
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) X[n][v] = p[v];
    }
  }
}

// sum_n acc[n] * 16^n as a float with one rounding.  Each digit sum is at most 512 per weight
// dword in magnitude, so for up to 16 dwords per lane the two halves stay below 2^22 and convert
// exactly.
__device__ __forceinline__ float join_digits(const int (&acc)[kPlanes]) {
  const int hi = (acc[5] * 16 + acc[4]) * 16 + acc[3];
  const int lo = (acc[2] * 16 + acc[1]) * 16 + acc[0];
  return fmaf((float)hi, 4096.f, (float)lo);
}

// Signed value of nibble k of w.
__device__ __forceinline__ int nibble_s(uint32_t w, int k) { return ((int)(w << (28 - 4 * k))) >> 28; }

// Per-byte path for group sizes that split a lane's span (any even gs): each column's integer
// activation is rebuilt from the planes and takes its own group's scale.  Only odd layouts
// (gs not a multiple of 8) take it, so it is written for size, not speed: the column loop stays
// rolled.
__device__ __noinline__ float dword_dot_generic(const float *srow, int gs, int C, uint32_t w, const uint32_t *planes,
                                                int positions, int d) {
  uint32_t X[kPlanes];
#pragma unroll
  for (int n = 0; n < kPlanes; ++n) X[n] = planes[n * positions + d];
  float acc = 0.f;
#pragma unroll 1
  for (int k = 0; k < 8; ++k) {
    const int col = 8 * d + k;
    if (col < C) {
      int x = 0;
#pragma unroll
      for (int n = kPlanes - 1; n >= 0; --n) x = x * 16 + nibble_s(X[n], k);
      acc = fmaf(srow[col / gs], (float)(nibble_s(w, k) * x), acc);
    }
  }
  return acc;
}

template <int V, int P>
__device__ float row_dot_generic(const TensorDesc &T, int o, const uint32_t (&w)[P][V], const uint32_t *planes,
                                 int positions, int lane, int RD) {
  float acc = 0.f;
  const float *srow = T.s + (size_t)o * T.ng;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * 64 * V + lane * V;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (ds + v < RD) acc += dword_dot_generic(srow, T.gs, T.C, w[p][v], planes, positions, ds + v);
  }
  return acc;
}

// Field-wise copy out of the constant address space (scalar loads).
__device__ __forceinline__ TensorDesc ld_desc(const TensorDesc I4MOE_AS4 &d) {
  TensorDesc t;
  t.q = d.q;
  t.s = d.s;
  t.O = d.O;
  t.C = d.C;
  t.row_bytes = d.row_bytes;
  t.gs = d.gs;
  t.ng = d.ng;
  t.live = d.live;
  return t;
}

// Weights (and their scales) of one pipeline step: RB consecutive rows of NT tensors.
template <int V, int P, int NT, int RB>
struct Step {
  uint32_t w[NT][RB][P][V];
  float s[NT][RB][P];
};

// Raw buffer resource over [base, base + bytes): loads at offsets past the end return zero
// without a memory access.  Word 3 selects 32-bit data for untyped buffer loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

constexpr int kNontemporal = 2;  // cache-policy bits of a streaming load

template <int V>
__device__ __forceinline__ void load_span(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&w)[V]) {
  if constexpr (V == 4) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNontemporal);
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  } else if constexpr (V == 2) {
    const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNontemporal);
    w[0] = u.x; w[1] = u.y;
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) w[v] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * v, 0, kNontemporal);
  }
}

// Every load of a step is issued, whatever the tile: a row at or past o_end gets an empty
// buffer range, so its loads return zeros and touch no memory.  Keeping the issue pattern
// identical on every path keeps the wait counts exact (a load issued on one path only would
// make the compiler wait for all loads in flight).  A span past the row's padded bytes reads
// zeros the same way (weight 0).  One pass of a step: the pass-p spans (and scales) of its rows.
template <int V, int P, int NT, int RB>
__device__ __forceinline__ void load_pass(Step<V, P, NT, RB> &st, const TensorDesc (&T)[NT], const int (&gi)[NT][P],
                                          int o, int o_end, int lane, int p) {
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const bool ok = o + r < o_end;
    const int row = ok ? o + r : 0;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T[n].q + (size_t)row * T[n].row_bytes, ok ? T[n].row_bytes : 0);
      const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T[n].s + (size_t)row * T[n].ng, ok ? 4 * T[n].ng : 0);
      load_span<V>(wr, 4 * (p * 64 * V + lane * V), st.w[n][r][p]);
      st.s[n][r][p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * gi[n][p], 0, 0));
    }
  }
}

template <int V, int P, int NT, int RB>
__device__ __forceinline__ void load_step(Step<V, P, NT, RB> &st, const TensorDesc (&T)[NT], const int (&gi)[NT][P],
                                          int o, int o_end, int lane) {
#pragma unroll
  for (int p = 0; p < P; ++p) load_pass<V, P, NT, RB>(st, T, gi, o, o_end, lane, p);
}

// Dot products of one step's rows, reduced over the wave; lane (o - o_begin + r) keeps row
// o + r's result, and the tile's results leave in one coalesced store at the end.  Per pass the
// lane's planes are read once for every row and tensor of the step.  A group-wise tensor joins
// its digit sums and applies the span's group scale after every pass; a per-row tensor joins
// once, after the last pass, and applies the row scale.
//
// ROLL: as soon as a pass of the step is consumed, its registers are reloaded with the same pass
// of rows o_next .. (the step after next), so loads are issued throughout the computation rather
// than after it, and a wave always has close to two steps of weights in flight.
template <int V, int P, int NT, int RB, bool GEN, bool ROLL>
__device__ __forceinline__ void compute_step(Step<V, P, NT, RB> &st, const TensorDesc (&T)[NT], const int (&gi)[NT][P],
                                             const bool (&grp)[NT], const bool (&gen)[NT], const uint32_t *planes,
                                             int positions, int E, int o, int o_end, int lane, int RD, int o_begin,
                                             int o_next, float &outv) {
  int acc[NT][RB][kPlanes];
  float fa[NT][RB];
  float srow[NT][RB];  // per-row scales, kept before pass 0 is reloaded
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < RB; ++r) srow[n][r] = st.s[n][r][0];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      fa[n][r] = 0.f;
#pragma unroll
      for (int d = 0; d < kPlanes; ++d) acc[n][r][d] = 0;
    }
  // The planes of pass p + 1 are read while pass p computes; a scheduling barrier after each
  // pass keeps the compiler from hoisting every pass's reads to the top (which would hold all P
  // passes' planes in registers at once).
  uint32_t X[2][kPlanes][V];
  read_planes<V>(X[0], planes, positions, lane * V);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p + 1 < P) read_planes<V>(X[(p + 1) & 1], planes, positions, (p + 1) * 64 * V + lane * V);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (gen[n]) continue;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
#pragma unroll
          for (int d = 0; d < kPlanes; ++d)
            acc[n][r][d] = __builtin_amdgcn_sdot8((int)st.w[n][r][p][v], (int)X[p & 1][d][v], acc[n][r][d], false);
        }
        if (grp[n]) {
          fa[n][r] = fmaf(join_digits(acc[n][r]), st.s[n][r][p], fa[n][r]);
#pragma unroll
          for (int d = 0; d < kPlanes; ++d) acc[n][r][d] = 0;
        }
      }
    }
    if constexpr (ROLL) load_pass<V, P, NT, RB>(st, T, gi, o_next, o_end, lane, p);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float sum[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float a = fa[n][r];
      if (gen[n]) {
        if constexpr (GEN) {
          if (o + r < o_end) a = row_dot_generic<V, P>(T[n], o + r, st.w[n][r], planes, positions, lane, RD);
        }
      } else if (!grp[n]) {
        a = join_digits(acc[n][r]) * srow[n][r];
      }
      sum[n] = __builtin_ldexpf(wave_sum(a), -E);
    }
    float res = sum[0];
    if constexpr (NT == 2) res = sum[0] / (1.f + expf(-sum[0])) * sum[1];
    if (lane == o - o_begin + r) outv = res;
  }
}

// Positions (dwords) of the staged row for V-dword spans in P passes.
template <int V, int P>
constexpr int proj_positions() {
  return P * 64 * V;
}

// NT = 2: dual gate/up with the SiLU-gated product; NT = 1: down projection.  SEL (dual, one
// token, E <= 64): every workgroup first runs the expert selection itself from the router's
// finished scores, so no selection launch sits between the router GEMV and the experts;
// workgroup 0 publishes the route and group records, the first workgroup of each row that row's
// descriptor (for the down projection, the take and the taps).  A tile holds at most 64 rows
// (one result per lane).
template <int V, int P, int NT, bool GEN, bool SEL = false>
__global__ __launch_bounds__(kBlock) void k_proj(ProjArgs a) {
  constexpr int RB = rows_per_step(V, P, NT, 16);
  constexpr int POS = proj_positions<V, P>();
  constexpr int NPOS = (POS + kBlock - 1) / kBlock;
  extern __shared__ uint32_t s_planes[];  // [kPlanes][POS]
  __shared__ uint32_t s_max[kBlock / kWave];
  const int lane = threadIdx.x & 63;
  // Every workgroup works on one group row; its four waves take consecutive tiles.  The wave
  // index is uniform by construction and readfirstlane lets the compiler keep it (and the row,
  // tile, descriptors and base addresses derived from it) in scalar registers.
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int jr = blockIdx.x / a.tile_groups;  // < kRows: the grid never exceeds the row cap
  const int tile = (blockIdx.x - jr * a.tile_groups) * (kBlock / kWave) + wib;

  TensorDesc T[NT];
  int arow, live;
  uint32_t touch = 0;
  if constexpr (SEL) {
    static_assert(NT == 2, "selection runs in the dual projection");
    const RouteArgs &ra = a.ra;
    __shared__ double s_cw[kWavesPerBlock][kWave];
    __shared__ int s_cnt[kWavesPerBlock][kWave];
    __shared__ uint32_t s_tab[kTabPrefetchE * kDescWords];
    // one batch of loads: this lane's expert score, and in the first workgroup of each row
    // (which writes the row's descriptor) the expert records (E <= 64); the other workgroups
    // issue the same loads over an empty range, so nothing is read
    const bool writer = blockIdx.x == jr * a.tile_groups;
    const double2 cs = ra.score[min(lane, ra.E - 1)];
    uint32_t tv[kTabPerThread];
    table_prefetch_rsrc(tv, ra.table, writer ? ra.E * (int)sizeof(ExpertRec) : 0);
    const SelOne r = select_one(ra, cs, s_cw, s_cnt, [&] { table_stage(s_tab, tv); });
    // this row is selection jr of the one token, or (jr == n, with the shared expert) its row
    const bool shared_row = ra.shared_rows != 0 && jr == r.n;
    live = jr < r.n || shared_row ? 1 : 0;
    const int e = shared_row ? kSharedRec : __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(r.e_k, jr));
    const float w = shared_row ? 1.f : __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(r.w_k), jr));
    arow = 0;
    GroupBuf *out = ra.out;
    if (blockIdx.x == 0 && wib == 0) {
      // route record and group record of the token: its selections, one row each, in order
      // (and the shared expert's row after them)
      RouteTok *rt = out->route;
      const int n = r.n;
      const int nr = n + (ra.shared_rows != 0 ? 1 : 0);
      if (lane == 0) rt->n = n;
      rt->idx[lane] = lane < ra.K ? r.e_k : -1;
      rt->w[lane] = r.w_k;
      GroupDev *G = &out->g;
      if (lane < nr) {
        const int ge = lane < n ? r.e_k : kSharedRec;
        const float gw = lane < n ? r.w_k : 1.f;
        G->entry_expert[lane] = ge;
        G->entry_row0[lane] = lane;
        G->row_token[lane] = 0;
        G->row_expert[lane] = ge;
        G->row_weight[lane] = gw;
        G->red_rows[lane] = lane;
      }
      if (lane == 0) {
        G->entry_row0[nr] = nr;
        G->tok_row0[0] = 0;
        G->tok_row0[1] = nr;
        G->n_entries = nr;
        G->n_rows = nr;
        G->S = 1;
        G->reserved = 0;
      }
    }
    if (writer && wib == 0 && lane < kDescWords) {
      // this row's descriptor for the down projection and the take (zeros for a dead row)
      uint32_t val = 0u;
      if (live) {
        if (lane == kLiveWord || lane == kSizeWord)
          val = 1u;  // live; an entry of one row (rank 0)
        else if (lane == kRankWord)
          val = 0u;
        else if (lane < kTabWords)
          val = shared_row ? reinterpret_cast<const uint32_t *>(ra.table + e)[lane] : s_tab[e * kDescWords + lane];
        else if (lane == kTabWords)
          val = 0u;  // token
        else
          val = __float_as_uint(w);
      }
      reinterpret_cast<uint32_t *>(out->rows + jr)[lane] = val;
    }
    // the row's gate and up records: scalar loads of the (L2-resident) layer table
    typedef const ExpertRec I4MOE_AS4 *CExpertRec;
    const CExpertRec rec = (CExpertRec)ra.table + e;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      T[n] = ld_desc(rec->t[n]);
      T[n].live = live;
    }
    if (!live) return;
  } else {
    // Touch the first word of every row record of the grid, so the first workgroups to start
    // bring all records into their XCD's L2 before the weight stream fills the memory queues
    // (a later workgroup's record read then hits or joins a read already in flight).  The
    // value is consumed at the very end, so nothing waits for it.
    touch = reinterpret_cast<const uint32_t *>(a.grp->rows + min(lane, a.grid_rows - 1))[0];
    const CGroupBuf G = (CGroupBuf)a.grp;
    // Everything about this row in one scalar record: tensors, token, weight, and whether the
    // row belongs to the group (one memory round trip).
    if constexpr (NT == 2) {
      T[0] = ld_desc(G->rows[jr].t[0]);
      T[1] = ld_desc(G->rows[jr].t[1]);
    } else {
      T[0] = ld_desc(G->rows[jr].t[2]);
    }
    arow = NT == 2 ? G->rows[jr].token : jr;
    live = G->rows[jr].t[0].live;
    // Pin the record's loads above the liveness branch (otherwise they are sunk below it and
    // cost a second memory round trip).
#pragma unroll
    for (int n = 0; n < NT; ++n)
      asm volatile("" ::"s"(T[n].q), "s"(T[n].s), "s"(T[n].O), "s"(T[n].C), "s"(T[n].row_bytes), "s"(T[n].gs),
                   "s"(T[n].ng));
    asm volatile("" ::"s"(arow), "s"(live));
    if (!live) return;
  }

  const int C = a.C;
  const int RD = (C + 7) >> 3;
  int gi[NT][P];
  bool gen[NT], grp[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int p = 0; p < P; ++p) gi[n][p] = 0;
    grp[n] = T[n].ng > 1;
    if (grp[n]) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int ds = p * 64 * V + lane * V;
        gi[n][p] = ds < RD ? (8 * ds) / T[n].gs : 0;
      }
    }
    // GEN launches carry the per-byte path; others hold only tensors whose groups align with spans.
    gen[n] = GEN && grp[n] && (T[n].gs % (8 * V)) != 0;
  }

  const int o_begin = tile * a.tile_rows;
  const int o_end = min(o_begin + a.tile_rows, a.O);
  const bool work = o_begin < o_end;

  // Activation loads first, then the first two steps of weights (empty ranges for a wave
  // without rows); the digit planes are built once the activation loads have landed.
  // Scheduling barriers keep the issue order: the wait counts below assume it.
  float xv[NPOS][8];
#pragma unroll
  for (int i = 0; i < NPOS; ++i)
    load_position(xv[i], a.act, a.act_bf16, (size_t)arow * a.act_ld, threadIdx.x + i * kBlock, POS, C);
  __builtin_amdgcn_sched_barrier(0);
  Step<V, P, NT, RB> b0, b1;
  load_step<V, P, NT, RB>(b0, T, gi, o_begin, o_end, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_step<V, P, NT, RB>(b1, T, gi, o_begin + RB, o_end, lane);
  __builtin_amdgcn_sched_barrier(0);
  const int E = stage_planes<NPOS>(s_planes, POS, xv, s_max);
  if (!work) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // Two-stage pipeline: while one step computes, the other step's weights are in flight.  The
  // loop has one exit, at the bottom; the last pass issues loads of empty ranges.
  float outv = 0.f;
  int o = o_begin;
  do {
    if constexpr (!GEN) {
      // rolling reloads inside the computation; the second step runs even past the tile (its
      // rows read zeros and its results land on lanes that are never stored), so the issue
      // pattern never depends on the tile length
      compute_step<V, P, NT, RB, GEN, true>(b0, T, gi, grp, gen, s_planes, POS, E, o, o_end, lane, RD, o_begin,
                                            o + 2 * RB, outv);
      compute_step<V, P, NT, RB, GEN, true>(b1, T, gi, grp, gen, s_planes, POS, E, o + RB, o_end, lane, RD, o_begin,
                                            o + 3 * RB, outv);
    } else {
      // the per-byte path reads a step's weights after its last pass: reload afterwards
      compute_step<V, P, NT, RB, GEN, false>(b0, T, gi, grp, gen, s_planes, POS, E, o, o_end, lane, RD, o_begin, 0,
                                             outv);
      load_step<V, P, NT, RB>(b0, T, gi, o + 2 * RB, o_end, lane);
      if (o + RB < o_end)
        compute_step<V, P, NT, RB, GEN, false>(b1, T, gi, grp, gen, s_planes, POS, E, o + RB, o_end, lane, RD,
                                               o_begin, 0, outv);
      load_step<V, P, NT, RB>(b1, T, gi, o + 3 * RB, o_end, lane);
    }
    o += 2 * RB;
  } while (o < o_end);
  if (lane < o_end - o_begin) a.out[(size_t)jr * a.out_ld + o_begin + lane] = outv;
  asm volatile("" ::"v"(touch));
}

// ---- Several rows of one expert per weight pass (S > 1).  The rows of a group are ordered
// expert by expert, so an entry's rows are consecutive and split into chunks of up to entry_rows
// rows.  The nr workgroups of a chunk's rows all run every row of the chunk, each over its own
// nr-th of the output tile: every weight row is read once for the whole chunk (each load feeds
// nr dot products, one per staged activation row), and each workgroup does the work of one row
// over a whole tile, as in k_proj, so no workgroup runs longer than the others.  The row record
// carries the row's rank in its entry and the entry's size, so the chunk is known from the same
// scalar loads as the tensors.  Each lane joins its digit sums per pass and row (for a per-row
// tensor too; its scale is applied after the last pass).

// The chunk of a row with this rank in an entry of `size` rows: its row count nr (0 for an entry
// the matrix-core kernels take, at least mfma_min rows) and the row's index k in it.
struct ChunkPos {
  int nr, k;
};
__device__ __forceinline__ ChunkPos chunk_of(int rank, int size, int chunk, int mfma_min) {
  ChunkPos c;
  c.k = rank % chunk;
  c.nr = (mfma_min > 0 && size >= mfma_min) ? 0 : min(chunk, size - (rank - c.k));
  return c;
}

// Output rows [b, e) of sub-tile k of nr, inside the tile [t0, t1), in steps of RB rows.
__device__ __forceinline__ void sub_tile(int t0, int t1, int tile_rows, int nr, int k, int RB, int &b, int &e) {
  const int sub = ((tile_rows + nr - 1) / nr + RB - 1) / RB * RB;
  b = min(t0 + k * sub, t1);
  e = min(b + sub, t1);
}

template <int V, int P, int NT, int RB>
__device__ __forceinline__ void compute_step_entry(Step<V, P, NT, RB> &st, const TensorDesc (&T)[NT],
                                                   const int (&gi)[NT][P], const bool (&grp)[NT],
                                                   const uint32_t *planes, int positions, const int (&E)[kEntryRows],
                                                   int nr, int o, int o_end, int lane, int o_begin, int o_next,
                                                   float (&outv)[kEntryRows]) {
  float fa[NT][RB][kEntryRows];
  float srow[NT][RB];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      srow[n][r] = st.s[n][r][0];
#pragma unroll
      for (int i = 0; i < kEntryRows; ++i) fa[n][r][i] = 0.f;
    }
  // per pass, row by row: the row's planes, then its dot products (the guard on the chunk's
  // row count, uniform over the wave, also keeps the compiler from holding several rows' planes)
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int i = 0; i < kEntryRows; ++i) {
      if (i < nr) {
        uint32_t X[kPlanes][V];
        read_planes<V>(X, planes + i * kPlanes * positions, positions, p * 64 * V + lane * V);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            int acc[kPlanes];
#pragma unroll
            for (int d = 0; d < kPlanes; ++d) acc[d] = 0;
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
              for (int d = 0; d < kPlanes; ++d)
                acc[d] = __builtin_amdgcn_sdot8((int)st.w[n][r][p][v], (int)X[d][v], acc[d], false);
            const float jd = join_digits(acc);
            fa[n][r][i] = grp[n] ? fmaf(jd, st.s[n][r][p], fa[n][r][i]) : fa[n][r][i] + jd;
          }
      }
    }
    load_pass<V, P, NT, RB>(st, T, gi, o_next, o_end, lane, p);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int i = 0; i < kEntryRows; ++i) {
      if (i < nr) {
        float sum[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const float a = grp[n] ? fa[n][r][i] : fa[n][r][i] * srow[n][r];
          sum[n] = __builtin_ldexpf(wave_sum(a), -E[i]);
        }
        float res = sum[0];
        if constexpr (NT == 2) res = sum[0] / (1.f + expf(-sum[0])) * sum[1];
        if (lane == o - o_begin + r) outv[i] = res;
      }
    }
}

// k_proj for the chunks of entries (span-aligned group sizes only).  The staged rows arrive
// one after another: row i + 1's activation loads are in flight while row i is staged.
template <int V, int P, int NT>
__global__ __launch_bounds__(kBlock) void k_proj_entry(ProjArgs a) {
  constexpr int RB = rows_per_step(V, P, NT, 16);
  constexpr int POS = proj_positions<V, P>();
  constexpr int NPOS = (POS + kBlock - 1) / kBlock;
  extern __shared__ uint32_t s_planes[];  // [entry_rows][kPlanes][POS]
  __shared__ uint32_t s_max[kBlock / kWave];
  const int lane = threadIdx.x & 63;
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int jr = blockIdx.x / a.tile_groups;
  const int tile = (blockIdx.x - jr * a.tile_groups) * (kBlock / kWave) + wib;
  const CGroupBuf G = (CGroupBuf)a.grp;
  TensorDesc T[NT];
  if constexpr (NT == 2) {
    T[0] = ld_desc(G->rows[jr].t[0]);
    T[1] = ld_desc(G->rows[jr].t[1]);
  } else {
    T[0] = ld_desc(G->rows[jr].t[2]);
  }
  const int live = G->rows[jr].t[0].live;
  const int rank = G->rows[jr].t[1].live, size = G->rows[jr].t[2].live;
  // the tokens of rows jr - 3 .. jr + 3, the rows a chunk holding jr may span (dual)
  constexpr int kSpan = 2 * kEntryRows - 1;
  int tok[kSpan];
#pragma unroll
  for (int d = 0; d < kSpan; ++d)
    tok[d] = NT == 2 ? G->rows[min(max(jr + d - (kEntryRows - 1), 0), kRows - 1)].token : 0;
#pragma unroll
  for (int n = 0; n < NT; ++n)
    asm volatile("" ::"s"(T[n].q), "s"(T[n].s), "s"(T[n].O), "s"(T[n].C), "s"(T[n].row_bytes), "s"(T[n].gs),
                 "s"(T[n].ng));
  asm volatile("" ::"s"(live), "s"(rank), "s"(size));
#pragma unroll
  for (int d = 0; d < kSpan; ++d) asm volatile("" ::"s"(tok[d]));
  if (!live) return;
  const ChunkPos cp = chunk_of(rank, size, a.entry_rows, a.mfma_min);
  const int nr = cp.nr;
  if (nr == 0) return;
  const int head = jr - cp.k;  // the chunk's first row
  int arow[kEntryRows];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) {
    const int c = min(i, nr - 1);  // rows past the chunk repeat its last row
    if constexpr (NT == 2) {
      int t = tok[0];
#pragma unroll
      for (int d = 1; d < kSpan; ++d)
        if (d == c - cp.k + kEntryRows - 1) t = tok[d];
      arow[i] = t;
    } else {
      arow[i] = head + c;
    }
  }

  const int C = a.C;
  const int RD = (C + 7) >> 3;
  int gi[NT][P];
  bool grp[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    grp[n] = T[n].ng > 1;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int ds = p * 64 * V + lane * V;
      gi[n][p] = grp[n] && ds < RD ? (8 * ds) / T[n].gs : 0;
    }
  }
  int o_begin, o_end;
  sub_tile(tile * a.tile_rows, min(tile * a.tile_rows + a.tile_rows, a.O), a.tile_rows, nr, cp.k, RB, o_begin, o_end);
  const bool work = o_begin < o_end;

  float xv[2][NPOS][8];
#pragma unroll
  for (int k = 0; k < NPOS; ++k)
    load_position(xv[0][k], a.act, a.act_bf16, (size_t)arow[0] * a.act_ld, threadIdx.x + k * kBlock, POS, C);
  __builtin_amdgcn_sched_barrier(0);
  Step<V, P, NT, RB> b0, b1;
  load_step<V, P, NT, RB>(b0, T, gi, o_begin, o_end, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_step<V, P, NT, RB>(b1, T, gi, o_begin + RB, o_end, lane);
  __builtin_amdgcn_sched_barrier(0);
  int E[kEntryRows];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) {
    if (i + 1 < kEntryRows) {
#pragma unroll
      for (int k = 0; k < NPOS; ++k)
        load_position(xv[(i + 1) & 1][k], a.act, a.act_bf16, (size_t)arow[i + 1] * a.act_ld, threadIdx.x + k * kBlock,
                      POS, C);
    }
    __builtin_amdgcn_sched_barrier(0);
    E[i] = 0;
    if (i < nr) E[i] = stage_planes<NPOS>(s_planes + i * kPlanes * POS, POS, xv[i & 1], s_max);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!work) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  float outv[kEntryRows];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) outv[i] = 0.f;
  int o = o_begin;
  do {
    compute_step_entry<V, P, NT, RB>(b0, T, gi, grp, s_planes, POS, E, nr, o, o_end, lane, o_begin, o + 2 * RB, outv);
    compute_step_entry<V, P, NT, RB>(b1, T, gi, grp, s_planes, POS, E, nr, o + RB, o_end, lane, o_begin, o + 3 * RB,
                                     outv);
    o += 2 * RB;
  } while (o < o_end);
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i)
    if (i < nr && lane < o_end - o_begin) a.out[(size_t)(head + i) * a.out_ld + o_begin + lane] = outv[i];
}

// ---- Short rows (the down projection, C <= 2048 columns): 16 lanes per row, so one wave
// instruction covers four rows.  A row's dot product is then summed over 16 lanes (four DPP
// steps, all four rows at once) instead of 64, and no lane idles when a row is shorter than
// 64 lanes x 16 bytes.  Per-row or span-aligned (gs a multiple of 32) group scales.
constexpr int kLR = 16;                  // lanes per row
constexpr int kGR = kWave / kLR;         // rows per wave instruction

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141, 0xF>(v);  // row_half_mirror
  v += dpp<0x140, 0xF>(v);  // row_mirror: every lane of the 16 now holds the row's sum
  return v;
}

template <int P>
struct Step16 {
  uint32_t w[P][4];
  float s[P];
};

// One step: four consecutive rows o .. o+3, lane group g on row o + g.  The buffer ranges end
// at row o_end, so rows past the tile read zeros without a memory access; spans past the row
// get an offset past every range for the same effect.  One pass at a time.
template <int P>
__device__ __forceinline__ void load_pass16(Step16<P> &st, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                            const TensorDesc &T, const int (&woff)[P], const int (&gi)[P], int o, int g,
                                            int p) {
  const int row = o + g;
  load_span<4>(wr, woff[p] < 0 ? 0x7ffffff0 : row * T.row_bytes + woff[p], st.w[p]);
  st.s[p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * (row * T.ng + gi[p]), 0, 0));
}

template <int P>
__device__ __forceinline__ void load_step16(Step16<P> &st, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                            const TensorDesc &T, const int (&woff)[P], const int (&gi)[P], int o,
                                            int g) {
#pragma unroll
  for (int p = 0; p < P; ++p) load_pass16<P>(st, wr, sr, T, woff, gi, o, g, p);
}

// Positions of a short row staged for P passes of 16 lanes x 4 dwords.
template <int P>
constexpr int rows16_positions() {
  return P * kLR * 4;
}

// One step's four rows: the lane's digit sums over its P spans, joined (per pass for group-wise
// scales, once for a per-row scale), summed over the row's 16 lanes; lane (o - o_begin + g)
// keeps row o + g.
// After each pass its registers are reloaded with the same pass of rows o_next .. (the step
// after next), as in k_proj.
template <int P>
__device__ __forceinline__ void compute_step16(Step16<P> &st, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                               const TensorDesc &T, const int (&woff)[P], const int (&gi)[P],
                                               const uint32_t *planes, int li, int g, bool grp, int E, int o,
                                               int o_begin, int o_next, int lane, float &outv) {
  constexpr int POS = rows16_positions<P>();
  int acc[kPlanes];
#pragma unroll
  for (int d = 0; d < kPlanes; ++d) acc[d] = 0;
  float fa = 0.f;
  const float srow = st.s[0];
  uint32_t X[2][kPlanes][4];
  read_planes<4>(X[0], planes, POS, li * 4);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p + 1 < P) read_planes<4>(X[(p + 1) & 1], planes, POS, (p + 1) * kLR * 4 + li * 4);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int d = 0; d < kPlanes; ++d)
        acc[d] = __builtin_amdgcn_sdot8((int)st.w[p][v], (int)X[p & 1][d][v], acc[d], false);
    if (grp) {
      fa = fmaf(join_digits(acc), st.s[p], fa);
#pragma unroll
      for (int d = 0; d < kPlanes; ++d) acc[d] = 0;
    }
    load_pass16<P>(st, wr, sr, T, woff, gi, o_next, g, p);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!grp) fa = join_digits(acc) * srow;
  const float sum = __builtin_ldexpf(row16_sum(fa), -E);
#pragma unroll
  for (int g = 0; g < kGR; ++g) {
    const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), g * kLR));
    if (lane == o - o_begin + g) outv = r;
  }
}

template <int P>
__global__ __launch_bounds__(kBlock) void k_rows16(ProjArgs a) {
  constexpr int V = 4;
  constexpr int POS = rows16_positions<P>();
  static_assert(POS <= kBlock, "one staged position per thread");
  extern __shared__ uint32_t s_planes[];  // [kPlanes][POS]
  __shared__ uint32_t s_max[kBlock / kWave];
  const int lane = threadIdx.x & 63;
  const int li = lane & (kLR - 1), g = lane / kLR;
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t touch = reinterpret_cast<const uint32_t *>(a.grp->rows + min(lane, a.grid_rows - 1))[0];
  const CGroupBuf G = (CGroupBuf)a.grp;
  const int jr = blockIdx.x / a.tile_groups;
  const int tile = (blockIdx.x - jr * a.tile_groups) * (kBlock / kWave) + wib;
  const TensorDesc T = ld_desc(G->rows[jr].t[2]);
  const int live = G->rows[jr].t[0].live;
  asm volatile("" ::"s"(T.q), "s"(T.s), "s"(T.O), "s"(T.C), "s"(T.row_bytes), "s"(T.gs), "s"(T.ng));
  asm volatile("" ::"s"(live));
  if (!live) return;

  const int C = a.C;
  const int RD = (C + 7) >> 3;
  const bool grp = T.ng > 1;
  int gi[P], woff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * kLR * V + li * V;
    gi[p] = (grp && ds < RD) ? (8 * ds) / T.gs : 0;
    woff[p] = ds < RD ? 4 * ds : -1;
  }
  const int o_begin = tile * a.tile_rows;
  const int o_end = min(o_begin + a.tile_rows, a.O);
  const bool work = o_begin < o_end;
  const int rows_in = work ? o_end : 0;  // buffer ranges: rows [0, o_end) of this tensor
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T.q, rows_in * T.row_bytes);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T.s, rows_in * T.ng * 4);

  float xv[1][8];
  load_position(xv[0], a.act, 0, (size_t)jr * a.act_ld, threadIdx.x, POS, C);
  __builtin_amdgcn_sched_barrier(0);
  Step16<P> b0, b1;
  load_step16<P>(b0, wr, sr, T, woff, gi, o_begin, g);
  __builtin_amdgcn_sched_barrier(0);
  load_step16<P>(b1, wr, sr, T, woff, gi, o_begin + kGR, g);
  __builtin_amdgcn_sched_barrier(0);
  const int E = stage_planes<1>(s_planes, POS, xv, s_max);
  if (!work) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  float outv = 0.f;
  int o = o_begin;
  do {
    // the second step runs even past the tile (zeros in, results on lanes never stored)
    compute_step16<P>(b0, wr, sr, T, woff, gi, s_planes, li, g, grp, E, o, o_begin, o + 2 * kGR, lane, outv);
    compute_step16<P>(b1, wr, sr, T, woff, gi, s_planes, li, g, grp, E, o + kGR, o_begin, o + 3 * kGR, lane, outv);
    o += 2 * kGR;
  } while (o < o_end);
  if (lane < o_end - o_begin) a.out[(size_t)jr * a.out_ld + o_begin + lane] = outv;
  asm volatile("" ::"v"(touch));
}

// k_rows16 for the chunks of entries: the staged h rows of the chunk share every weight pass.
template <int P>
__device__ __forceinline__ void compute_step16_entry(Step16<P> &st, __amdgpu_buffer_rsrc_t wr,
                                                     __amdgpu_buffer_rsrc_t sr, const TensorDesc &T,
                                                     const int (&woff)[P], const int (&gi)[P], const uint32_t *planes,
                                                     int li, int g, bool grp, const int (&E)[kEntryRows], int nr, int o,
                                                     int o_begin, int o_next, int lane, float (&outv)[kEntryRows]) {
  constexpr int POS = rows16_positions<P>();
  float fa[kEntryRows];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) fa[i] = 0.f;
  const float srow = st.s[0];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int i = 0; i < kEntryRows; ++i) {
      if (i < nr) {
        uint32_t X[kPlanes][4];
        read_planes<4>(X, planes + i * kPlanes * POS, POS, p * kLR * 4 + li * 4);
        int acc[kPlanes];
#pragma unroll
        for (int d = 0; d < kPlanes; ++d) acc[d] = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int d = 0; d < kPlanes; ++d)
            acc[d] = __builtin_amdgcn_sdot8((int)st.w[p][v], (int)X[d][v], acc[d], false);
        const float jd = join_digits(acc);
        fa[i] = grp ? fmaf(jd, st.s[p], fa[i]) : fa[i] + jd;
      }
    }
    load_pass16<P>(st, wr, sr, T, woff, gi, o_next, g, p);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) {
    if (i < nr) {
      const float sum = __builtin_ldexpf(row16_sum(grp ? fa[i] : fa[i] * srow), -E[i]);
#pragma unroll
      for (int q = 0; q < kGR; ++q) {
        const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), q * kLR));
        if (lane == o - o_begin + q) outv[i] = r;
      }
    }
  }
}

template <int P>
__global__ __launch_bounds__(kBlock) void k_rows16_entry(ProjArgs a) {
  constexpr int V = 4;
  constexpr int POS = rows16_positions<P>();
  static_assert(POS <= kBlock, "one staged position per thread");
  extern __shared__ uint32_t s_planes[];  // [entry_rows][kPlanes][POS]
  __shared__ uint32_t s_max[kBlock / kWave];
  const int lane = threadIdx.x & 63;
  const int li = lane & (kLR - 1), g = lane / kLR;
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const CGroupBuf G = (CGroupBuf)a.grp;
  const int jr = blockIdx.x / a.tile_groups;
  const int tile = (blockIdx.x - jr * a.tile_groups) * (kBlock / kWave) + wib;
  const TensorDesc T = ld_desc(G->rows[jr].t[2]);
  const int live = G->rows[jr].t[0].live;
  const int rank = G->rows[jr].t[1].live, size = G->rows[jr].t[2].live;
  asm volatile("" ::"s"(T.q), "s"(T.s), "s"(T.O), "s"(T.C), "s"(T.row_bytes), "s"(T.gs), "s"(T.ng));
  asm volatile("" ::"s"(live), "s"(rank), "s"(size));
  if (!live) return;
  const ChunkPos cp = chunk_of(rank, size, a.entry_rows, a.mfma_min);
  const int nr = cp.nr;
  if (nr == 0) return;
  const int head = jr - cp.k;

  const int C = a.C;
  const int RD = (C + 7) >> 3;
  const bool grp = T.ng > 1;
  int gi[P], woff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * kLR * V + li * V;
    gi[p] = (grp && ds < RD) ? (8 * ds) / T.gs : 0;
    woff[p] = ds < RD ? 4 * ds : -1;
  }
  int o_begin, o_end;
  sub_tile(tile * a.tile_rows, min(tile * a.tile_rows + a.tile_rows, a.O), a.tile_rows, nr, cp.k, kGR, o_begin,
           o_end);
  const bool work = o_begin < o_end;
  const int rows_in = work ? o_end : 0;
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T.q, rows_in * T.row_bytes);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T.s, rows_in * T.ng * 4);

  // every row's position, loaded unconditionally (rows past the chunk repeat its last row)
  float xv[kEntryRows][1][8];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i)
    load_position(xv[i][0], a.act, 0, (size_t)(head + min(i, nr - 1)) * a.act_ld, threadIdx.x, POS, C);
  __builtin_amdgcn_sched_barrier(0);
  Step16<P> b0, b1;
  load_step16<P>(b0, wr, sr, T, woff, gi, o_begin, g);
  __builtin_amdgcn_sched_barrier(0);
  load_step16<P>(b1, wr, sr, T, woff, gi, o_begin + kGR, g);
  __builtin_amdgcn_sched_barrier(0);
  int E[kEntryRows];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) {
    E[i] = 0;
    if (i < nr) E[i] = stage_planes<1>(s_planes + i * kPlanes * POS, POS, xv[i], s_max);
  }
  if (!work) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  float outv[kEntryRows];
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i) outv[i] = 0.f;
  int o = o_begin;
  do {
    compute_step16_entry<P>(b0, wr, sr, T, woff, gi, s_planes, li, g, grp, E, nr, o, o_begin, o + 2 * kGR, lane, outv);
    compute_step16_entry<P>(b1, wr, sr, T, woff, gi, s_planes, li, g, grp, E, nr, o + kGR, o_begin, o + 3 * kGR, lane,
                            outv);
    o += 2 * kGR;
  } while (o < o_end);
#pragma unroll
  for (int i = 0; i < kEntryRows; ++i)
    if (i < nr && lane < o_end - o_begin) a.out[(size_t)(head + i) * a.out_ld + o_begin + lane] = outv[i];
}

const void *rows16_ptr(int P) {
  switch (P) {
    case 1: return reinterpret_cast<const void *>(&k_rows16<1>);
    case 2: return reinterpret_cast<const void *>(&k_rows16<2>);
    case 3: return reinterpret_cast<const void *>(&k_rows16<3>);
    case 4: return reinterpret_cast<const void *>(&k_rows16<4>);
    default: return nullptr;
  }
}

size_t rows16_lds_bytes(int P) { return 4u * kPlanes * (size_t)P * kLR * 4; }

// ---- Down projection and take in one launch (one token, one issue, at most kDTRows rows,
// short down rows).  A workgroup owns TL = 16 output columns of the residual and has one wave
// per group row: the wave stages its row's h as digit planes in its own LDS region (its own
// row scale, from a wave reduction) and computes its expert's TL outputs exactly as k_rows16
// does; the rows then meet in LDS and are summed in row (route) order with the take's
// arithmetic, fmaf over the live rows, added to the residual.  No y rows go through memory and
// no take launch follows.  (Measured on the medium decode layer: 8-column tiles double the h
// staging traffic and 32-column tiles leave half the CUs idle; both are slower.)
template <int P>
__global__ __launch_bounds__(kDTRows * kWave) void k_down_take(ProjArgs a) {
  // launched with one wave per group row (a.grid_rows <= kDTRows waves)
  constexpr int V = 4;
  constexpr int TL = kDTTile;
  constexpr int POS = rows16_positions<P>();
  constexpr int NX = POS / kWave;  // positions per lane
  static_assert(TL % (2 * kGR) == 0 && TL <= kWave, "whole pipeline passes, one output per lane");
  extern __shared__ uint32_t s_planes[];  // [kDTRows][kPlanes][POS]
  __shared__ float s_y[kDTRows][TL];
  __shared__ float s_w[kDTRows];
  __shared__ int s_live[kDTRows];
  const int lane = threadIdx.x & 63;
  const int li = lane & (kLR - 1), g = lane / kLR;
  const int r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // group row of this wave
  const int i0 = blockIdx.x * TL;
  const int i_end = min(i0 + TL, a.O);
  const CGroupBuf G = (CGroupBuf)a.grp;
  const int rr = min(r, a.grid_rows - 1);
  const TensorDesc T = ld_desc(G->rows[rr].t[2]);
  const int live = r < a.grid_rows ? G->rows[rr].t[0].live : 0;
  const float wr_row = G->rows[rr].weight;
  asm volatile("" ::"s"(T.q), "s"(T.s), "s"(T.O), "s"(T.C), "s"(T.row_bytes), "s"(T.gs), "s"(T.ng));
  asm volatile("" ::"s"(live));
  // the residual of the tile, in flight from the start
  const float r_in = a.out[min(i0 + (lane % TL), a.O - 1)];

  const int C = a.C;
  const int RD = (C + 7) >> 3;
  const bool grp = T.ng > 1;
  int gi[P], woff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * kLR * V + li * V;
    gi[p] = (grp && ds < RD) ? (8 * ds) / T.gs : 0;
    woff[p] = ds < RD ? 4 * ds : -1;
  }
  const int rows_in = live && i0 < a.O ? i_end : 0;  // a dead row's loads read nothing
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T.q, rows_in * T.row_bytes);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T.s, rows_in * T.ng * 4);

  // the wave's row of h: eight columns per position, NX positions per lane (clamped,
  // unconditional loads; rows are 16-byte aligned and padded to a multiple of 64 columns)
  const float *hrow = static_cast<const float *>(a.act) + (size_t)rr * a.act_ld;
  float xv[NX][8];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int j = lane + i * kWave;
    const float4 *src = reinterpret_cast<const float4 *>(hrow + (8 * j < C ? 8 * j : 0));
    const float4 u0 = src[0], u1 = src[1];
    xv[i][0] = u0.x; xv[i][1] = u0.y; xv[i][2] = u0.z; xv[i][3] = u0.w;
    xv[i][4] = u1.x; xv[i][5] = u1.y; xv[i][6] = u1.z; xv[i][7] = u1.w;
  }
  __builtin_amdgcn_sched_barrier(0);
  Step16<P> b0, b1;
  load_step16<P>(b0, wr, sr, T, woff, gi, i0, g);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t *planes = s_planes + r * (kPlanes * POS);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int j = lane + i * kWave;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (8 * j + k >= C) xv[i][k] = 0.f;  // the zeros of the row's padding (and the clamped reads)
      m = max(m, abs_bits(xv[i][k]));
    }
  }
  const int E = row_exponent(wave_max_u32(m));
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    uint32_t z[8];
    position_planes(z, xv[i], E);
#pragma unroll
    for (int n = 0; n < kPlanes; ++n) planes[n * POS + lane + i * kWave] = z[n];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the second step only now: a smaller first burst lands h and the first step sooner
  load_step16<P>(b1, wr, sr, T, woff, gi, i0 + kGR, g);
  __builtin_amdgcn_sched_barrier(0);

  float outv = 0.f;
  int o = i0;
  do {
    compute_step16<P>(b0, wr, sr, T, woff, gi, planes, li, g, grp, E, o, i0, o + 2 * kGR, lane, outv);
    compute_step16<P>(b1, wr, sr, T, woff, gi, planes, li, g, grp, E, o + kGR, i0, o + 3 * kGR, lane, outv);
    o += 2 * kGR;
  } while (o < i_end);
  if (lane < TL) s_y[r][lane] = outv;
  if (lane == 0) {
    s_w[r] = wr_row;
    s_live[r] = live;
  }
  __syncthreads();
  if (r == 0 && lane < TL && i0 + lane < a.O) {
    float acc = 0.f;
    for (int q = 0; q < a.grid_rows; ++q)
      if (s_live[q]) acc = fmaf(s_w[q], s_y[q][lane], acc);
    a.out[i0 + lane] = r_in + acc;
  }
}

const void *down_take_ptr(int P) {
  switch (P) {
    case 1: return reinterpret_cast<const void *>(&k_down_take<1>);
    case 2: return reinterpret_cast<const void *>(&k_down_take<2>);
    case 3: return reinterpret_cast<const void *>(&k_down_take<3>);
    case 4: return reinterpret_cast<const void *>(&k_down_take<4>);
    default: return nullptr;
  }
}

template <int NT, bool GEN, bool SEL = false>
const void *kernel_ptr_t(int V, int P) {
#define I4MOE_PTR(v, p) \
  if (V == v && P == p) return reinterpret_cast<const void *>(&k_proj<v, p, NT, GEN, SEL>);
  I4MOE_PTR(1, 1) I4MOE_PTR(1, 2) I4MOE_PTR(1, 3) I4MOE_PTR(1, 4)
  I4MOE_PTR(2, 1) I4MOE_PTR(2, 2) I4MOE_PTR(2, 3) I4MOE_PTR(2, 4)
  I4MOE_PTR(4, 1) I4MOE_PTR(4, 2) I4MOE_PTR(4, 3) I4MOE_PTR(4, 4)
#undef I4MOE_PTR
  return nullptr;
}

// The instantiation a launch uses.
const void *kernel_ptr(int V, int P, int NT, bool gen, bool sel = false) {
  if (NT == 1) return gen ? kernel_ptr_t<1, true>(V, P) : kernel_ptr_t<1, false>(V, P);
  if (gen) return sel ? nullptr : kernel_ptr_t<2, true>(V, P);
  return sel ? kernel_ptr_t<2, false, true>(V, P) : kernel_ptr_t<2, false>(V, P);
}

size_t lds_bytes(int V, int P) { return 4u * kPlanes * (size_t)P * 64 * V; }

template <int NT>
const void *entry_ptr_t(int V, int P) {
#define I4MOE_PTR(v, p) \
  if (V == v && P == p) return reinterpret_cast<const void *>(&k_proj_entry<v, p, NT>);
  I4MOE_PTR(1, 1) I4MOE_PTR(1, 2) I4MOE_PTR(1, 3) I4MOE_PTR(1, 4)
  I4MOE_PTR(2, 1) I4MOE_PTR(2, 2) I4MOE_PTR(2, 3) I4MOE_PTR(2, 4)
  I4MOE_PTR(4, 1) I4MOE_PTR(4, 2) I4MOE_PTR(4, 3) I4MOE_PTR(4, 4)
#undef I4MOE_PTR
  return nullptr;
}

const void *rows16_entry_ptr(int P) {
  switch (P) {
    case 1: return reinterpret_cast<const void *>(&k_rows16_entry<1>);
    case 2: return reinterpret_cast<const void *>(&k_rows16_entry<2>);
    case 3: return reinterpret_cast<const void *>(&k_rows16_entry<3>);
    case 4: return reinterpret_cast<const void *>(&k_rows16_entry<4>);
    default: return nullptr;
  }
}

// Dynamic LDS beyond 48 KB needs the kernel's limit raised (once per kernel and device).
hipError_t raise_lds(const void *k, size_t lds) {
  if (lds <= 48 * 1024) return hipSuccess;
  constexpr int kKeys = 64;
  static const void *keys[kKeys];
  static bool done[kKeys][kMaxDevices];
  static int nk = 0;
  int i = 0;
  while (i < nk && keys[i] != k) ++i;
  if (i == nk) {
    if (nk == kKeys) return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    keys[nk++] = k;
  }
  return raise_lds_once(k, (int)lds, done[i]);
}

hipError_t launch(int V, int P, int NT, bool gen, bool sel, const ProjArgs &a, int blocks, hipStream_t st,
                  hipEvent_t t0, hipEvent_t t1) {
  const bool entry = a.entry_rows > 0;
  if (entry && (gen || sel || a.entry_rows > kEntryRows)) return hipErrorInvalidValue;
  const void *k = entry ? (NT == 2 ? entry_ptr_t<2>(V, P) : entry_ptr_t<1>(V, P)) : kernel_ptr(V, P, NT, gen, sel);
  if (!k) return hipErrorInvalidValue;
  ProjArgs args = a;
  void *params[] = {&args};
  const size_t lds = lds_bytes(V, P) * (entry ? a.entry_rows : 1);
  const hipError_t e = raise_lds(k, lds);
  if (e != hipSuccess) return e;
  if (t0 || t1) return hipExtLaunchKernel(k, dim3(blocks), dim3(kBlock), params, lds, st, t0, t1, 0);
  return hipLaunchKernel(k, dim3(blocks), dim3(kBlock), params, lds, st);
}

}  // namespace

int proj_blocks_per_cu(int V, int P, int NT, bool gen) {
  static int cache[5][5][3][2] = {};
  if (V < 1 || V > 4 || V == 3 || P < 1 || P > 4 || NT < 1 || NT > 2) return 1;
  int &c = cache[V][P][NT][gen ? 1 : 0];
  if (c == 0) {
    const void *k = kernel_ptr(V, P, NT, gen);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kBlock, lds_bytes(V, P)) != hipSuccess || n < 1) {
      (void)hipGetLastError();
      n = 1;
    }
    c = n;
  }
  return c;
}

bool dual_sel_ok(const RouteArgs &ra, bool gen) {
  return !gen && ra.S == 1 && ra.E <= kTabPrefetchE && ra.table != nullptr && ra.K <= kRows;
}

hipError_t launch_dual(int V, int P, bool gen, bool sel, const ProjArgs &a, int blocks, hipStream_t st, hipEvent_t t0,
                       hipEvent_t t1) {
  if (sel && !dual_sel_ok(a.ra, gen)) return hipErrorInvalidValue;
  hipError_t e = launch(V, P, 2, gen, sel, a, blocks, st, t0, t1);
  return e != hipSuccess ? e : hipGetLastError();
}

int entry_rows_fit(int V, int P, bool rows16, int want) {
  // keep three workgroups' staged rows within a CU's 160 KB of LDS
  constexpr size_t kBudget = 160 * 1024 / 3;
  const size_t per_row = rows16 ? rows16_lds_bytes(P) : lds_bytes(V, P);
  int n = (int)(kBudget / per_row);
  n = n < 1 ? 1 : n;
  n = n < want ? n : want;
  return n < kEntryRows ? n : kEntryRows;
}

int rows16_blocks_per_cu(int P) {
  static int cache[5] = {};
  if (P < 1 || P > 4) return 1;
  if (cache[P] == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rows16_ptr(P), kBlock, rows16_lds_bytes(P)) != hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      n = 1;
    }
    cache[P] = n;
  }
  return cache[P];
}

hipError_t launch_down16(int P, const ProjArgs &a, int blocks, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  const bool entry = a.entry_rows > 0;
  if (a.entry_rows > kEntryRows) return hipErrorInvalidValue;
  const void *k = entry ? rows16_entry_ptr(P) : rows16_ptr(P);
  if (!k) return hipErrorInvalidValue;
  ProjArgs args = a;
  void *params[] = {&args};
  const size_t lds = rows16_lds_bytes(P) * (entry ? a.entry_rows : 1);
  hipError_t e = raise_lds(k, lds);
  if (e != hipSuccess) return e;
  e = (t0 || t1) ? hipExtLaunchKernel(k, dim3(blocks), dim3(kBlock), params, lds, st, t0, t1, 0)
                 : hipLaunchKernel(k, dim3(blocks), dim3(kBlock), params, lds, st);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_down_take(int P, const ProjArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  const void *k = down_take_ptr(P);
  if (!k || a.grid_rows < 1 || a.grid_rows > kDTRows || a.act_ld % 4 != 0 || reinterpret_cast<uintptr_t>(a.act) % 16 != 0)
    return hipErrorInvalidValue;
  // one wave per group row, each with its own staged h row
  const size_t lds = (size_t)a.grid_rows * rows16_lds_bytes(P);
  static bool raised[5][kMaxDevices] = {};
  if (lds > 48 * 1024) {  // raised once, to what the most rows need
    const hipError_t e = raise_lds_once(k, (int)(kDTRows * rows16_lds_bytes(P)), raised[P]);
    if (e != hipSuccess) return e;
  }
  ProjArgs args = a;
  void *params[] = {&args};
  const dim3 grid((a.O + kDTTile - 1) / kDTTile), block(a.grid_rows * kWave);
  hipError_t e = (t0 || t1) ? hipExtLaunchKernel(k, grid, block, params, lds, st, t0, t1, 0)
                            : hipLaunchKernel(k, grid, block, params, lds, st);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_down(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st, hipEvent_t t0,
                       hipEvent_t t1) {
  hipError_t e = launch(V, P, 1, gen, false, a, blocks, st, t0, t1);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace i4moe
