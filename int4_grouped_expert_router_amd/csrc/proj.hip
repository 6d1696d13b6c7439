// Grouped W4A16 projections for decode (gfx950, wave64, no MFMA: at S<=4 every int4 weight
// feeds one to four FMAs, so the launch is bound by the HBM weight stream).
//
//   dual : h[row][o] = silu(G_e[o,:] . x_t) * (U_e[o,:] . x_t)     (gate/up fused, SiLU fused)
//   down : y[row][o] = Dn_e[o,:] . h[row]
//
// for every group row (expert e, token t) and output row o.  Sources: the grouped
// dual/silu/down decode path of the TC_W4A16 gating commit and the group-wise kernels of the
// g4 commit ("Commit history of c/backend_cuda.cu"): the per-group scale is applied inside the
// accumulation, gs = 0 is per-row, and per-row and group-wise tensors run in one launch.
//
// Work decomposition.  One wavefront owns a tile of consecutive output rows of one group row,
// so the activation slice it needs is fixed: it is loaded once into registers and reused for
// every row of the tile.  A row is covered by P passes of the whole wave; in pass p lane l
// owns V consecutive weight dwords (8V columns) starting at dword p*64*V + l*V, fetched with
// one V-dword load, so every pass of the wave reads 256*V contiguous bytes.
//
// Dequantisation.  Nibbles stay offset-binary.  For a weight dword w the masks
// w & 0x0F0F0F0F and w & 0xF0F0F0F0 put the even-column nibbles q and 16 * (odd-column
// nibbles) in the four bytes, which v_cvt_f32_ubyte{0..3} convert directly; the odd-column
// activations are pre-divided by 16 (exact) so both give q * x.  The offset is folded in once
// per span: sum (q - 8) x = sum q x - 8 sum x, with the span sums of x precomputed with the
// slice.  That is 2.25 VALU ops per weight.  Each span accumulator is multiplied by its
// scale (the row scale, or the span's group scale when gs is a multiple of 8V), then the
// lane partials are summed across the wave with DPP in a fixed pattern (deterministic).
// Group sizes that split a span fall back to a per-byte path.
//
// Kernels here:
//   k_proj<V, P, NT, GEN, XB, SEL>  the dual (NT = 2) and long-row down (NT = 1) projections;
//                                   SEL runs a one-token expert selection first (select.h)
//   k_rows16<P>                     down projection of short rows, 16 lanes per row
//   k_down_take<P, W>               down projection of short rows fused with the take (one
//                                   token, one issue): the weighted, fixed-order sum of the
//                                   rows is added to the residual in the same launch
#include <hip/hip_ext.h>

#include "select.h"

namespace i4moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Keep the compiler from folding the byte masks into each conversion (which would cost a
// shift+mask per nibble instead of one mask per four nibbles).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float ub0(uint32_t a) { return (float)(a & 0xffu); }
__device__ __forceinline__ float ub1(uint32_t a) { return (float)((a >> 8) & 0xffu); }
__device__ __forceinline__ float ub2(uint32_t a) { return (float)((a >> 16) & 0xffu); }
__device__ __forceinline__ float ub3(uint32_t a) { return (float)(a >> 24); }

// Eight columns of one weight dword: xe = activations of the even columns, xo = activations
// of the odd columns divided by 16.
__device__ __forceinline__ float dot8(uint32_t w, const float (&xe)[4], const float (&xo)[4], float acc) {
  const uint32_t lo = opaque(w & 0x0F0F0F0Fu);
  const uint32_t hi = opaque(w & 0xF0F0F0F0u);
  acc = fmaf(ub0(lo), xe[0], acc);
  acc = fmaf(ub1(lo), xe[1], acc);
  acc = fmaf(ub2(lo), xe[2], acc);
  acc = fmaf(ub3(lo), xe[3], acc);
  acc = fmaf(ub0(hi), xo[0], acc);
  acc = fmaf(ub1(hi), xo[1], acc);
  acc = fmaf(ub2(hi), xo[2], acc);
  acc = fmaf(ub3(hi), xo[3], acc);
  return acc;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  bf16x2 r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

// Eight columns of one weight dword against packed bf16 activation pairs.  Nibble k (column
// 8d+k) sits at bits 4k..4k+3.  t0 = w & 0x0F0F0F0F isolates nibbles 0,2,4,6 in the low bits
// of its bytes, t1 = (w >> 4) & 0x0F0F0F0F nibbles 1,3,5,7; one v_perm_b32 then puts two of
// them under the bf16 high byte 0x43, giving the exact bf16 values 128 + q.  v_dot2_f32_bf16
// takes (128 + q_a) x_a + (128 + q_b) x_b into the f32 accumulator; the pairs are (0,4),
// (2,6), (1,5), (3,7) and the activations are packed to match.  The 128 + 8 offset comes out
// once per span through the initial value -136 * sum(x).  7 integer ops + 4 dot2 per 8 weights.
__device__ __forceinline__ float dot8_bf16(uint32_t w, const uint32_t (&xp)[4], float acc) {
  const uint32_t t0 = w & 0x0F0F0F0Fu;
  const uint32_t t1 = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t hi = 0x43434343u;
  const uint32_t p04 = __builtin_amdgcn_perm(hi, t0, 0x04020400u);
  const uint32_t p26 = __builtin_amdgcn_perm(hi, t0, 0x04030401u);
  const uint32_t p15 = __builtin_amdgcn_perm(hi, t1, 0x04020400u);
  const uint32_t p37 = __builtin_amdgcn_perm(hi, t1, 0x04030401u);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(p04), as_bf16x2(xp[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(p26), as_bf16x2(xp[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(p15), as_bf16x2(xp[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(p37), as_bf16x2(xp[3]), acc, false);
  return acc;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
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

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Eight activations of columns c0..c0+7 (zero past C).  f32 rows are 8-byte aligned and bf16
// rows 4-byte aligned because C is even.
__device__ __forceinline__ void load8(const void *act, int bf16, size_t row_off, int c0, int C, float (&t)[8]) {
  if (c0 + 8 <= C) {
    if (bf16) {
      const uint32_t *p = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(act) + row_off + c0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t u = p[k];
        t[2 * k] = bf16_to_f32(u & 0xffffu);
        t[2 * k + 1] = bf16_to_f32(u >> 16);
      }
    } else {
      const float2 *p = reinterpret_cast<const float2 *>(static_cast<const float *>(act) + row_off + c0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 u = p[k];
        t[2 * k] = u.x;
        t[2 * k + 1] = u.y;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = 0.f;
    for (int c = c0; c < C && c < c0 + 8; ++c) {
      t[c - c0] = bf16 ? bf16_to_f32(static_cast<const uint16_t *>(act)[row_off + c])
                       : static_cast<const float *>(act)[row_off + c];
    }
  }
}

// Per-byte path for group sizes that split a lane's span (any even gs): each byte's two
// columns share one group because gs is even.
template <int V, int P>
__device__ float row_dot_generic(const TensorDesc &T, int o, const uint32_t (&w)[P][V], const float (&xe)[P][V][4],
                                 const float (&xo)[P][V][4], int lane, int RD) {
  float acc = 0.f;
  const float *srow = T.s + (size_t)o * T.ng;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * 64 * V + lane * V;
    if (ds >= RD) continue;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int d = ds + v;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int col = 8 * d + 2 * k;
        if (col < T.C) {
          const float s = srow[col / T.gs];
          const float lo = (float)(int)((w[p][v] >> (8 * k)) & 15u) - 8.f;
          const float hi = (float)(int)((w[p][v] >> (8 * k + 4)) & 15u) - 8.f;
          acc = fmaf(s, fmaf(lo, xe[p][v][k], hi * (16.f * xo[p][v][k])), acc);
        }
      }
    }
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

// Activation slice of one lane.  f32 path: x of the even columns and x/16 of the odd columns,
// offset term -8 * sum(x) per span.  bf16 path: packed pairs (x_k, x_{k+4}) in the order the
// weight pairs are built, offset term -136 * sum(x) per span.
template <int V, int P, bool XB>
struct Act {
  float xe[P][V][4], xo[P][V][4];
  float xm[P];
};
template <int V, int P>
struct Act<V, P, true> {
  uint32_t xp[P][V][4];
  float xm[P];
};

// Words of the staged activation row: the row padded with zeros to the columns all lanes of
// all passes cover (8V columns per lane per pass); bf16 pairs for XB, f32 otherwise.
template <int V, int P, bool XB>
constexpr int act_words() {
  return XB ? P * 64 * V * 4 : P * 64 * V * 8;
}

// The workgroup copies its activation row into LDS with coalesced 4-byte loads (every wave of
// the workgroup works on the same group row).  A lane's slice is contiguous in the row but
// 16V (bf16) or 32V (f32) bytes from its neighbour's, so reading it from global memory directly
// would touch a separate cache line per lane and load; LDS takes that access pattern for free.
// The copy is split in two so the kernel can issue these loads before its first weight loads:
// the LDS writes then wait only for the (older) activation loads, not for weights in flight.
template <int V, int P, bool XB>
constexpr int stage_words() {
  return act_words<V, P, XB>() / kBlock;
}

template <bool XB, int N>
__device__ __forceinline__ void stage_load(uint32_t (&xs)[N], const void *act, int bf16, size_t row_off, int C) {
  if (XB) {
    const uint32_t *row = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(act) + row_off);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int w = threadIdx.x + i * kBlock;
      xs[i] = row[2 * w < C ? w : 0];
    }
  } else if (bf16) {
    const uint16_t *row = static_cast<const uint16_t *>(act) + row_off;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int w = threadIdx.x + i * kBlock;
      xs[i] = row[w < C ? w : 0];
    }
  } else {
    const uint32_t *row = reinterpret_cast<const uint32_t *>(static_cast<const float *>(act) + row_off);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int w = threadIdx.x + i * kBlock;
      xs[i] = row[w < C ? w : 0];
    }
  }
}

// Zeros past the row's C columns; bf16 values widened to f32 bits except for XB (pairs).
template <bool XB, int N>
__device__ __forceinline__ void stage_store(uint32_t *lds, const uint32_t (&xs)[N], int bf16, int C) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int w = threadIdx.x + i * kBlock;
    uint32_t v;
    if (XB)
      v = 2 * w < C ? xs[i] : 0u;
    else
      v = w < C ? (bf16 ? xs[i] << 16 : xs[i]) : 0u;
    lds[w] = v;
  }
}

// The lane's slice of the staged row: dword spans p * LR * V + lane * V + [0, V) for LR lanes
// per row.
template <int V, int P, bool XB, int LR = kWave>
__device__ __forceinline__ void read_act(uint32_t (&raw)[P][V][XB ? 4 : 8], const uint32_t *lds, int lane) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int d = p * LR * V + lane * V + v;
      if constexpr (XB) {
        const u4 q = *reinterpret_cast<const u4 *>(lds + 4 * d);
        raw[p][v][0] = q.x; raw[p][v][1] = q.y; raw[p][v][2] = q.z; raw[p][v][3] = q.w;
      } else {
        const u4 q0 = *reinterpret_cast<const u4 *>(lds + 8 * d);
        const u4 q1 = *reinterpret_cast<const u4 *>(lds + 8 * d + 4);
        raw[p][v][0] = q0.x; raw[p][v][1] = q0.y; raw[p][v][2] = q0.z; raw[p][v][3] = q0.w;
        raw[p][v][4] = q1.x; raw[p][v][5] = q1.y; raw[p][v][6] = q1.z; raw[p][v][7] = q1.w;
      }
    }
  }
}

template <int V, int P, bool XB>
__device__ __forceinline__ void finish_act(Act<V, P, XB> &A, const uint32_t (&raw)[P][V][XB ? 4 : 8]) {
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float span = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      if constexpr (XB) {
        const uint32_t *u = raw[p][v];  // u[k] holds columns 2k (low half) and 2k+1 (high half)
        A.xp[p][v][0] = (u[0] & 0xffffu) | (u[2] << 16);          // columns 0, 4
        A.xp[p][v][1] = (u[1] & 0xffffu) | (u[3] << 16);          // columns 2, 6
        A.xp[p][v][2] = (u[0] >> 16) | (u[2] & 0xffff0000u);      // columns 1, 5
        A.xp[p][v][3] = (u[1] >> 16) | (u[3] & 0xffff0000u);      // columns 3, 7
#pragma unroll
        for (int k = 0; k < 4; ++k) span += bf16_to_f32(u[k] & 0xffffu) + bf16_to_f32(u[k] >> 16);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float e = __uint_as_float(raw[p][v][2 * k]), o = __uint_as_float(raw[p][v][2 * k + 1]);
          A.xe[p][v][k] = e;
          A.xo[p][v][k] = o * 0.0625f;
          span += e + o;
        }
      }
    }
    A.xm[p] = (XB ? -136.f : -8.f) * span;
  }
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
// zeros the same way; its activations are zero, so it adds nothing.
template <int V, int P, int NT, int RB>
__device__ __forceinline__ void load_step(Step<V, P, NT, RB> &st, const TensorDesc (&T)[NT], const int (&gi)[NT][P],
                                          int o, int o_end, int lane) {
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const bool ok = o + r < o_end;
    const int row = ok ? o + r : 0;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T[n].q + (size_t)row * T[n].row_bytes, ok ? T[n].row_bytes : 0);
      const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T[n].s + (size_t)row * T[n].ng, ok ? 4 * T[n].ng : 0);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        load_span<V>(wr, 4 * (p * 64 * V + lane * V), st.w[n][r][p]);
        st.s[n][r][p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * gi[n][p], 0, 0));
      }
    }
  }
}

// Dot products of one step's rows, reduced over the wave; lane (o - o_begin + r) keeps row
// o + r's result, and the tile's results leave in one coalesced store at the end.
template <int V, int P, int NT, int RB, bool GEN, bool XB>
__device__ __forceinline__ void compute_step(const Step<V, P, NT, RB> &st, const TensorDesc (&T)[NT],
                                             const bool (&gen)[NT], const Act<V, P, XB> &A, int o, int o_end,
                                             int lane, int RD, int o_begin, float &outv) {
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float sum[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float acc = 0.f;
      if (!gen[n]) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          float ap = A.xm[p];
#pragma unroll
          for (int v = 0; v < V; ++v) {
            if constexpr (XB)
              ap = dot8_bf16(st.w[n][r][p][v], A.xp[p][v], ap);
            else
              ap = dot8(st.w[n][r][p][v], A.xe[p][v], A.xo[p][v], ap);
          }
          acc = fmaf(st.s[n][r][p], ap, acc);
        }
      } else if constexpr (GEN && !XB) {
        if (o + r < o_end) acc = row_dot_generic<V, P>(T[n], o + r, st.w[n][r], A.xe, A.xo, lane, RD);
      }
      sum[n] = wave_sum(acc);
    }
    float res = sum[0];
    if constexpr (NT == 2) res = sum[0] / (1.f + expf(-sum[0])) * sum[1];
    if (lane == o - o_begin + r) outv = res;
  }
}

// NT = 2: dual gate/up with the SiLU-gated product; NT = 1: down projection.  XB: bf16
// activations through v_dot2_f32_bf16 (dual only).  SEL (dual, one token, E <= 64): every
// workgroup first runs the expert selection itself from the router's finished scores, so no
// selection launch sits between the router GEMV and the experts; workgroup 0 publishes the
// route and group records, the first workgroup of each row that row's descriptor (for the
// down projection, the take and the taps).  A tile holds at most 64 rows (one result per
// lane).
template <int V, int P, int NT, bool GEN, bool XB, bool SEL = false>
__global__ __launch_bounds__(kBlock) void k_proj(ProjArgs a) {
  constexpr int RB = rows_per_step(V, P, NT, 16);
  extern __shared__ uint32_t s_act[];
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
    // this row is selection jr of the one token
    live = jr < r.n ? 1 : 0;
    const int e = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(r.e_k, jr));
    const float w = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(r.w_k), jr));
    arow = 0;
    GroupBuf *out = ra.out;
    if (blockIdx.x == 0 && wib == 0) {
      // route record and group record of the token: its selections, one row each, in order
      RouteTok *rt = out->route;
      const int n = r.n;
      if (lane == 0) rt->n = n;
      rt->idx[lane] = lane < ra.K ? r.e_k : -1;
      rt->w[lane] = r.w_k;
      GroupDev *G = &out->g;
      if (lane < n) {
        G->entry_expert[lane] = r.e_k;
        G->entry_row0[lane] = lane;
        G->row_token[lane] = 0;
        G->row_expert[lane] = r.e_k;
        G->row_weight[lane] = r.w_k;
        G->red_rows[lane] = lane;
      }
      if (lane == 0) {
        G->entry_row0[n] = n;
        G->tok_row0[0] = 0;
        G->tok_row0[1] = n;
        G->n_entries = n;
        G->n_rows = n;
        G->S = 1;
        G->reserved = 0;
      }
    }
    if (writer && wib == 0 && lane < kDescWords) {
      // this row's descriptor for the down projection and the take (zeros for a dead row)
      uint32_t val = 0u;
      if (live) {
        if (lane == kLiveWord)
          val = 1u;
        else if (lane < kTabWords)
          val = s_tab[e * kDescWords + lane];
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
  bool gen[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int p = 0; p < P; ++p) gi[n][p] = 0;
    if (T[n].ng > 1) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int ds = p * 64 * V + lane * V;
        gi[n][p] = ds < RD ? (8 * ds) / T[n].gs : 0;
      }
    }
    // GEN launches carry the per-byte path; others hold only tensors whose groups align with spans.
    gen[n] = GEN && T[n].ng > 1 && (T[n].gs % (8 * V)) != 0;
  }

  const int o_begin = tile * a.tile_rows;
  const int o_end = min(o_begin + a.tile_rows, a.O);
  const bool work = o_begin < o_end;

  // Activation loads first, then the first two steps of weights (empty ranges for a wave
  // without rows); the activation row goes to LDS as soon as its own loads have landed.
  // Scheduling barriers keep the issue order: the wait counts below assume it.
  uint32_t xs[stage_words<V, P, XB>()];
  stage_load<XB>(xs, a.act, a.act_bf16, (size_t)arow * a.act_ld, C);
  __builtin_amdgcn_sched_barrier(0);
  Step<V, P, NT, RB> b0, b1;
  load_step<V, P, NT, RB>(b0, T, gi, o_begin, o_end, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_step<V, P, NT, RB>(b1, T, gi, o_begin + RB, o_end, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<XB>(s_act, xs, a.act_bf16, C);
  __syncthreads();
  if (!work) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  uint32_t raw[P][V][XB ? 4 : 8];
  read_act<V, P, XB>(raw, s_act, lane);
  Act<V, P, XB> A;
  finish_act<V, P, XB>(A, raw);

  // Two-stage pipeline: while one step computes, the other step's weights are in flight.  The
  // loop has one exit, at the bottom; the last pass issues loads of empty ranges.
  float outv = 0.f;
  int o = o_begin;
  do {
    compute_step<V, P, NT, RB, GEN, XB>(b0, T, gen, A, o, o_end, lane, RD, o_begin, outv);
    load_step<V, P, NT, RB>(b0, T, gi, o + 2 * RB, o_end, lane);
    if (o + RB < o_end) compute_step<V, P, NT, RB, GEN, XB>(b1, T, gen, A, o + RB, o_end, lane, RD, o_begin, outv);
    load_step<V, P, NT, RB>(b1, T, gi, o + 3 * RB, o_end, lane);
    o += 2 * RB;
  } while (o < o_end);
  if (lane < o_end - o_begin) a.out[(size_t)jr * a.out_ld + o_begin + lane] = outv;
  asm volatile("" ::"v"(touch));
}

// ---- Short rows (the down projection, C <= 2048 columns): 16 lanes per row, so one wave
// instruction covers four rows.  A row's dot product is then summed over 16 lanes (four DPP
// steps, all four rows at once) instead of 64, and no lane idles when a row is shorter than
// 64 lanes x 16 bytes.  f32 activations, per-row or span-aligned group scales.
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
// get an offset past every range for the same effect.
template <int P>
__device__ __forceinline__ void load_step16(Step16<P> &st, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                            const TensorDesc &T, const int (&woff)[P], const int (&gi)[P], int o,
                                            int g) {
  const int row = o + g;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    load_span<4>(wr, woff[p] < 0 ? 0x7ffffff0 : row * T.row_bytes + woff[p], st.w[p]);
    st.s[p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * (row * T.ng + gi[p]), 0, 0));
  }
}

// LDS word of column pair-half `half` of dword span (p, v) for lane li: the 16 lanes' 16-byte
// chunks of one (p, v, half) are contiguous, so each read is conflict-free.
__device__ __forceinline__ int act16_word(int p, int v, int half, int li) { return (((p * 4 + v) * 2 + half) * kLR + li) * 4; }

// The activations are read from LDS per step (two ds_read_b128 per weight dword) rather than
// held in registers: a 96-column slice would take 96 VGPRs, and with it the kernel fits
// three waves per SIMD instead of six.  Odd columns are staged already divided by 16.
template <int P>
__device__ __forceinline__ void compute_step16(const Step16<P> &st, const uint32_t *lds, int li, const float (&xm)[P],
                                               int o, int o_begin, int lane, float &outv) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float ap = xm[p];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f4 q0 = *reinterpret_cast<const f4 *>(lds + act16_word(p, v, 0, li));
      const f4 q1 = *reinterpret_cast<const f4 *>(lds + act16_word(p, v, 1, li));
      const float xe[4] = {q0.x, q0.z, q1.x, q1.z}, xo[4] = {q0.y, q0.w, q1.y, q1.w};
      ap = dot8(st.w[p][v], xe, xo, ap);
    }
    acc = fmaf(st.s[p], ap, acc);
  }
  const float sum = row16_sum(acc);
#pragma unroll
  for (int g = 0; g < kGR; ++g) {
    const float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum), g * kLR));
    if (lane == o - o_begin + g) outv = r;
  }
}

// Stage column w (value x; 0 past the row) of a short row: odd columns divided by 16 (exact),
// as dot8 takes them.
__device__ __forceinline__ void stage16(uint32_t *lds, int w, float x) {
  const int d = w >> 3, j = w & 7;  // dword span d = p * 64 + li * 4 + v, column j in it
  lds[act16_word(d >> 6, d & 3, j >> 2, (d >> 2) & (kLR - 1)) + (j & 3)] = __float_as_uint((w & 1) ? x * 0.0625f : x);
}

// The same for columns c4 .. c4 + 3 (c4 a multiple of 4): one 16-byte LDS write.
__device__ __forceinline__ void stage16x4(uint32_t *lds, int c4, float4 x) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int d = c4 >> 3;
  f4 v = {x.x, x.y * 0.0625f, x.z, x.w * 0.0625f};
  *reinterpret_cast<f4 *>(lds + act16_word(d >> 6, d & 3, (c4 & 7) >> 2, (d >> 2) & (kLR - 1))) = v;
}

// Offset term of each of the lane's spans: -8 * (sum of its activations), summed in
// column-pair order.
template <int P>
__device__ __forceinline__ void span_offsets16(float (&xm)[P], const uint32_t *lds, int li) {
  constexpr int V = 4;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float span = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = 2 * k;
        span += __uint_as_float(lds[act16_word(p, v, j >> 2, li) + (j & 3)]) +
                16.f * __uint_as_float(lds[act16_word(p, v, (j + 1) >> 2, li) + ((j + 1) & 3)]);
      }
    }
    xm[p] = -8.f * span;
  }
}

template <int P>
__global__ __launch_bounds__(kBlock) void k_rows16(ProjArgs a) {
  constexpr int V = 4;
  extern __shared__ uint32_t s_act[];
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
  int gi[P], woff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * kLR * V + li * V;
    gi[p] = (T.ng > 1 && ds < RD) ? (8 * ds) / T.gs : 0;
    woff[p] = ds < RD ? 4 * ds : -1;
  }
  const int o_begin = tile * a.tile_rows;
  const int o_end = min(o_begin + a.tile_rows, a.O);
  const bool work = o_begin < o_end;
  const int rows_in = work ? o_end : 0;  // buffer ranges: rows [0, o_end) of this tensor
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T.q, rows_in * T.row_bytes);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T.s, rows_in * T.ng * 4);

  uint32_t xs[stage_words<V, P, false>() * kLR / kWave];
  stage_load<false>(xs, a.act, 0, (size_t)jr * a.act_ld, C);
  __builtin_amdgcn_sched_barrier(0);
  Step16<P> b0, b1;
  load_step16<P>(b0, wr, sr, T, woff, gi, o_begin, g);
  __builtin_amdgcn_sched_barrier(0);
  load_step16<P>(b1, wr, sr, T, woff, gi, o_begin + kGR, g);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(xs) / sizeof(xs[0])); ++i) {
    const int w = threadIdx.x + i * kBlock;  // column
    stage16(s_act, w, w < C ? __uint_as_float(xs[i]) : 0.f);
  }
  __syncthreads();
  if (!work) {
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  float xm[P];
  span_offsets16<P>(xm, s_act, li);

  float outv = 0.f;
  int o = o_begin;
  do {
    compute_step16<P>(b0, s_act, li, xm, o, o_begin, lane, outv);
    load_step16<P>(b0, wr, sr, T, woff, gi, o + 2 * kGR, g);
    if (o + kGR < o_end) compute_step16<P>(b1, s_act, li, xm, o + kGR, o_begin, lane, outv);
    load_step16<P>(b1, wr, sr, T, woff, gi, o + 3 * kGR, g);
    o += 2 * kGR;
  } while (o < o_end);
  if (lane < o_end - o_begin) a.out[(size_t)jr * a.out_ld + o_begin + lane] = outv;
  asm volatile("" ::"v"(touch));
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

size_t rows16_lds_bytes(int P) { return 4u * (size_t)P * kLR * 4 * 8; }

// ---- Down projection and take in one launch (one token, one issue, at most kDTRows rows,
// short down rows).  A workgroup owns TL = 16 output columns of the residual and has one wave
// per group row: the wave stages its row's h in its own LDS region and computes its expert's
// TL outputs exactly as k_rows16 does; the rows then meet in LDS and are summed in row
// (route) order with the take's arithmetic, fmaf over the live rows, added to the residual.
// No y rows go through memory and no take launch follows.  (Measured on the medium decode
// layer: 8-column tiles double the h staging traffic and 32-column tiles leave half the CUs
// idle; both are slower.)  W > 1 splits a row's outputs over W waves that share its staged h.
template <int P, int W>
__global__ __launch_bounds__(kDTRows * W * kWave) void k_down_take(ProjArgs a) {
  constexpr int V = 4;
  constexpr int TL = kDTTile;
  constexpr int RW = TL / W;  // outputs per wave
  static_assert(RW % (2 * kGR) == 0 && RW <= kWave, "whole pipeline passes, one output per lane");
  extern __shared__ uint32_t s_act[];  // [kDTRows][P * 512] staged h rows
  __shared__ float s_y[kDTRows][TL];
  __shared__ float s_w[kDTRows];
  __shared__ int s_live[kDTRows];
  const int lane = threadIdx.x & 63;
  const int li = lane & (kLR - 1), g = lane / kLR;
  const int wi = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = wi / W;          // group row of this wave
  const int part = wi - r * W;   // its share of the tile's outputs and of the row's staging
  const int i0 = blockIdx.x * TL + part * RW;
  const int i_end = min(i0 + RW, a.O);
  const CGroupBuf G = (CGroupBuf)a.grp;
  const int rr = min(r, a.grid_rows - 1);
  const TensorDesc T = ld_desc(G->rows[rr].t[2]);
  const int live = r < a.grid_rows ? G->rows[rr].t[0].live : 0;
  const float wr_row = G->rows[rr].weight;
  asm volatile("" ::"s"(T.q), "s"(T.s), "s"(T.O), "s"(T.C), "s"(T.row_bytes), "s"(T.gs), "s"(T.ng));
  asm volatile("" ::"s"(live));
  // the residual of the tile, in flight from the start
  const float r_in = a.out[min(i0 + (lane % RW), a.O - 1)];

  const int C = a.C;
  const int RD = (C + 7) >> 3;
  int gi[P], woff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * kLR * V + li * V;
    gi[p] = (T.ng > 1 && ds < RD) ? (8 * ds) / T.gs : 0;
    woff[p] = ds < RD ? 4 * ds : -1;
  }
  const int rows_in = live && i0 < a.O ? i_end : 0;  // a dead row's loads read nothing
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(T.q, rows_in * T.row_bytes);
  const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(T.s, rows_in * T.ng * 4);

  // the wave's share of its row's h, four columns per lane and load (clamped, unconditional;
  // rows are 16-byte aligned and padded to a multiple of 64 columns)
  constexpr int NX = P * 512 / (4 * kWave * W);
  const float *hrow = static_cast<const float *>(a.act) + (size_t)rr * a.act_ld;
  float4 xs[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int c4 = 4 * (lane + (i * W + part) * kWave);
    xs[i] = *reinterpret_cast<const float4 *>(hrow + (c4 < C ? c4 : 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  Step16<P> b0, b1;
  load_step16<P>(b0, wr, sr, T, woff, gi, i0, g);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t *lds = s_act + r * (P * 512);
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int c4 = 4 * (lane + (i * W + part) * kWave);
    float4 x = xs[i];
    // C is even: a group of four is whole, half or empty
    if (c4 + 2 > C) x.x = x.y = 0.f;
    if (c4 + 4 > C) x.z = x.w = 0.f;
    stage16x4(lds, c4, x);
  }
  if constexpr (W == 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
  // the second step only now: a smaller first burst lands h and the first step sooner
  // (measured 0.25 us per layer faster than issuing both steps with h)
  load_step16<P>(b1, wr, sr, T, woff, gi, i0 + kGR, g);
  __builtin_amdgcn_sched_barrier(0);
  float xm[P];
  span_offsets16<P>(xm, lds, li);

  float outv = 0.f;
  int o = i0;
  do {
    compute_step16<P>(b0, lds, li, xm, o, i0, lane, outv);
    load_step16<P>(b0, wr, sr, T, woff, gi, o + 2 * kGR, g);
    if (o + kGR < i_end) compute_step16<P>(b1, lds, li, xm, o + kGR, i0, lane, outv);
    load_step16<P>(b1, wr, sr, T, woff, gi, o + 3 * kGR, g);
    o += 2 * kGR;
  } while (o < i_end);
  if (lane < RW) s_y[r][part * RW + lane] = outv;
  if (lane == 0 && part == 0) {
    s_w[r] = wr_row;
    s_live[r] = live;
  }
  __syncthreads();
  if (r == 0 && lane < RW && i0 + lane < a.O) {
    float acc = 0.f;
    for (int q = 0; q < a.grid_rows; ++q)
      if (s_live[q]) acc = fmaf(s_w[q], s_y[q][part * RW + lane], acc);
    a.out[i0 + lane] = r_in + acc;
  }
}

// Waves per group row.  Measured on the medium decode layer: one wave of 16 outputs per row
// 9.7 us, two waves of 8 outputs per row (16 waves per workgroup) 11.4 us.
constexpr int kDTWaves = 1;
const void *down_take_ptr(int P) {
  switch (P) {
    case 1: return reinterpret_cast<const void *>(&k_down_take<1, kDTWaves>);
    case 2: return reinterpret_cast<const void *>(&k_down_take<2, kDTWaves>);
    case 3: return reinterpret_cast<const void *>(&k_down_take<3, kDTWaves>);
    case 4: return reinterpret_cast<const void *>(&k_down_take<4, kDTWaves>);
    default: return nullptr;
  }
}
template <int NT, bool GEN, bool XB, bool SEL = false>
const void *kernel_ptr_t(int V, int P) {
#define I4MOE_PTR(v, p) \
  if (V == v && P == p) return reinterpret_cast<const void *>(&k_proj<v, p, NT, GEN, XB, SEL>);
  I4MOE_PTR(1, 1) I4MOE_PTR(1, 2) I4MOE_PTR(1, 3) I4MOE_PTR(1, 4)
  I4MOE_PTR(2, 1) I4MOE_PTR(2, 2) I4MOE_PTR(2, 3) I4MOE_PTR(2, 4)
  I4MOE_PTR(4, 1) I4MOE_PTR(4, 2) I4MOE_PTR(4, 3) I4MOE_PTR(4, 4)
#undef I4MOE_PTR
  return nullptr;
}

// The instantiation a launch uses: bf16 pairs only for dual launches over bf16 activations
// without per-byte group tensors.
const void *kernel_ptr(int V, int P, int NT, bool gen, bool xb, bool sel = false) {
  if (NT == 1) return gen ? kernel_ptr_t<1, true, false>(V, P) : kernel_ptr_t<1, false, false>(V, P);
  if (gen) return sel ? nullptr : kernel_ptr_t<2, true, false>(V, P);
  if (sel) return xb ? kernel_ptr_t<2, false, true, true>(V, P) : kernel_ptr_t<2, false, false, true>(V, P);
  return xb ? kernel_ptr_t<2, false, true>(V, P) : kernel_ptr_t<2, false, false>(V, P);
}

size_t lds_bytes(int V, int P, bool xb) { return 4u * (size_t)(xb ? P * 64 * V * 4 : P * 64 * V * 8); }

hipError_t launch(int V, int P, int NT, bool gen, bool xb, bool sel, const ProjArgs &a, int blocks, hipStream_t st,
                  hipEvent_t t0, hipEvent_t t1) {
  const void *k = kernel_ptr(V, P, NT, gen, xb, sel);
  if (!k) return hipErrorInvalidValue;
  ProjArgs args = a;
  void *params[] = {&args};
  const size_t lds = lds_bytes(V, P, xb);
  if (t0 || t1) return hipExtLaunchKernel(k, dim3(blocks), dim3(kBlock), params, lds, st, t0, t1, 0);
  return hipLaunchKernel(k, dim3(blocks), dim3(kBlock), params, lds, st);
}

}  // namespace

int proj_blocks_per_cu(int V, int P, int NT, bool gen, bool xb) {
  static int cache[5][5][3][2][2] = {};
  if (V < 1 || V > 4 || V == 3 || P < 1 || P > 4 || NT < 1 || NT > 2) return 1;
  int &c = cache[V][P][NT][gen ? 1 : 0][xb ? 1 : 0];
  if (c == 0) {
    const void *k = kernel_ptr(V, P, NT, gen, xb);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kBlock, lds_bytes(V, P, xb)) != hipSuccess || n < 1) {
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

hipError_t launch_dual(int V, int P, bool gen, bool xb, bool sel, const ProjArgs &a, int blocks, hipStream_t st,
                       hipEvent_t t0, hipEvent_t t1) {
  if (sel && !dual_sel_ok(a.ra, gen)) return hipErrorInvalidValue;
  hipError_t e = launch(V, P, 2, gen, xb && !gen, sel, a, blocks, st, t0, t1);
  return e != hipSuccess ? e : hipGetLastError();
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
  const void *k = rows16_ptr(P);
  if (!k) return hipErrorInvalidValue;
  ProjArgs args = a;
  void *params[] = {&args};
  hipError_t e = (t0 || t1) ? hipExtLaunchKernel(k, dim3(blocks), dim3(kBlock), params, rows16_lds_bytes(P), st, t0, t1, 0)
                            : hipLaunchKernel(k, dim3(blocks), dim3(kBlock), params, rows16_lds_bytes(P), st);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_down_take(int P, const ProjArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  const void *k = down_take_ptr(P);
  if (!k || a.grid_rows < 1 || a.grid_rows > kDTRows || a.act_ld % 4 != 0 || reinterpret_cast<uintptr_t>(a.act) % 16 != 0)
    return hipErrorInvalidValue;
  const size_t lds = (size_t)kDTRows * rows16_lds_bytes(P);
  static bool raised[5][kMaxDevices] = {};
  if (lds > 48 * 1024) {
    const hipError_t e = raise_lds_once(k, (int)lds, raised[P]);
    if (e != hipSuccess) return e;
  }
  ProjArgs args = a;
  void *params[] = {&args};
  const dim3 grid((a.O + kDTTile - 1) / kDTTile), block(kDTRows * kDTWaves * kWave);
  hipError_t e = (t0 || t1) ? hipExtLaunchKernel(k, grid, block, params, lds, st, t0, t1, 0)
                            : hipLaunchKernel(k, grid, block, params, lds, st);
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_down(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st, hipEvent_t t0,
                       hipEvent_t t1) {
  hipError_t e = launch(V, P, 1, gen, false, false, a, blocks, st, t0, t1);
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace i4moe
