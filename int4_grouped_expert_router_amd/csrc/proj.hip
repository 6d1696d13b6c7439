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
#include "common.h"

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

template <int V>
__device__ __forceinline__ void load_span(const uint8_t *p, uint32_t (&w)[V]) {
  if constexpr (V == 4) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
  } else if constexpr (V == 2) {
    const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    w[0] = u.x; w[1] = u.y;
  } else {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
    for (int v = 0; v < V; ++v) w[v] = __builtin_nontemporal_load(q + v);
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

template <int V, int P, bool DUAL, bool GEN>
__global__ __launch_bounds__(kBlock) void k_proj(ProjArgs a) {
  constexpr int NT = DUAL ? 2 : 1;
  constexpr int RB = rows_per_step(V, P, NT);
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
  const GroupDev *__restrict__ g = a.group;

  if (DUAL && a.group_copy != nullptr && blockIdx.x == 0) {
    const int32_t *src = reinterpret_cast<const int32_t *>(g);
    int32_t *dst = reinterpret_cast<int32_t *>(a.group_copy);
    for (int i = threadIdx.x; i < I4MOE_GROUP_WORDS; i += kBlock) dst[i] = src[i];
  }

  const int nrows = min(g->n_rows, kRows);
  const int jr = wave / a.tiles;
  if (jr >= nrows) return;
  const int tile = wave - jr * a.tiles;
  const int e = g->row_expert[jr];
  const int arow = DUAL ? g->row_token[jr] : jr;
  const TensorDesc TA = a.tA[e];
  TensorDesc TB = TA;
  if (DUAL) TB = a.tB[e];

  const int C = a.C;
  const int RD = (C + 7) >> 3;

  // Activation slice of this lane, span sums and the group index of every span.
  float xe[P][V][4], xo[P][V][4], xm8[P];
  int giA[P], giB[P];
  const size_t row_off = (size_t)arow * a.act_ld;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int ds = p * 64 * V + lane * V;
    float span = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float t[8];
      load8(a.act, a.act_bf16, row_off, 8 * (ds + v), C, t);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xe[p][v][k] = t[2 * k];
        xo[p][v][k] = t[2 * k + 1] * 0.0625f;
        span += t[2 * k] + t[2 * k + 1];
      }
    }
    xm8[p] = -8.f * span;
    giA[p] = (TA.ng == 1 || ds >= RD) ? 0 : (8 * ds) / TA.gs;
    giB[p] = (TB.ng == 1 || ds >= RD) ? 0 : (8 * ds) / TB.gs;
  }
  // GEN launches carry the per-byte path; others only hold tensors whose groups align with spans.
  const bool genA = GEN && TA.ng > 1 && (TA.gs % (8 * V)) != 0;
  const bool genB = GEN && DUAL && TB.ng > 1 && (TB.gs % (8 * V)) != 0;

  const int o_begin = tile * a.tile_rows;
  const int o_end = min(o_begin + a.tile_rows, a.O);
  float *outp = a.out + (size_t)jr * a.out_ld;

  for (int o0 = o_begin; o0 < o_end; o0 += RB) {
    uint32_t wa[RB][P][V], wb[RB][P][V];
    float sa[RB][P], sb[RB][P];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int o = o0 + r;
      const bool rv = o < o_end;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int ds = p * 64 * V + lane * V;
        const bool ok = rv && ds < RD;
        if (ok) {
          load_span<V>(TA.q + (size_t)o * TA.row_bytes + 4 * ds, wa[r][p]);
          sa[r][p] = TA.s[(size_t)o * TA.ng + giA[p]];
        } else {
#pragma unroll
          for (int v = 0; v < V; ++v) wa[r][p][v] = 0u;
          sa[r][p] = 0.f;
        }
        if (DUAL) {
          if (ok) {
            load_span<V>(TB.q + (size_t)o * TB.row_bytes + 4 * ds, wb[r][p]);
            sb[r][p] = TB.s[(size_t)o * TB.ng + giB[p]];
          } else {
#pragma unroll
            for (int v = 0; v < V; ++v) wb[r][p][v] = 0u;
            sb[r][p] = 0.f;
          }
        }
      }
    }

    float outv = 0.f;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int o = o0 + r;
      float accA = 0.f, accB = 0.f;
      if (!genA) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          float ap = xm8[p];
#pragma unroll
          for (int v = 0; v < V; ++v) ap = dot8(wa[r][p][v], xe[p][v], xo[p][v], ap);
          accA = fmaf(sa[r][p], ap, accA);
        }
      } else if constexpr (GEN) {
        if (o < o_end) accA = row_dot_generic<V, P>(TA, o, wa[r], xe, xo, lane, RD);
      }
      const float sumA = wave_sum(accA);
      float res = sumA;
      if (DUAL) {
        if (!genB) {
#pragma unroll
          for (int p = 0; p < P; ++p) {
            float bp = xm8[p];
#pragma unroll
            for (int v = 0; v < V; ++v) bp = dot8(wb[r][p][v], xe[p][v], xo[p][v], bp);
            accB = fmaf(sb[r][p], bp, accB);
          }
        } else if constexpr (GEN) {
          if (o < o_end) accB = row_dot_generic<V, P>(TB, o, wb[r], xe, xo, lane, RD);
        }
        const float sumB = wave_sum(accB);
        res = sumA / (1.f + expf(-sumA)) * sumB;
      }
      if (lane == r) outv = res;
    }
    if (lane < RB && o0 + lane < o_end) outp[o0 + lane] = outv;
  }
}

template <bool DUAL>
hipError_t launch(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st) {
#define I4MOE_CASE(v, p)                                                                   \
  if (V == v && P == p) {                                                                  \
    if (gen)                                                                               \
      hipLaunchKernelGGL((k_proj<v, p, DUAL, true>), dim3(blocks), dim3(kBlock), 0, st, a); \
    else                                                                                   \
      hipLaunchKernelGGL((k_proj<v, p, DUAL, false>), dim3(blocks), dim3(kBlock), 0, st, a); \
    return hipGetLastError();                                                              \
  }
  I4MOE_CASE(1, 1) I4MOE_CASE(1, 2) I4MOE_CASE(1, 3) I4MOE_CASE(1, 4)
  I4MOE_CASE(2, 1) I4MOE_CASE(2, 2) I4MOE_CASE(2, 3) I4MOE_CASE(2, 4)
  I4MOE_CASE(3, 1) I4MOE_CASE(3, 2) I4MOE_CASE(3, 3) I4MOE_CASE(3, 4)
  I4MOE_CASE(4, 1) I4MOE_CASE(4, 2) I4MOE_CASE(4, 3) I4MOE_CASE(4, 4)
#undef I4MOE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dual(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st) {
  return launch<true>(V, P, gen, a, blocks, st);
}
hipError_t launch_down(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st) {
  return launch<false>(V, P, gen, a, blocks, st);
}

}  // namespace i4moe
