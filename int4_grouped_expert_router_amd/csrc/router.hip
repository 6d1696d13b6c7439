// Device router for decode (gfx950): a GEMV launch for the E x D logits of S tokens, then a
// one-workgroup launch for the selection, the route records and the expert group.
//
// Source: the device-router commit ("First increment of the #431 plan") on the page "Commit
// history of c/backend_cuda.cu": logits GEMV + sigmoid, bias-augmented top-K by choice with
// strict-'>' tie-breaking, weights from the raw logit, route-level top-p truncation,
// norm_topk, routed_scale, one packed result; the batched router over S rows of the
// GPU-resident-pipeline commit; the S<=4 small-batch groups of the COLI_GROUP_ASYNC page.
//
// Precision: the f32 x f32 (or f32 x bf16) products are exact in f64 and are summed in f64;
// sigmoid, scores, top-p, norm and scale are f64; each weight is rounded to f32 once.  The
// selection therefore decides on f64 values.
//
// Selection: expert e is chosen in round r exactly when r experts beat it in the order
// (score descending, index ascending), which is what K rounds of an ascending strict-'>' scan
// produce.  So every lane counts, for the experts it holds, how many experts beat each one;
// counts below K are the selection positions.  No sequential rounds.
#include <hip/hip_ext.h>

#include "norm.h"
#include "select.h"

namespace i4moe {
namespace {


__device__ __forceinline__ float x_at(const void *x, int bf16, size_t i) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(x)[i]) << 16);
  return static_cast<const float *>(x)[i];
}

// Order this wave's LDS traffic (lanes of one wave exchanging through shared memory).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave's dot products of a W row segment [c0, c1) with up to kGT consecutive x rows
// t0 .. t0 + nt - 1, in f64 (every f32 x f32 or f32 x bf16 product is exact in f64).  Each
// W chunk is loaded once for all of the group's tokens.  Vector path: four float4 chunks per
// lane in flight per batch, with every x chunk they meet (addresses clamped into the segment
// and the token range, so the loads are unconditional); per token, FMAs in column order.
constexpr int kGT = 4;
template <bool XBF, int NG>
__device__ __forceinline__ void gemv_vec(double (&acc)[kGT], const float *wrow, const void *x, int D, int t0, int nt,
                                         int c0, int c1, int lane) {
#pragma unroll
  for (int t = 0; t < kGT; ++t) acc[t] = 0.0;
  for (int c = c0 + 4 * lane; c < c1; c += 16 * kWave) {
    float4 w[4];
    float xv[NG][4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cj = c + 4 * kWave * j < c1 ? c + 4 * kWave * j : c;
      w[j] = *reinterpret_cast<const float4 *>(wrow + cj);
#pragma unroll
      for (int t = 0; t < NG; ++t) {
        const size_t xoff = (size_t)(t0 + (t < nt ? t : nt - 1)) * D + cj;
        if constexpr (XBF) {
          const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + xoff);
          xv[t][j][0] = __uint_as_float(u.x << 16);
          xv[t][j][1] = __uint_as_float(u.x & 0xffff0000u);
          xv[t][j][2] = __uint_as_float(u.y << 16);
          xv[t][j][3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 q = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + xoff);
          xv[t][j][0] = q.x;
          xv[t][j][1] = q.y;
          xv[t][j][2] = q.z;
          xv[t][j][3] = q.w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c + 4 * kWave * j < c1) {
#pragma unroll
        for (int t = 0; t < NG; ++t) {
          acc[t] = fma((double)w[j].x, (double)xv[t][j][0], acc[t]);
          acc[t] = fma((double)w[j].y, (double)xv[t][j][1], acc[t]);
          acc[t] = fma((double)w[j].z, (double)xv[t][j][2], acc[t]);
          acc[t] = fma((double)w[j].w, (double)xv[t][j][3], acc[t]);
        }
      }
    }
  }
}

// One workgroup per `epb` experts, one wave per (expert, column split).  Each wave sums its
// split of W[e] . x[t] (f64, DPP wave sum); then one thread per (token, expert) adds the
// splits in split order into the logit and forms sigma and the choice score, so the selection
// starts from finished scores.  With a.vec (D % 4 == 0, 16-byte aligned W and x) every lane
// reads four consecutive columns per load.
constexpr int kGemvWaves = 16;
__global__ __launch_bounds__(kGemvWaves * kWave) void k_route_gemv(RouteArgs a) {
  __shared__ double s_part[kTokens][kGemvWaves];
  const int lane = threadIdx.x & 63;
  const int wib = threadIdx.x >> 6;
  const int el = wib / a.splits;
  const int sp = wib - el * a.splits;
  const int e = blockIdx.x * a.epb + el;
  // the finishing thread's expert and its bias, loaded before the long stream
  const int ft = threadIdx.x / a.epb, fe = blockIdx.x * a.epb + (threadIdx.x - ft * a.epb);
  const bool fin = ft < a.S && fe < a.E;
  const float fb = a.bias[min(fe, a.E - 1)];
  if (e < a.E) {
    const int c0 = sp * a.cols_per_split;
    const int c1 = min(a.D, c0 + a.cols_per_split);
    const float *wrow = a.W + (size_t)e * a.D;
    for (int t0 = 0; t0 < a.S; t0 += kGT) {
      const int nt = min(kGT, a.S - t0);
      double acc[kGT];
      if (a.vec) {
        // one token: a group of one, no repeated x loads or FMAs
        if (a.x_bf16)
          nt == 1 ? gemv_vec<true, 1>(acc, wrow, a.x, a.D, t0, nt, c0, c1, lane)
                  : gemv_vec<true, kGT>(acc, wrow, a.x, a.D, t0, nt, c0, c1, lane);
        else
          nt == 1 ? gemv_vec<false, 1>(acc, wrow, a.x, a.D, t0, nt, c0, c1, lane)
                  : gemv_vec<false, kGT>(acc, wrow, a.x, a.D, t0, nt, c0, c1, lane);
      } else {
#pragma unroll
        for (int t = 0; t < kGT; ++t) {
          acc[t] = 0.0;
          if (t < nt) {
            const size_t xoff = (size_t)(t0 + t) * a.D;
            for (int c = c0 + lane; c < c1; c += kWave)
              acc[t] = fma((double)wrow[c], (double)x_at(a.x, a.x_bf16, xoff + c), acc[t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kGT; ++t) {
        if (t < nt) {  // uniform
          const double v = wave_sum_f64(acc[t]);
          if (lane == 0) s_part[t0 + t][wib] = v;
        }
      }
    }
  }
  __syncthreads();
  if (fin) {
    const int fl = threadIdx.x - ft * a.epb;
    double l = 0.0;
    for (int j = 0; j < a.splits; ++j) l += s_part[ft][fl * a.splits + j];
    const double sg = 1.0 / (1.0 + exp(-l));
    double c = sg + (double)fb;
    if (c != c) c = -__builtin_inf();
    a.logits[(size_t)ft * a.E + fe] = l;
    a.score[(size_t)ft * a.E + fe] = make_double2(c, sg);
  }
}

// One workgroup, run once per layer on one CU, so written for latency: each wave selects for
// one token (four tokens per pass), every global read of a phase is issued in one batch, and
// the code is kept small.
__global__ __launch_bounds__(kBlock) void k_route_select(RouteArgs a) {
  extern __shared__ double s_dyn[];
  __shared__ int s_pidx[kRows];
  __shared__ float s_pw[kRows];
  __shared__ int s_n[kTokens];
  __shared__ int s_row_e[kRows], s_row_t[kRows], s_row_rank[kRows], s_row_size[kRows];
  __shared__ float s_row_w[kRows];
  __shared__ int s_rows;
  __shared__ __attribute__((aligned(16))) uint32_t s_tab[kSelTabE * kDescWords];  // expert records, E <= 256

  // With up to 256 experts, every expert's 128-byte record is loaded now, in the same batch as
  // the scores, so the row descriptors need no further memory round trip at the end.
  const bool tab_pre = a.table != nullptr && a.E <= kSelTabE;
  uint32_t tv[kSelTabPerThread];
  SelShared sh{s_pidx, s_pw, s_n, s_row_e, s_row_t, s_row_w, s_row_rank, s_row_size, &s_rows, tab_pre ? s_tab : nullptr};
  // behind each pass's first scores (the same records every pass, so the loads and the wait
  // counts do not depend on the pass)
  const int tab_bytes = tab_pre ? a.E * (int)sizeof(ExpertRec) : 0;
  for (int t0 = 0; t0 < a.S; t0 += select_slots(a.S))
    select_pass(a, s_dyn, t0, sh, [&] { table_prefetch_rsrc(tv, a.table, tab_bytes); });
  if (tab_pre) table_stage(s_tab, tv);
  publish_group(a, sh);
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, int parts, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (a.splits * a.epb > kGemvWaves || a.S * a.epb > a.splits * a.epb * kWave) return hipErrorInvalidValue;
  // dynamic LDS up to 64 KB (E = 1024, four tokens per pass) beside 34 KB of static arrays
  const size_t lds = select_lds_bytes(a.E, a.S);
  static bool raised[kMaxDevices] = {};
  if (parts & kRouteSelect) {
    const hipError_t e = raise_lds_once(reinterpret_cast<const void *>(&k_route_select),
                                        (int)select_lds_bytes(kMaxE, kTokens), raised);
    if (e != hipSuccess) return e;
  }
  // the event pair spans every launched part
  hipEvent_t g1 = (parts & kRouteSelect) ? nullptr : t1;
  hipEvent_t s0 = (parts & kRouteGemv) ? nullptr : t0;
  if (parts & kRouteGemv) {
    const dim3 grid((a.E + a.epb - 1) / a.epb), block(a.splits * a.epb * kWave);
    if (t0 || g1)
      hipExtLaunchKernelGGL(k_route_gemv, grid, block, 0, st, t0, g1, 0, a);
    else
      hipLaunchKernelGGL(k_route_gemv, grid, block, 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (parts & kRouteSelect) {
    if (s0 || t1)
      hipExtLaunchKernelGGL(k_route_select, dim3(1), dim3(kBlock), lds, st, s0, t1, 0, a);
    else
      hipLaunchKernelGGL(k_route_select, dim3(1), dim3(kBlock), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace i4moe
