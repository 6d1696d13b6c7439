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
#include "common.h"

namespace i4moe {
namespace {

constexpr int kPerLane = kMaxE / kWave;  // 16
constexpr int kWaves = kBlock / kWave;   // 4

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Fixed-pattern wave sum of doubles; the total is returned wave-uniform.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0xB1, 0xF>(v);
  v += dpp_f64<0x4E, 0xF>(v);
  v += dpp_f64<0x141, 0xF>(v);
  v += dpp_f64<0x140, 0xF>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

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

// partial[t][e][split] = sum over the split's columns of W[e][c] * x[t][c], one wave per
// (expert row, column split).  With a.vec (D % 4 == 0, 16-byte aligned W and x) every lane
// reads four consecutive columns per load.
__global__ __launch_bounds__(kBlock) void k_route_gemv(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (unit >= a.E * a.splits) return;
  const int e = unit / a.splits;
  const int sp = unit - e * a.splits;
  const int c0 = sp * a.cols_per_split;
  const int c1 = min(a.D, c0 + a.cols_per_split);
  const float *wrow = a.W + (size_t)e * a.D;
  for (int t = 0; t < a.S; ++t) {
    const size_t xoff = (size_t)t * a.D;
    double acc = 0.0;
    int c = c0;
    if (a.vec) {
      for (c = c0 + 4 * lane; c + 3 < c1; c += 4 * kWave) {
        const float4 w = *reinterpret_cast<const float4 *>(wrow + c);
        float x0, x1, x2, x3;
        if (a.x_bf16) {
          const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(a.x) + xoff + c);
          x0 = __uint_as_float(u.x << 16);
          x1 = __uint_as_float(u.x & 0xffff0000u);
          x2 = __uint_as_float(u.y << 16);
          x3 = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 xv = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) + xoff + c);
          x0 = xv.x;
          x1 = xv.y;
          x2 = xv.z;
          x3 = xv.w;
        }
        acc = fma((double)w.x, (double)x0, acc);
        acc = fma((double)w.y, (double)x1, acc);
        acc = fma((double)w.z, (double)x2, acc);
        acc = fma((double)w.w, (double)x3, acc);
      }
    } else {
      for (c = c0 + lane; c < c1; c += kWave) acc = fma((double)wrow[c], (double)x_at(a.x, a.x_bf16, xoff + c), acc);
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) a.partial[((size_t)t * a.E + e) * a.splits + sp] = acc;
  }
}

__global__ __launch_bounds__(kBlock) void k_route_select(RouteArgs a) {
  __shared__ double s_c[kWaves][kMaxE];    // scores of the token a wave is ranking
  __shared__ double s_sig[kWaves][kMaxK];  // sigma of its selections, then the final weights
  __shared__ int s_pidx[kRows];            // [t * K + k]: selections of every token
  __shared__ float s_pw[kRows];            // [t * K + k]: final f32 weights
  __shared__ int s_n[kTokens];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int E = a.E, K = a.K, S = a.S;

  const int nper = (E + kWave - 1) / kWave;
  for (int t = wid; t < S; t += kWaves) {
    // logit of each expert this lane holds: its splits summed in split order (kept for the
    // logits tap), then sigma and the choice score.
    double sig[kPerLane], sc[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      sig[i] = 0.0;
      sc[i] = 0.0;
      const int e = lane + kWave * i;
      if (i < nper && e < E) {
        const double *p = a.partial + ((size_t)t * E + e) * a.splits;
        double l = 0.0;
        for (int s = 0; s < a.splits; ++s) l += p[s];
        a.logits[(size_t)t * E + e] = l;
        sig[i] = 1.0 / (1.0 + exp(-l));
        double c = sig[i] + (double)a.bias[e];
        if (c != c) c = -__builtin_inf();  // NaN ranks last, so the selection stays a permutation
        sc[i] = c;
        s_c[wid][e] = c;
      }
    }
    wave_sync();
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + kWave * i;
      if (i < nper && e < E) {
        const double c = sc[i];
        int rank = 0;
        int f = 0;
        for (; f + 3 < E; f += 4) {
          const double c0 = s_c[wid][f], c1 = s_c[wid][f + 1], c2 = s_c[wid][f + 2], c3 = s_c[wid][f + 3];
          rank += (c0 > c || (c0 == c && f < e)) ? 1 : 0;
          rank += (c1 > c || (c1 == c && f + 1 < e)) ? 1 : 0;
          rank += (c2 > c || (c2 == c && f + 2 < e)) ? 1 : 0;
          rank += (c3 > c || (c3 == c && f + 3 < e)) ? 1 : 0;
        }
        for (; f < E; ++f) {
          const double cf = s_c[wid][f];
          rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
        }
        if (rank < K) {
          s_pidx[t * K + rank] = e;
          s_sig[wid][rank] = sig[i];
          if (S == 1 && a.table) {
            // one token: row = rank, so the expert's tensors can be placed now
            RowDesc *rd = a.out->rows + rank;
            rd->t[0] = a.table[e];
            rd->t[1] = a.table[kMaxE + e];
            rd->t[2] = a.table[2 * kMaxE + e];
          }
        }
      }
    }
    wave_sync();
    if (lane == 0) {
      int n = K;
      const double p = (double)a.topp;
      if (p > 0.0 && p < 1.0) {
        double total = 0.0;
        for (int k = 0; k < K; ++k) total += s_sig[wid][k];
        const double thr = p * total;
        double run = 0.0;
        for (int m = 1; m <= K; ++m) {
          run += s_sig[wid][m - 1];
          if (run >= thr) {
            n = m;
            break;
          }
        }
      }
      double den = 0.0;
      if (a.norm_topk)
        for (int k = 0; k < n; ++k) den += s_sig[wid][k];
      const double scale = (double)a.routed_scale;
      for (int k = 0; k < n; ++k) s_sig[wid][k] = (a.norm_topk ? s_sig[wid][k] / den : s_sig[wid][k]) * scale;
      s_n[t] = n;
    }
    wave_sync();
    const int n = s_n[t];
    const float wk = lane < n ? (float)s_sig[wid][lane] : 0.f;
    RouteTok *rt = a.out->route + t;
    if (lane == 0) rt->n = n;
    rt->idx[lane] = lane < K ? s_pidx[t * K + lane] : -1;
    rt->w[lane] = wk;
    if (lane < K) s_pw[t * K + lane] = wk;
    wave_sync();
  }
  __syncthreads();

  // ---- group build (wave 0): pairs (t, k < n_t) in token-major order; distinct experts in
  // first-appearance order; an expert's rows are its tokens in ascending order.
  if (wid != 0) return;
  GroupDev *G = &a.out->g;
  if (S == 1) {
    // one token: the selections are already distinct, one row each, in route order
    const int n = s_n[0];
    if (lane < n) {
      const int e = s_pidx[lane];
      const float w = s_pw[lane];
      G->entry_expert[lane] = e;
      G->entry_row0[lane] = lane;
      G->row_token[lane] = 0;
      G->row_expert[lane] = e;
      G->row_weight[lane] = w;
      G->red_rows[lane] = lane;
      RowDesc *rd = a.out->rows + lane;
      rd->token = 0;
      rd->weight = w;
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
    return;
  }
  int my_t = -1, my_k = 0, base = 0;
  for (int t = 0; t < S; ++t) {
    const int nt = s_n[t];
    if (lane >= base && lane < base + nt) {
      my_t = t;
      my_k = lane - base;
    }
    base += nt;
  }
  const int npairs = base;  // <= S * K <= 64
  const int my_e = my_t >= 0 ? s_pidx[my_t * K + my_k] : -1;
  const float my_w = my_t >= 0 ? s_pw[my_t * K + my_k] : 0.f;

  int ent_e = -1, n_ent = 0, my_entry = -1;
  for (int p = 0; p < npairs; ++p) {
    const int ep = __shfl(my_e, p, kWave);
    const unsigned long long hit = __ballot(lane < n_ent && ent_e == ep);
    int j;
    if (hit) {
      j = __ffsll((long long)hit) - 1;
    } else {
      j = n_ent;
      if (lane == n_ent) ent_e = ep;
      ++n_ent;
    }
    if (lane == p) my_entry = j;
  }
  // rows per entry and the rank of each pair inside its entry
  int cnt = 0, rank = 0;
  for (int p = 0; p < npairs; ++p) {
    const int jp = __shfl(my_entry, p, kWave);
    cnt += (jp == lane) ? 1 : 0;
    rank += (p < lane && jp == my_entry) ? 1 : 0;
  }
  int row0 = 0;
  for (int j = 0; j < n_ent; ++j) {
    const int cj = __shfl(cnt, j, kWave);
    row0 += (j < lane) ? cj : 0;
  }
  const int my_row = __shfl(row0, my_entry < 0 ? 0 : my_entry, kWave) + rank;

  if (lane < n_ent) {
    G->entry_expert[lane] = ent_e;
    G->entry_row0[lane] = row0;
  }
  if (lane == n_ent) G->entry_row0[lane] = npairs;
  if (lane < npairs) {
    G->row_token[my_row] = my_t;
    G->row_expert[my_row] = my_e;
    G->row_weight[my_row] = my_w;
    G->red_rows[lane] = my_row;
    RowDesc *rd = a.out->rows + my_row;
    if (a.table) {
      rd->t[0] = a.table[my_e];
      rd->t[1] = a.table[kMaxE + my_e];
      rd->t[2] = a.table[2 * kMaxE + my_e];
    }
    rd->token = my_t;
    rd->weight = my_w;
  }
  int tb = 0;
  for (int t = 0; t < S; ++t) tb += (t < lane) ? s_n[t] : 0;
  if (lane <= S) G->tok_row0[lane] = tb;
  if (lane == 0) {
    G->n_entries = n_ent;
    G->n_rows = npairs;
    G->S = S;
    G->reserved = 0;
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  const int units = a.E * a.splits;
  hipLaunchKernelGGL(k_route_gemv, dim3((units + kWaves - 1) / kWaves), dim3(kBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_select, dim3(1), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace i4moe
