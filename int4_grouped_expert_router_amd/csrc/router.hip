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

#include "common.h"

namespace i4moe {
namespace {

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

// One wave's dot product of a W row segment [c0, c1) with x row t, in f64 (every f32 x f32
// or f32 x bf16 product is exact in f64).  Vector path: four float4 chunks per lane in flight
// per batch (addresses clamped into the segment, so the loads are unconditional), FMAs in
// column order.
template <bool XBF>
__device__ __forceinline__ double gemv_vec(const float *wrow, const void *x, size_t xoff, int c0, int c1, int lane) {
  double acc = 0.0;
  for (int c = c0 + 4 * lane; c < c1; c += 16 * kWave) {
    float4 w[4];
    float xv[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cj = c + 4 * kWave * j < c1 ? c + 4 * kWave * j : c;
      w[j] = *reinterpret_cast<const float4 *>(wrow + cj);
      if constexpr (XBF) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + xoff + cj);
        xv[j][0] = __uint_as_float(u.x << 16);
        xv[j][1] = __uint_as_float(u.x & 0xffff0000u);
        xv[j][2] = __uint_as_float(u.y << 16);
        xv[j][3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 q = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + xoff + cj);
        xv[j][0] = q.x;
        xv[j][1] = q.y;
        xv[j][2] = q.z;
        xv[j][3] = q.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c + 4 * kWave * j < c1) {
        acc = fma((double)w[j].x, (double)xv[j][0], acc);
        acc = fma((double)w[j].y, (double)xv[j][1], acc);
        acc = fma((double)w[j].z, (double)xv[j][2], acc);
        acc = fma((double)w[j].w, (double)xv[j][3], acc);
      }
    }
  }
  return acc;
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
    if (a.vec) {
      acc = a.x_bf16 ? gemv_vec<true>(wrow, a.x, xoff, c0, c1, lane) : gemv_vec<false>(wrow, a.x, xoff, c0, c1, lane);
    } else {
      for (int c = c0 + lane; c < c1; c += kWave) acc = fma((double)wrow[c], (double)x_at(a.x, a.x_bf16, xoff + c), acc);
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) a.partial[((size_t)t * a.E + e) * a.splits + sp] = acc;
  }
}

constexpr int kTabWords = 3 * sizeof(TensorDesc) / 4;          // tensor words of a row descriptor
constexpr int kLiveWord = offsetof(TensorDesc, live) / 4;     // t[0].live inside a row descriptor
constexpr int kDescWords = sizeof(RowDesc) / 4;               // 32
constexpr int kDescPerThread = kRows * kDescWords / kBlock;   // 8
constexpr int kTabPrefetchE = 64;                             // experts whose records are staged early

// One workgroup; wave w ranks tokens w, w + 4, ...  The kernel runs once per layer on one CU, so
// it is written for latency: every global read is issued in a batch (one memory round trip per
// phase), and the code is kept small (no unrolled per-expert arrays), since instruction fetch
// of a cold kernel is on its critical path too.
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Tokens are ranked in passes of up to four; a token gets 4 / (tokens in the pass) waves.
// Dynamic LDS per token slot: np doubles (split partials), E doubles (logits), E doubles
// (choice scores), E floats (bias), wpt * E ints (rank counts per wave of the token).
__host__ __device__ inline int select_slots(int S) { return S < kWaves ? S : kWaves; }
__host__ __device__ inline size_t select_slot_doubles(int E, int splits, int wpt) {
  return (size_t)E * splits + 3 * (size_t)E + (E + 1) / 2 + ((size_t)wpt * E + 1) / 2;
}
size_t select_lds_bytes(int E, int splits, int S) {
  const int slots = select_slots(S);
  return 8 * (size_t)slots * select_slot_doubles(E, splits, kWaves / slots);
}

// One workgroup, run once per layer on one CU, so written for latency: every global read of
// a phase is issued in one batch, the waves of a token split its experts and its comparisons,
// and the code is kept small.
__global__ __launch_bounds__(kBlock) void k_route_select(RouteArgs a) {
  extern __shared__ double s_dyn[];
  __shared__ double s_sig[kWaves][kMaxK];  // sigma of the selections, per token slot
  __shared__ int s_pidx[kRows];            // [t * K + k]: selections of every token
  __shared__ float s_pw[kRows];            // [t * K + k]: final f32 weights
  __shared__ int s_n[kTokens];
  __shared__ int s_row_e[kRows], s_row_t[kRows];
  __shared__ float s_row_w[kRows];
  __shared__ int s_rows;
  __shared__ uint32_t s_tab[kTabPrefetchE * kDescWords];  // expert records, when E is small

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int E = a.E, K = a.K, S = a.S, splits = a.splits;
  const int np = E * splits;  // <= kMaxE partials per token (checked on the host)
  const int nq = np + E;
  const int slots = select_slots(S), wpt = kWaves / slots;
  const int slot = wid / wpt, u = wid - slot * wpt;  // token slot of this wave, index inside it
  const int gt = u * kWave + lane, gn = wpt * kWave;  // thread index / count within the slot

  double *s_v = s_dyn + slot * select_slot_doubles(E, splits, wpt);  // partials
  double *s_c = s_v + np;                   // logits
  double *s_x = s_c + E;                    // choice scores
  double *s_sg = s_x + E;                   // sigma
  float *s_b = reinterpret_cast<float *>(s_sg + E);
  int *s_r = reinterpret_cast<int *>(s_b + ((E + 1) & ~1));  // [wpt][E] rank counts

  // With few experts, every expert's 128-byte record is loaded now, in the same batch as the
  // partials, so the row descriptors need no further memory round trip at the end.
  const bool tab_pre = a.table != nullptr && E <= kTabPrefetchE;
  uint32_t tv[kTabPrefetchE * kDescWords / kBlock];
  if (tab_pre) {
    const uint32_t *tsrc = reinterpret_cast<const uint32_t *>(a.table);
#pragma unroll
    for (int j = 0; j < kTabPrefetchE * kDescWords / kBlock; ++j) tv[j] = tsrc[min(tid + j * kBlock, E * kDescWords - 1)];
  }

  for (int t0 = 0; t0 < S; t0 += slots) {
    const int t = t0 + slot;
    const bool act = slot < slots && t < S;
    // the token's partials ([e][split], contiguous) and the bias: clamped, unconditional
    // loads, eight in flight per thread, no branch between them
    if (act) {
      const uint64_t *src = reinterpret_cast<const uint64_t *>(a.partial + (size_t)t * np);
      const uint32_t *bsrc = reinterpret_cast<const uint32_t *>(a.bias);
      for (int q0 = 0; q0 < nq; q0 += 8 * gn) {
        uint64_t pv[8];
        uint32_t bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int q = q0 + j * gn + gt;
          pv[j] = src[min(q, np - 1)];
          bv[j] = bsrc[min(max(q - np, 0), E - 1)];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int q = q0 + j * gn + gt;
          if (q < np)
            s_v[q] = __longlong_as_double((long long)pv[j]);
          else if (q < nq)
            s_b[q - np] = __uint_as_float(bv[j]);
        }
      }
    }
    __syncthreads();
    // logit = the splits summed in split order; choice score c = sigma + bias, NaN ranked last
    if (act) {
      for (int e = gt; e < E; e += gn) {
        double l = 0.0;
        for (int sp = 0; sp < splits; ++sp) l += s_v[e * splits + sp];
        s_c[e] = l;
        const double sg = 1.0 / (1.0 + exp(-l));
        s_sg[e] = sg;
        double c = sg + (double)s_b[e];
        if (c != c) c = -__builtin_inf();
        s_x[e] = c;
      }
    }
    __syncthreads();
    // rank in (score desc, index asc), the comparisons split over the token's waves: wave u
    // counts the experts f = u, u + wpt, ... that beat e
    if (act) {
      for (int e = lane; e < E; e += kWave) {
        const double c = s_x[e];
        int rank = 0;
        int f = u;
        for (; f + 7 * wpt < E; f += 8 * wpt) {  // eight broadcast reads in flight
          double cf[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) cf[j] = s_x[f + j * wpt];
#pragma unroll
          for (int j = 0; j < 8; ++j) rank += (cf[j] > c || (cf[j] == c && f + j * wpt < e)) ? 1 : 0;
        }
        for (; f < E; f += wpt) {
          const double cf = s_x[f];
          rank += (cf > c || (cf == c && f < e)) ? 1 : 0;
        }
        s_r[u * E + e] = rank;
      }
    }
    __syncthreads();
    // the experts of rank < K are the selection, in order; sigma from the raw logit
    if (act && u == 0) {
      for (int e = lane; e < E; e += kWave) {
        int rank = 0;
        for (int w = 0; w < wpt; ++w) rank += s_r[w * E + e];
        if (rank < K) {
          s_pidx[t * K + rank] = e;
          s_sig[slot][rank] = s_sg[e];
        }
      }
    }
    __syncthreads();
    if (act && u == 0) {
      // top-p, norm, scale: lane k holds sigma_k; the sums run over k in order (uniform values)
      const double my_sig = lane < K ? s_sig[slot][lane] : 0.0;
      int n = K;
      const double p = (double)a.topp;
      if (p > 0.0 && p < 1.0) {
        double total = 0.0;
        for (int k = 0; k < K; ++k) total += readlane_f64(my_sig, k);
        const double thr = p * total;
        double run = 0.0;
        for (int m = 1; m <= K; ++m) {
          run += readlane_f64(my_sig, m - 1);
          if (run >= thr) {
            n = m;
            break;
          }
        }
      }
      double den = 0.0;
      if (a.norm_topk)
        for (int k = 0; k < n; ++k) den += readlane_f64(my_sig, k);
      const double wv = (a.norm_topk ? my_sig / den : my_sig) * (double)a.routed_scale;
      if (lane == 0) s_n[t] = n;
      const float wk = lane < n ? (float)wv : 0.f;
      RouteTok *rt = a.out->route + t;
      if (lane == 0) rt->n = n;
      rt->idx[lane] = lane < K ? s_pidx[t * K + lane] : -1;
      rt->w[lane] = wk;
      if (lane < K) s_pw[t * K + lane] = wk;
    }
    if (act)
      for (int e = gt; e < E; e += gn) a.logits[(size_t)t * E + e] = s_c[e];  // logits tap
    __syncthreads();
  }

  // ---- group build (wave 0): pairs (t, k < n_t) in token-major order; distinct experts in
  // first-appearance order; an expert's rows are its tokens in ascending order.
  if (wid == 0) {
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
        s_row_e[lane] = e;
        s_row_t[lane] = 0;
        s_row_w[lane] = w;
      }
      if (lane == 0) {
        G->entry_row0[n] = n;
        G->tok_row0[0] = 0;
        G->tok_row0[1] = n;
        G->n_entries = n;
        G->n_rows = n;
        G->S = 1;
        G->reserved = 0;
        s_rows = n;
      }
    } else {
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
        s_row_e[my_row] = my_e;
        s_row_t[my_row] = my_t;
        s_row_w[my_row] = my_w;
      }
      int tb = 0;
      for (int t = 0; t < S; ++t) tb += (t < lane) ? s_n[t] : 0;
      if (lane <= S) G->tok_row0[lane] = tb;
      if (lane == 0) {
        G->n_entries = n_ent;
        G->n_rows = npairs;
        G->S = S;
        G->reserved = 0;
        s_rows = npairs;
      }
    }
  }
  __syncthreads();

  // ---- row descriptors: 32 words per row (the expert's three tensor records, token, weight),
  // every row of the buffer rewritten, rows past the group cleared so a row's own record says
  // whether it is live.  All table reads are in flight together.
  const int rows = s_rows;
  if (tab_pre) {
#pragma unroll
    for (int j = 0; j < kTabPrefetchE * kDescWords / kBlock; ++j) s_tab[tid + j * kBlock] = tv[j];
    __syncthreads();
  }
  uint32_t v[kDescPerThread];
#pragma unroll
  for (int j = 0; j < kDescPerThread; ++j) {
    const int q = tid + j * kBlock;
    const int row = q / kDescWords, d = q % kDescWords;
    const int e = row < rows ? s_row_e[row] : 0;
    const int dd = d < kTabWords ? d : 0;
    v[j] = tab_pre ? s_tab[e * kDescWords + dd]
                   : (a.table ? reinterpret_cast<const uint32_t *>(a.table + e)[dd] : 0u);
  }
#pragma unroll
  for (int j = 0; j < kDescPerThread; ++j) {
    const int q = tid + j * kBlock;
    const int row = q / kDescWords, d = q % kDescWords;
    uint32_t val = 0u;
    if (row < rows && a.table) {
      if (d == kLiveWord)
        val = 1u;
      else if (d < kTabWords)
        val = v[j];
      else if (d == kTabWords)
        val = (uint32_t)s_row_t[row];
      else
        val = __float_as_uint(s_row_w[row]);
    }
    reinterpret_cast<uint32_t *>(a.out->rows)[q] = val;
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  const int units = a.E * a.splits;
  const size_t lds = select_lds_bytes(a.E, a.splits, a.S);
  static bool lds_raised = false;
  if (lds > 64 * 1024 && !lds_raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_route_select),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_route_gemv, dim3((units + kWaves - 1) / kWaves), dim3(kBlock), 0, st, t0, nullptr, 0, a);
  else
    hipLaunchKernelGGL(k_route_gemv, dim3((units + kWaves - 1) / kWaves), dim3(kBlock), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_route_select, dim3(1), dim3(kBlock), lds, st, nullptr, t1, 0, a);
  else
    hipLaunchKernelGGL(k_route_select, dim3(1), dim3(kBlock), lds, st, a);
  return hipGetLastError();
}

}  // namespace i4moe
