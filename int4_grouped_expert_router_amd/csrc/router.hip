// Device router for decode (gfx950): one launch computes the E x D logits GEMV for S tokens,
// then the last workgroup to finish does the selection and builds the expert group.
//
// Source: the device-router commit ("First increment of the #431 plan") on the page "Commit
// history of c/backend_cuda.cu": logits GEMV + sigmoid, bias-augmented top-K by choice with
// strict-'>' tie-breaking, weights from the raw logit, route-level top-p truncation,
// norm_topk, routed_scale, packed result; the batched router over S rows of the
// GPU-resident-pipeline commit; the S<=4 small-batch groups of the COLI_GROUP_ASYNC page.
//
// Precision: the f32 x f32 (or f32 x bf16) products are exact in f64 and are summed in f64;
// sigmoid, scores, top-p, norm and scale are f64; each weight is rounded to f32 once.  The
// selection therefore decides on f64 values, the same precision the CPU reference uses.
//
// Selection runs one wavefront per token: each lane holds up to 16 experts (e = lane + 64 i)
// and every round takes the lexicographic maximum of (score descending, index ascending) over
// the wave, which is exactly the first strictly-greater element of an ascending scan.
#include "common.h"

namespace i4moe {
namespace {

constexpr int kPerLane = kMaxE / kWave;  // 16

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float x_at(const void *x, int bf16, size_t i) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(x)[i]) << 16);
  return static_cast<const float *>(x)[i];
}

// Better candidate in (score desc, index asc) order; index < 0 means "no candidate".
__device__ __forceinline__ bool better(double c1, int e1, double c2, int e2) {
  if (e1 < 0) return false;
  if (e2 < 0) return true;
  return c1 > c2 || (c1 == c2 && e1 < e2);
}

// Order this wave's LDS traffic (lanes of one wave exchanging through shared memory).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kBlock) void k_route(RouteArgs a) {
  __shared__ int s_last;
  __shared__ double s_w64[kBlock / kWave][kMaxK];  // per-wave scratch for one token
  __shared__ int s_pidx[kRows];                    // [t * K + k]: selections of every token
  __shared__ float s_pw[kRows];                    // [t * K + k]: final f32 weights
  __shared__ int s_n[kTokens];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int unit = blockIdx.x * (kBlock / kWave) + wid;  // (expert row, column split)

  // ---- GEMV: partial[t][e][split] = sum over the split's columns of W[e][c] * x[t][c].
  if (unit < a.E * a.splits) {
    const int e = unit / a.splits;
    const int sp = unit - e * a.splits;
    const int c0 = sp * a.cols_per_split;
    const int c1 = min(a.D, c0 + a.cols_per_split);
    const float *wrow = a.W + (size_t)e * a.D;
    for (int t = 0; t < a.S; ++t) {
      const size_t xoff = (size_t)t * a.D;
      double acc = 0.0;
      for (int c = c0 + lane; c < c1; c += kWave)
        acc = fma((double)wrow[c], (double)x_at(a.x, a.x_bf16, xoff + c), acc);
      acc = wave_sum_f64(acc);
      if (lane == 0) a.partial[((size_t)t * a.E + e) * a.splits + sp] = acc;
    }
  }

  // ---- the last workgroup to finish sees every partial (device-scope release/acquire).
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(a.counter, 1u);
    s_last = (prev == gridDim.x - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // logits[t][e]: the splits of one (t, e) summed in split order.
  for (int i = threadIdx.x; i < a.S * a.E; i += kBlock) {
    const double *p = a.partial + (size_t)i * a.splits;
    double l = 0.0;
    for (int s = 0; s < a.splits; ++s) l += p[s];
    a.logits[i] = l;
  }
  __threadfence_block();
  __syncthreads();

  // ---- selection, one wave per token.
  const int K = a.K;
  for (int t = wid; t < a.S; t += kBlock / kWave) {
    double sig[kPerLane], sc[kPerLane];
    bool taken[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + kWave * i;
      taken[i] = true;
      sig[i] = 0.0;
      sc[i] = 0.0;
      if (e < a.E) {
        const double l = a.logits[(size_t)t * a.E + e];
        sig[i] = 1.0 / (1.0 + exp(-l));
        sc[i] = sig[i] + (double)a.bias[e];
        taken[i] = false;
      }
    }
    for (int k = 0; k < K; ++k) {
      // this lane's best unchosen expert: ascending scan, strict '>'
      double bc = 0.0, bs = 0.0;
      int be = -1;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) {
        if (!taken[i] && (be < 0 || sc[i] > bc)) {
          bc = sc[i];
          bs = sig[i];
          be = lane + kWave * i;
        }
      }
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) {
        const double oc = __shfl_xor(bc, m, kWave);
        const double os = __shfl_xor(bs, m, kWave);
        const int oe = __shfl_xor(be, m, kWave);
        if (better(oc, oe, bc, be)) {
          bc = oc;
          bs = os;
          be = oe;
        }
      }
      // every lane now holds the same winner
#pragma unroll
      for (int i = 0; i < kPerLane; ++i)
        if (lane + kWave * i == be) taken[i] = true;
      if (lane == k) {
        s_pidx[t * K + k] = be;
        s_w64[wid][k] = bs;
      }
    }
    wave_sync();
    if (lane == 0) {
      int n = K;
      const double p = (double)a.topp;
      if (p > 0.0 && p < 1.0) {
        double total = 0.0;
        for (int k = 0; k < K; ++k) total += s_w64[wid][k];
        const double thr = p * total;
        double run = 0.0;
        for (int m = 1; m <= K; ++m) {
          run += s_w64[wid][m - 1];
          if (run >= thr) {
            n = m;
            break;
          }
        }
      }
      double den = 0.0;
      if (a.norm_topk)
        for (int k = 0; k < n; ++k) den += s_w64[wid][k];
      const double scale = (double)a.routed_scale;
      for (int k = 0; k < n; ++k) s_w64[wid][k] = (a.norm_topk ? s_w64[wid][k] / den : s_w64[wid][k]) * scale;
      s_n[t] = n;
    }
    wave_sync();
    const int n = s_n[t];
    const float wk = lane < n ? (float)s_w64[wid][lane] : 0.f;
    RouteTok *rt = a.route + t;
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
  const int S = a.S;
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

  GroupDev *G = a.group;
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
  }
  int tb = 0;
  for (int t = 0; t < S; ++t) tb += (t < lane) ? s_n[t] : 0;
  if (lane <= S) G->tok_row0[lane] = tb;
  if (lane == 0) {
    G->n_entries = n_ent;
    G->n_rows = npairs;
    G->S = S;
    G->reserved = 0;
    *a.counter = 0u;  // ready for the next launch
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
  const int units = a.E * a.splits;
  const int blocks = (units + 3) / 4;
  hipLaunchKernelGGL(k_route, dim3(blocks), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace i4moe
