// Expert selection of the device router, shared by the select kernel and the fused
// select-in-dual path of the projection kernel (one token).  See router.hip for the method.
#pragma once

#include <cstddef>

#include "common.h"

namespace i4moe {

constexpr int kWavesPerBlock = kBlock / kWave;                 // 4
constexpr int kTabWords = 3 * sizeof(TensorDesc) / 4;          // tensor words of a row descriptor
constexpr int kLiveWord = offsetof(TensorDesc, live) / 4;     // t[0].live inside a row descriptor
constexpr int kDescWords = sizeof(RowDesc) / 4;               // 32
constexpr int kDescPerThread = kRows * kDescWords / kBlock;   // 8
constexpr int kTabPrefetchE = 64;                             // experts whose records are staged early
constexpr int kTabPerThread = kTabPrefetchE * kDescWords / kBlock;

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Tokens are ranked in passes of up to four; a token gets 4 / (tokens in the pass) waves.
// Dynamic LDS per token slot: np doubles (split partials), E doubles (logits), E doubles
// (choice scores), E doubles (sigma), E floats (bias), wpt * E ints (rank counts per wave).
__host__ __device__ inline int select_slots(int S) { return S < kWavesPerBlock ? S : kWavesPerBlock; }
__host__ __device__ inline size_t select_slot_doubles(int E, int splits, int wpt) {
  return (size_t)E * splits + 3 * (size_t)E + (E + 1) / 2 + ((size_t)wpt * E + 1) / 2;
}
__host__ __device__ inline size_t select_lds_bytes(int E, int splits, int S) {
  const int slots = select_slots(S);
  return 8 * (size_t)slots * select_slot_doubles(E, splits, kWavesPerBlock / slots);
}

// Workgroup-shared results and scratch of a selection (static __shared__ arrays of the kernel).
struct SelShared {
  double (*sig)[kMaxK];  // [slot][k]: sigma of the selections
  int *pidx;             // [t * K + k]: selections of every token
  float *pw;             // [t * K + k]: final f32 weights
  int *n;                // [t]: kept count after top-p
  int *row_e, *row_t;    // per group row: expert, token
  float *row_w;          // per group row: weight
  int *rows;             // group rows
  const uint32_t *tab;   // staged expert records [E][32] (E <= kTabPrefetchE), or null
};

// Expert records loaded early, in the same batch as the first partials (E <= kTabPrefetchE).
__device__ __forceinline__ void table_prefetch(uint32_t (&tv)[kTabPerThread], const ExpertRec *table, int E) {
  const uint32_t *tsrc = reinterpret_cast<const uint32_t *>(table);
#pragma unroll
  for (int j = 0; j < kTabPerThread; ++j) tv[j] = tsrc[min((int)threadIdx.x + j * kBlock, E * kDescWords - 1)];
}
__device__ __forceinline__ void table_stage(uint32_t *s_tab, const uint32_t (&tv)[kTabPerThread]) {
#pragma unroll
  for (int j = 0; j < kTabPerThread; ++j) s_tab[threadIdx.x + j * kBlock] = tv[j];
}

// One pass: tokens t0 .. t0 + slots - 1.  All threads of the workgroup call it (it holds
// workgroup barriers).  With `out`, the pass also writes the route records and the logits tap.
static __device__ __forceinline__ void select_pass(const RouteArgs &a, double *s_dyn, int t0, const SelShared &sh, bool out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int E = a.E, K = a.K, S = a.S, splits = a.splits;
  const int np = E * splits;  // <= kMaxE partials per token (checked on the host)
  const int nq = np + E;
  const int slots = select_slots(S), wpt = kWavesPerBlock / slots;
  const int slot = wid / wpt, u = wid - slot * wpt;  // token slot of this wave, index inside it
  const int gt = u * kWave + lane, gn = wpt * kWave;  // thread index / count within the slot
  double *s_v = s_dyn + slot * select_slot_doubles(E, splits, wpt);  // partials
  double *s_c = s_v + np;                   // logits
  double *s_x = s_c + E;                    // choice scores
  double *s_sg = s_x + E;                   // sigma
  float *s_b = reinterpret_cast<float *>(s_sg + E);
  int *s_r = reinterpret_cast<int *>(s_b + ((E + 1) & ~1));  // [wpt][E] rank counts
  int *s_pidx = sh.pidx;
  float *s_pw = sh.pw;
  int *s_n = sh.n;
  double (*s_sig)[kMaxK] = sh.sig;

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
    if (out) {
      RouteTok *rt = a.out->route + t;
      if (lane == 0) rt->n = n;
      rt->idx[lane] = lane < K ? s_pidx[t * K + lane] : -1;
      rt->w[lane] = wk;
    }
    if (lane < K) s_pw[t * K + lane] = wk;
  }
  if (act && out)
    for (int e = gt; e < E; e += gn) a.logits[(size_t)t * E + e] = s_c[e];  // logits tap
  __syncthreads();

}

// Group record and row descriptors of the finished selection (all threads of the workgroup;
// holds workgroup barriers).
static __device__ __forceinline__ void publish_group(const RouteArgs &a, const SelShared &sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int K = a.K, S = a.S;
  const int *s_pidx = sh.pidx;
  const float *s_pw = sh.pw;
  const int *s_n = sh.n;
  int *s_row_e = sh.row_e, *s_row_t = sh.row_t;
  float *s_row_w = sh.row_w;
  int &s_rows = *sh.rows;
  const bool tab_pre = sh.tab != nullptr;
  const uint32_t *s_tab = sh.tab;

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
  const int rows = *sh.rows;
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

}  // namespace i4moe
