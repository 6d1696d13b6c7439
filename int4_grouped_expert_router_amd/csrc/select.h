// Expert selection of the device router, shared by the select kernel (any S) and the dual
// projection, which runs the selection of one token itself.  See router.hip for the method.
#pragma once

#include <cstddef>

#include "common.h"

namespace i4moe {

constexpr int kWavesPerBlock = kBlock / kWave;                 // 4
constexpr int kTabWords = 3 * sizeof(TensorDesc) / 4;          // tensor words of a row descriptor
constexpr int kLiveWord = offsetof(TensorDesc, live) / 4;     // t[0].live inside a row descriptor
constexpr int kRankWord = kLiveWord + sizeof(TensorDesc) / 4;  // t[1].live: the row's rank in its entry
constexpr int kSizeWord = kRankWord + sizeof(TensorDesc) / 4;  // t[2].live: its entry's row count
constexpr int kDescWords = sizeof(RowDesc) / 4;               // 32
constexpr int kTabPrefetchE = 64;                             // fused selection: records staged early
constexpr int kTabPerThread = kTabPrefetchE * kDescWords / kBlock;
constexpr int kSelTabE = 256;                                 // select kernel: records staged early
constexpr int kSelTabPerThread = kSelTabE * kDescWords / kBlock;

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Tokens are selected in passes of up to four, one wave per token.  Dynamic LDS per token
// slot: E doubles (choice scores) and E doubles (sigma).
__host__ __device__ inline int select_slots(int S) { return S < kWavesPerBlock ? S : kWavesPerBlock; }
__host__ __device__ inline size_t select_lds_bytes(int E, int S) { return 16 * (size_t)select_slots(S) * E; }

// Workgroup-shared results and scratch of a selection (static __shared__ arrays of the kernel).
struct SelShared {
  int *pidx;             // [t * K + k]: selections of every token
  float *pw;             // [t * K + k]: final f32 weights
  int *n;                // [t]: kept count after top-p
  int *row_e, *row_t;    // per group row: expert, token
  float *row_w;          // per group row: weight
  int *row_rank, *row_size;  // per group row: rank in its entry, the entry's row count
  int *rows;             // group rows
  const uint32_t *tab;   // staged expert records [E][32], or null
};

// Expert records loaded early, in the same batch as the scores (E <= N * kBlock / 32).
template <int N>
__device__ __forceinline__ void table_prefetch(uint32_t (&tv)[N], const ExpertRec *table, int E) {
  const uint32_t *tsrc = reinterpret_cast<const uint32_t *>(table);
#pragma unroll
  for (int j = 0; j < N; ++j) tv[j] = tsrc[min((int)threadIdx.x + j * kBlock, E * kDescWords - 1)];
}
// The same through a buffer range of `bytes` (0: the loads read nothing and return zeros), so
// the load pattern does not depend on whether the table is wanted.
template <int N>
__device__ __forceinline__ void table_prefetch_rsrc(uint32_t (&tv)[N], const ExpertRec *table, int bytes) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<ExpertRec *>(table), (short)0, bytes,
                                                                     0x00020000);
#pragma unroll
  for (int j = 0; j < N; ++j) tv[j] = __builtin_amdgcn_raw_buffer_load_b32(r, 4 * ((int)threadIdx.x + j * kBlock), 0, 0);
}
template <int N>
__device__ __forceinline__ void table_stage(uint32_t *s_tab, const uint32_t (&tv)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) s_tab[threadIdx.x + j * kBlock] = tv[j];
}

// Top-p, norm and scale of one token's selection.  Lane k < K holds sigma of selection k;
// control is wave-uniform.  The running sums run over k in order, one chain of f64 adds whose
// prefix k lane k keeps: the top-p total is the whole chain, the cut is the first prefix that
// reaches p * total, and the norm divisor is the kept prefix.  Returns the lane's f32 weight
// (0 from n on) and the kept count n.
__device__ __forceinline__ float finish_weights(const RouteArgs &a, double my_sig, int &n_out) {
  const int lane = threadIdx.x & 63;
  const int K = a.K;
  double run = 0.0, pre = 0.0;
  for (int k = 0; k < K; ++k) {
    run += readlane_f64(my_sig, k);
    if (lane == k) pre = run;
  }
  int n = K;
  const double p = (double)a.topp;
  if (p > 0.0 && p < 1.0) {
    const double thr = p * run;
    const unsigned long long m = __ballot(lane < K && pre >= thr);
    if (m) n = __ffsll((long long)m);
  }
  const double den = a.norm_topk ? readlane_f64(pre, n - 1) : 1.0;
  const double wv = (a.norm_topk ? my_sig / den : my_sig) * (double)a.routed_scale;
  n_out = n;
  return lane < n ? (float)wv : 0.f;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64s(double v) {
  const uint64_t u = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL, ROW_MASK>((int)(uint32_t)u);
  const int hi = dpp_i32<CTRL, ROW_MASK>((int)(uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// The larger of two scores (scores are never NaN: the GEMV maps a NaN score to -inf).
__device__ __forceinline__ double max_score(double x, double y) { return y > x ? y : x; }

// K rounds of the selection for E > 64 (lane e & 63 holds expert e in column e / 64, PER
// columns).  A round takes the largest score among the experts not yet taken (the lane's
// maximum, DPP steps inside rows of 16 lanes, then the four rows) and then the lowest index
// holding it (one ballot per column, lowest column first): the first maximum of an ascending
// scan.  A taken expert's score becomes -inf, and its bit in `taken` keeps it out of the
// ballots should the remaining scores be -inf too.  Lane k < K returns selection k.
template <int PER>
__device__ __forceinline__ int select_rounds(const double *s_x, int E, int K, int lane) {
  double cv[PER];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    const double x = s_x[min(e, E - 1)];
    cv[i] = e < E ? x : -__builtin_inf();
    if (e >= E) taken |= 1u << i;
  }
  int sel_e = 0;
  for (int k = 0; k < K; ++k) {
    double m = cv[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) m = max_score(m, cv[i]);
    m = max_score(m, dpp_f64s<0xB1, 0xF>(m));   // quad_perm [1,0,3,2]
    m = max_score(m, dpp_f64s<0x4E, 0xF>(m));   // quad_perm [2,3,0,1]
    m = max_score(m, dpp_f64s<0x141, 0xF>(m));  // row_half_mirror
    m = max_score(m, dpp_f64s<0x140, 0xF>(m));  // row_mirror: every lane holds its row's maximum
    const double M = max_score(max_score(readlane_f64(m, 0), readlane_f64(m, 16)),
                               max_score(readlane_f64(m, 32), readlane_f64(m, 48)));
    // M is one of the untaken scores, so some column holds it
    int we = 0;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      const unsigned long long hit = __ballot(!((taken >> i) & 1u) && cv[i] == M);
      if (hit) we = kWave * i + __ffsll((long long)hit) - 1;
    }
    const int wc = we / kWave;
    const bool mine = lane == (we & (kWave - 1));
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i == wc && mine) cv[i] = -__builtin_inf();
    if (mine) taken |= 1u << wc;
    if (lane == k) sel_e = we;
  }
  return sel_e;
}

// Inclusive prefix sum over the 64 lanes (Kogge-Stone steps inside rows of 16 lanes, then
// the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += dpp_i32<0x111, 0xF>(v);  // row_shr:1 (lanes without a source add 0)
  v += dpp_i32<0x112, 0xF>(v);  // row_shr:2
  v += dpp_i32<0x114, 0xF>(v);  // row_shr:4
  v += dpp_i32<0x118, 0xF>(v);  // row_shr:8
  v += dpp_i32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_i32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// One pass of the select kernel: tokens t0 .. t0 + slots - 1, wave w on token t0 + w.  All
// threads of the workgroup call it (it holds workgroup barriers); it writes the route records.
//   E <= 64: lane e counts the experts that beat expert e (its rank); ranks below K are the
//            selection positions.
//   E > 64:  K rounds; each takes the largest score not yet taken and, among experts holding
//            it, the lowest index, which is the strict ascending scan itself.
// Both give the experts of rank 0 .. K-1 in the order (score desc, index asc).
template <class F>
__device__ __forceinline__ void select_pass(const RouteArgs &a, double *s_dyn, int t0, const SelShared &sh,
                                            F &&after_loads) {
  const int lane = threadIdx.x & 63;
  const int slot = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int E = a.E, K = a.K, S = a.S;
  double *s_x = s_dyn + (size_t)slot * 2 * E;  // choice scores
  double *s_sg = s_x + E;                       // sigma
  const int t = t0 + slot;
  const bool act = slot < select_slots(S) && t < S;
  // the token's scores: clamped, unconditional loads, four in flight per lane; the first
  // batch is issued before `after_loads` (which may issue loads of its own for later use)
  const double2 *src = a.score + (size_t)min(t, S - 1) * E;
  double2 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = src[min(j * kWave + lane, E - 1)];
  after_loads();
  if (act) {
    for (int e0 = 0; e0 < E; e0 += 4 * kWave) {
      if (e0 > 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = src[min(e0 + j * kWave + lane, E - 1)];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + j * kWave + lane;
        if (e < E) {
          s_x[e] = v[j].x;
          s_sg[e] = v[j].y;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int sel_e = 0;         // lane k < K: expert of selection k
    double my_sig = 0.0;   // lane k < K: its sigma
    if (E <= kWave) {
      const double c = lane < E ? s_x[lane] : 0.0;
      int rank = 0;
      int f = 0;
      for (; f + 8 <= E; f += 8) {  // eight broadcast reads in flight
        double cf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) cf[j] = s_x[f + j];
#pragma unroll
        for (int j = 0; j < 8; ++j) rank += (cf[j] > c || (cf[j] == c && f + j < lane)) ? 1 : 0;
      }
      for (; f < E; ++f) {
        const double cf = s_x[f];
        rank += (cf > c || (cf == c && f < lane)) ? 1 : 0;
      }
      if (lane >= E) rank = lane;
      // each expert's index goes to the lane of its rank
      sel_e = __builtin_amdgcn_ds_permute(rank * 4, lane);
      my_sig = lane < K ? s_sg[sel_e] : 0.0;
    } else {
      const int per = (E + kWave - 1) / kWave;
      sel_e = per <= 2 ? select_rounds<2>(s_x, E, K, lane)
            : per <= 4 ? select_rounds<4>(s_x, E, K, lane)
            : per <= 8 ? select_rounds<8>(s_x, E, K, lane)
                       : select_rounds<16>(s_x, E, K, lane);
      my_sig = lane < K ? s_sg[sel_e] : 0.0;
    }
    int n;
    const float wk = finish_weights(a, my_sig, n);
    if (lane == 0) sh.n[t] = n;
    RouteTok *rt = a.out->route + t;
    if (lane == 0) rt->n = n;
    rt->idx[lane] = lane < K ? sel_e : -1;
    rt->w[lane] = wk;
    if (lane < K) {
      sh.pidx[t * K + lane] = sel_e;
      sh.pw[t * K + lane] = wk;
    }
  }
  __syncthreads();
}

// The selection of one token (S == 1, E <= 64) inside a workgroup of four waves, with one
// workgroup barrier.  Lane e holds expert e's score; each wave counts, for every expert, the
// experts of its quarter that beat it; the counts meet in LDS; the ranks then send each
// expert's index and sigma to the lane of its rank (ds_permute), and every wave finishes
// the weights itself.  `cs` is the lane's (choice score, sigma); `s_cw` [4][64] doubles and
// `s_cnt` [4][64] ints are scratch.  `before_barrier` runs just ahead of the barrier (it
// stages the expert table).  Lane k < K returns selection k's expert in `e_k` and its weight.
struct SelOne {
  int e_k;      // expert of selection `lane` (lanes past E: unspecified)
  float w_k;    // f32 weight of selection `lane` (0 from n on)
  int n;        // kept count
};
template <class F>
__device__ __forceinline__ SelOne select_one(const RouteArgs &a, double2 cs, double (*s_cw)[kWave], int (*s_cnt)[kWave],
                                             F &&before_barrier) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int E = a.E;
  const double c = cs.x;
  s_cw[wid][lane] = c;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kQ = kWave / kWavesPerBlock;  // 16 experts per wave
  const int f0 = wid * kQ;
  double cf[kQ];
#pragma unroll
  for (int j = 0; j < kQ; ++j) cf[j] = s_cw[wid][f0 + j];  // broadcast reads
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kQ; ++j) cnt += (f0 + j < E && (cf[j] > c || (cf[j] == c && f0 + j < lane))) ? 1 : 0;
  s_cnt[wid][lane] = cnt;
  before_barrier();
  __syncthreads();
  int rank = lane;
  if (lane < E) rank = s_cnt[0][lane] + s_cnt[1][lane] + s_cnt[2][lane] + s_cnt[3][lane];
  const uint64_t sb = __double_as_longlong(cs.y);
  SelOne r;
  r.e_k = __builtin_amdgcn_ds_permute(rank * 4, lane);
  const uint32_t lo = __builtin_amdgcn_ds_permute(rank * 4, (int)(uint32_t)sb);
  const uint32_t hi = __builtin_amdgcn_ds_permute(rank * 4, (int)(uint32_t)(sb >> 32));
  const double sig_k = __longlong_as_double(((uint64_t)hi << 32) | lo);
  r.w_k = finish_weights(a, lane < a.K ? sig_k : 0.0, r.n);
  return r;
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
  int *s_row_rank = sh.row_rank, *s_row_size = sh.row_size;
  float *s_row_w = sh.row_w;
  int &s_rows = *sh.rows;
  const bool tab_pre = sh.tab != nullptr;
  const uint32_t *s_tab = sh.tab;

  // ---- group build (wave 0): pairs (t, k < n_t) in token-major order; distinct experts in
  // first-appearance order; an expert's rows are its tokens in ascending order.
  if (wid == 0) {
    GroupDev *G = &a.out->g;
    const bool sh = a.shared_rows != 0;
    if (S == 1) {
      // one token: the selections are already distinct, one row each, in route order (and the
      // shared expert's row after them)
      const int n = s_n[0];
      const int nr = n + (sh ? 1 : 0);
      if (lane < nr) {
        const int e = lane < n ? s_pidx[lane] : kSharedRec;
        const float w = lane < n ? s_pw[lane] : 1.f;
        G->entry_expert[lane] = e;
        G->entry_row0[lane] = lane;
        G->row_token[lane] = 0;
        G->row_expert[lane] = e;
        G->row_weight[lane] = w;
        G->red_rows[lane] = lane;
        s_row_e[lane] = e;
        s_row_t[lane] = 0;
        s_row_w[lane] = w;
        s_row_rank[lane] = 0;
        s_row_size[lane] = 1;
      }
      if (lane == 0) {
        G->entry_row0[nr] = nr;
        G->tok_row0[0] = 0;
        G->tok_row0[1] = nr;
        G->n_entries = nr;
        G->n_rows = nr;
        G->S = 1;
        G->reserved = 0;
        s_rows = nr;
      }
    } else {
      // lane p < npairs holds pair p = (token t, selection k < n_t), token-major.  Token t's
      // first pair is the prefix sum of the kept counts before it (every count is at least 1,
      // so the first pairs rise strictly and a pair's token is the last one starting at or
      // before it).
      const int nl = lane < S ? s_n[lane] : 0;
      const int tok_end = wave_scan_incl(nl);
      const int tok0 = tok_end - nl;
      const int npairs = __builtin_amdgcn_readlane(tok_end, S - 1);  // <= S * K <= 64
      int my_t = -1, my_k = 0;
      for (int t = 0; t < S; ++t) {
        const int b = __builtin_amdgcn_readlane(tok0, t);
        if (lane >= b) {
          my_t = t;
          my_k = lane - b;
        }
      }
      if (lane >= npairs) my_t = -1;
      const int my_e = my_t >= 0 ? s_pidx[my_t * K + my_k] : -1;
      const float my_w = my_t >= 0 ? s_pw[my_t * K + my_k] : 0.f;
      const bool pl = lane < npairs;
      // the pairs of my expert, one ballot per index bit (a token's selections are distinct,
      // so the pairs of one expert are its tokens in ascending order)
      const int ebits = 32 - __clz(a.E > 1 ? a.E - 1 : 1);
      unsigned long long same = __ballot(pl);
      for (int b = 0; b < ebits; ++b) {
        const bool bit = (my_e >> b) & 1;
        const unsigned long long m = __ballot(pl && bit);
        same &= bit ? m : ~m;
      }
      // entries are the experts in first-appearance order: the head pair of an entry is its
      // expert's lowest pair, and the entry's rows are its pairs in pair order
      const int first = pl ? __ffsll((long long)same) - 1 : 0;
      const bool head = pl && first == lane;
      const int cnt = head ? __popcll(same) : 0;
      const unsigned long long fm = __ballot(head);
      const int n_ent = __popcll(fm);
      const int my_entry = __popcll(fm & ((1ull << first) - 1ull));
      // an entry's first row: the pairs of the entries whose heads come before it
      const int row0 = wave_scan_incl(cnt) - cnt;
      const int rank = __popcll(same & ((1ull << lane) - 1ull));
      const int my_row = __shfl(row0, first, kWave) + rank;

      if (head) {
        G->entry_expert[my_entry] = my_e;
        G->entry_row0[my_entry] = row0;
      }
      if (lane == 0) G->entry_row0[n_ent] = npairs;  // n_ent may be 64
      // with the shared expert: its rows npairs + t (one per token t) form the last entry, and
      // each token's reduce list is its routed rows in route order, then its shared row (so a
      // pair's reduce position moves up by one per earlier token)
      if (pl && my_row < kRows) {  // always: the rows are a permutation of the pairs
        G->row_token[my_row] = my_t;
        G->row_expert[my_row] = my_e;
        G->row_weight[my_row] = my_w;
        G->red_rows[lane + (sh ? my_t : 0)] = my_row;
        s_row_e[my_row] = my_e;
        s_row_t[my_row] = my_t;
        s_row_w[my_row] = my_w;
        s_row_rank[my_row] = rank;
        s_row_size[my_row] = __popcll(same);
      }
      if (sh && lane < S) {  // the host keeps npairs + S <= kRows
        const int r = npairs + lane;
        G->row_token[r] = lane;
        G->row_expert[r] = kSharedRec;
        G->row_weight[r] = 1.f;
        G->red_rows[tok_end + lane] = r;
        s_row_e[r] = kSharedRec;
        s_row_t[r] = lane;
        s_row_w[r] = 1.f;
        s_row_rank[r] = lane;
        s_row_size[r] = S;
      }
      if (sh && lane == 0) {
        G->entry_expert[n_ent] = kSharedRec;
        G->entry_row0[n_ent + 1] = npairs + S;
      }
      if (lane < S) G->tok_row0[lane] = tok0 + (sh ? lane : 0);
      if (lane == 0) {
        const int nr = npairs + (sh ? S : 0);
        G->tok_row0[S] = nr;  // S may be 64
        G->n_entries = n_ent + (sh ? 1 : 0);
        G->n_rows = nr;
        G->S = S;
        G->reserved = 0;
        s_rows = nr;
      }
    }
  }
  __syncthreads();

  // ---- row descriptors: 32 words per row (the expert's three tensor records, token, weight)
  // in 16-byte chunks; every row of the buffer rewritten, rows past the group cleared so a
  // row's own record says whether it is live.  All table reads are in flight together.
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  static_assert(kTabWords == kDescWords - 2, "a row descriptor ends with token and weight");
  constexpr int kChunks = kDescWords / 4;
  constexpr int kChunksPerThread = kRows * kChunks / kBlock;
  const int rows = a.table ? *sh.rows : 0;
  u4 v[kChunksPerThread];
#pragma unroll
  for (int j = 0; j < kChunksPerThread; ++j) {
    const int q = tid + j * kBlock;
    const int row = q / kChunks, c = q % kChunks;
    const int e = row < rows ? s_row_e[row] : 0;
    if (tab_pre && e != kSharedRec)  // the shared expert's record is not among the staged ones
      v[j] = *reinterpret_cast<const u4 *>(s_tab + e * kDescWords + 4 * c);
    else
      v[j] = a.table ? reinterpret_cast<const u4 *>(a.table + e)[c] : u4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kChunksPerThread; ++j) {
    const int q = tid + j * kBlock;
    const int row = q / kChunks, c = q % kChunks;
    u4 val = {0u, 0u, 0u, 0u};
    if (row < rows) {
      val = v[j];
      if (c == kLiveWord / 4) val[kLiveWord % 4] = 1u;
      if (c == kRankWord / 4) val[kRankWord % 4] = (uint32_t)s_row_rank[row];
      if (c == kSizeWord / 4) val[kSizeWord % 4] = (uint32_t)s_row_size[row];
      if (c == kChunks - 1) {
        val.z = (uint32_t)s_row_t[row];
        val.w = __float_as_uint(s_row_w[row]);
      }
    }
    reinterpret_cast<u4 *>(a.out->rows)[q] = val;
  }
}

}  // namespace i4moe
