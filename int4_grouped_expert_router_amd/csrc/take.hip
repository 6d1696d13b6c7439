// Take: join the issued slots into the residual (gfx950).
//
// Source: the resident take of "cuda: COLI_CUDA_RESID=1 - expert-group results stay on device"
// (section "What"): the home stream reduces the per-issue slots in issue order, deterministic
// and without atomics, and joins the residual; and the per-expert weighting with a
// fixed-order reduce of the same page.  For token t and column i:
//
//   acc_s = sum over the rows of t in slot s, in route order, of w_row * y_s[row][i]
//   residual[t][i] += acc_0 + acc_1 + ... (issue order)
//
// One thread owns one (t, i); the order of every sum is fixed, so results are bitwise
// reproducible run to run.
#include <hip/hip_ext.h>

#include "common.h"

namespace i4moe {
namespace {

static_assert(kRows == kWave, "take stages one slot per wave");

// One token whose rows reduce in row order (a device route at S = 1: its selections are
// distinct experts, one row each, in route order): every read is independent of the group
// record (live flags and weights come from the row descriptors), so the take is one memory round
// trip: one wave per 64 columns (so the reads spread over many CUs); lane j loads row j's weight
// and live flag while every lane loads its column of all of a slot's y rows (a slot has at most
// kRows = 64), then the FMAs run in row order with each row's weight read from its lane.  The
// arithmetic is the general path's: fmaf over the live rows in order, slots in order.
__global__ __launch_bounds__(kWave) void k_take_in_order(TakeArgs a) {
  const int lane = threadIdx.x;
  const int i = blockIdx.x * kWave + lane;
  const int ic = min(i, a.D - 1);  // every lane stays for the broadcasts; lanes past D store nothing
  float *rp = a.resid + ic;
  const float r_in = *rp;  // in flight with the rows' loads
  float total = 0.f;
  for (int s = 0; s < a.nslots; ++s) {
    const CGroupBuf G = (CGroupBuf)a.groups[s];
    const float *__restrict__ y = a.y[s];
    const int rows = min(a.rows[s], kRows);
    const int rl = min(lane, max(rows - 1, 0));
    const float wl = G->rows[rl].weight;
    const int livel = lane < rows ? G->rows[rl].t[0].live : 0;
    float v[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) v[j] = j < rows ? y[(size_t)j * a.y_ld + ic] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int live = __builtin_amdgcn_readlane(livel, j);
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
      if (live) acc = fmaf(w, v[j], acc);
    }
    total = (s == 0) ? acc : total + acc;
  }
  if (i < a.D) *rp = r_in + total;
}

__global__ __launch_bounds__(kBlock) void k_take(TakeArgs a) {
  __shared__ int s_rr[kSlots][kRows];    // reduce order of each slot (group rows, token-major)
  __shared__ float s_rw[kSlots][kRows];  // route weight of each group row
  __shared__ int s_r0[kSlots], s_cnt[kSlots];
  const int t = blockIdx.y;
  // Each slot's records for token t, staged once per workgroup: all reads of a slot are
  // independent (whole arrays, not chased through the row indices), so they are in flight
  // together.
  for (int q = threadIdx.x; q < a.nslots * kRows; q += kBlock) {
    // kRows == kWave: the slot is uniform across a wave, so its record pointer is a scalar load
    const int s = __builtin_amdgcn_readfirstlane(q / kRows), k = q - s * kRows;
    const GroupDev &g = a.groups[s]->g;
    const int rr = g.red_rows[k];
    const float rw = g.row_weight[k];
    // clamped into the record's arrays: every index below stays inside them whatever the
    // record holds
    const int r0 = min(max(g.tok_row0[t], 0), kRows), r1 = min(max(g.tok_row0[t + 1], r0), kRows);
    s_rr[s][k] = min(max(rr, 0), kRows - 1);
    s_rw[s][k] = rw;
    s_r0[s] = r0;  // every lane stores the same value
    s_cnt[s] = r1 - r0;
  }
  __syncthreads();
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= a.D) return;
  float total = 0.f;
  for (int s = 0; s < a.nslots; ++s) {
    const float *__restrict__ y = a.y[s];
    const int cnt = s_cnt[s];
    float acc = 0.f;
    // eight rows' loads in flight at a time (clamped row index, unconditional loads), then the
    // FMAs in route order
    for (int k0 = 0; k0 < cnt; k0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = y[(size_t)s_rr[s][s_r0[s] + min(k0 + j, cnt - 1)] * a.y_ld + i];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < cnt) acc = fmaf(s_rw[s][s_rr[s][s_r0[s] + k0 + j]], v[j], acc);
    }
    total = (s == 0) ? acc : total + acc;
  }
  float *rp = a.resid + (size_t)t * a.D + i;
  *rp = *rp + total;
}

// Store an explicit (host-built) group record and fill its row descriptors from the layer's
// expert table; the record travels as a kernel argument, so the store is ordered on the
// stream like every other step.
__global__ void k_group_store(GroupDev g, const ExpertRec *table, GroupBuf *dst) {
  const int32_t *src = reinterpret_cast<const int32_t *>(&g);
  int32_t *d = reinterpret_cast<int32_t *>(&dst->g);
  for (int w = threadIdx.x; w < I4MOE_GROUP_WORDS; w += blockDim.x) d[w] = src[w];
  for (int r = threadIdx.x; r < kRows; r += blockDim.x) {
    RowDesc &rd = dst->rows[r];
    if (r < g.n_rows) {
      const int e = g.row_expert[r];
      int j = 0;  // the row's entry (entries list their rows consecutively, in row order)
      while (j + 1 < g.n_entries && g.entry_row0[j + 1] <= r) ++j;
      rd.t[0] = table[e].t[0];
      rd.t[1] = table[e].t[1];
      rd.t[2] = table[e].t[2];
      rd.t[0].live = 1;
      rd.t[1].live = r - g.entry_row0[j];                    // rank in the entry
      rd.t[2].live = g.entry_row0[j + 1] - g.entry_row0[j];  // the entry's rows
      rd.token = g.row_token[r];
      rd.weight = g.row_weight[r];
    } else {
      rd.t[0].live = 0;
    }
  }
}

}  // namespace

hipError_t launch_take(const TakeArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (a.in_order) {
    const dim3 grid((a.D + kWave - 1) / kWave);
    if (t0 || t1)
      hipExtLaunchKernelGGL(k_take_in_order, grid, dim3(kWave), 0, st, t0, t1, 0, a);
    else
      hipLaunchKernelGGL(k_take_in_order, grid, dim3(kWave), 0, st, a);
    return hipGetLastError();
  }
  dim3 grid((a.D + kBlock - 1) / kBlock, a.S);
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_take, grid, dim3(kBlock), 0, st, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_take, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_group_store(const GroupDev &g, const ExpertRec *table, GroupBuf *dst, hipStream_t st) {
  hipLaunchKernelGGL(k_group_store, dim3(1), dim3(kBlock), 0, st, g, table, dst);
  return hipGetLastError();
}

}  // namespace i4moe
