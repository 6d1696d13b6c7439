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
#include "common.h"

namespace i4moe {
namespace {

__global__ __launch_bounds__(kBlock) void k_take(TakeArgs a) {
  __shared__ int s_rows[kSlots][kRows];
  __shared__ float s_w[kSlots][kRows];
  __shared__ int s_cnt[kSlots];
  const int t = blockIdx.y;
  // This token's rows of every slot, in reduce order, staged once per workgroup.
  for (int q = threadIdx.x; q < a.nslots * kRows; q += kBlock) {
    const int s = q / kRows, k = q - s * kRows;
    const GroupDev &g = a.groups[s]->g;
    const int r0 = g.tok_row0[t], r1 = g.tok_row0[t + 1];
    if (k == 0) s_cnt[s] = r1 - r0;
    if (k < r1 - r0) {
      const int row = g.red_rows[r0 + k];
      s_rows[s][k] = row;
      s_w[s][k] = g.row_weight[row];
    }
  }
  __syncthreads();
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= a.D) return;
  float total = 0.f;
  for (int s = 0; s < a.nslots; ++s) {
    const float *__restrict__ y = a.y[s];
    float acc = 0.f;
    for (int k = 0; k < s_cnt[s]; ++k) acc = fmaf(s_w[s][k], y[(size_t)s_rows[s][k] * a.y_ld + i], acc);
    total = (s == 0) ? acc : total + acc;
  }
  float *rp = a.resid + (size_t)t * a.D + i;
  *rp = *rp + total;
}

// Store an explicit (host-built) group record and fill its row descriptors from the layer's
// expert table; the record travels as a kernel argument, so the store is ordered on the
// stream like every other step.
__global__ void k_group_store(GroupDev g, const TensorDesc *table, GroupBuf *dst) {
  const int32_t *src = reinterpret_cast<const int32_t *>(&g);
  int32_t *d = reinterpret_cast<int32_t *>(&dst->g);
  for (int w = threadIdx.x; w < I4MOE_GROUP_WORDS; w += blockDim.x) d[w] = src[w];
  for (int r = threadIdx.x; r < g.n_rows && r < kRows; r += blockDim.x) {
    const int e = g.row_expert[r];
    RowDesc &rd = dst->rows[r];
    rd.t[0] = table[e];
    rd.t[1] = table[kMaxE + e];
    rd.t[2] = table[2 * kMaxE + e];
    rd.token = g.row_token[r];
    rd.weight = g.row_weight[r];
  }
}

}  // namespace

hipError_t launch_take(const TakeArgs &a, hipStream_t st) {
  dim3 grid((a.D + kBlock - 1) / kBlock, a.S);
  hipLaunchKernelGGL(k_take, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_group_store(const GroupDev &g, const TensorDesc *table, GroupBuf *dst, hipStream_t st) {
  hipLaunchKernelGGL(k_group_store, dim3(1), dim3(kBlock), 0, st, g, table, dst);
  return hipGetLastError();
}

}  // namespace i4moe
