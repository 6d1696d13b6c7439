// The steps around the routed experts of an MoE block (gfx950): rmsnorm of the residual rows
// into the experts' input.  The shared expert reuses the grouped projections (proj.hip) and the
// residual add is the take (take.hip).
//
// Source: the "GPU resident pipeline" commit of "Commit history of c/backend_cuda.cu" lists
// rmsnorm over strided rows among the device primitives of the layer's data plane, checked
// against the engine's CPU math.  For row t (stride ld_x) of D float32 values and gamma:
//
//   out[t][i] = round( x[t][i] / sqrt(sum_i x[t][i]^2 / D + eps) * gamma[i] )
//
// in f64 (every square of a float32 is exact in f64; the sum runs in a fixed order; the division
// is a multiplication by the row's reciprocal, within an f64 ulp or two of it), rounded once,
// directly from the f64 value, to the output dtype: float32, or bfloat16 through
// round-to-odd float32 (which, with 16 spare bits, makes the final round-to-nearest-even to
// bf16 the same as rounding the f64 value directly).
#include <hip/hip_ext.h>

#include "norm.h"

namespace i4moe {
namespace {

constexpr int kNormBlock = kNormWaves * kWave;  // 1024 threads per row

// One workgroup per row: the row's reciprocal root (rms_rinv: the sum of squares in its fixed
// order), then each value times it and gamma in f64, rounded once.
__global__ __launch_bounds__(kNormBlock) void k_rmsnorm(NormArgs a) {
  __shared__ double s_norm[kNormWaves];
  const int t = blockIdx.x;
  const float *x = a.x + (size_t)t * a.ld_x;
  const double rinv = rms_rinv(x, a.D, a.eps, s_norm);
  for (int i = threadIdx.x; i < a.D; i += kNormBlock)
    norm_store(a.out, (size_t)t * a.ld_out + i, x[i], rinv, a.gamma[i], a.out_bf16 != 0);
}

}  // namespace

hipError_t launch_rmsnorm(const NormArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (a.S < 1 || a.D < 1) return hipErrorInvalidValue;
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_rmsnorm, dim3(a.S), dim3(kNormBlock), 0, st, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_rmsnorm, dim3(a.S), dim3(kNormBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace i4moe
