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

#include "common.h"

namespace i4moe {
namespace {

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

// v rounded to float32 with round-to-odd: the nearest float32 toward zero, with its last bit set
// when v was not exact.
__device__ __forceinline__ uint32_t f32_round_odd_bits(double v) {
  const float f = (float)v;  // round to nearest even
  uint32_t b = __float_as_uint(f);
  const double back = (double)f;
  if (back != v) {
    if (fabs(back) > fabs(v)) b -= 1u;  // the neighbour toward zero (same sign, one ulp less)
    b |= 1u;
  }
  return b;
}

// Round-to-nearest-even of a float32 bit pattern to bfloat16 (finite inputs; infinity stays).
__device__ __forceinline__ uint16_t bf16_rne_bits(uint32_t b) {
  return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}

constexpr int kNormBlock = 1024;  // threads per row: a decode row of a few thousand values is a few per thread

// One workgroup per row.  The sum of squares: each thread's columns in column order (fma: the
// square is exact, one rounding per add), a fixed-pattern wave sum, then the waves' sums in wave
// order.  Each value is then multiplied by the row's 1 / sqrt(mean + eps) and by gamma in f64 and
// rounded once.
__global__ __launch_bounds__(kNormBlock) void k_rmsnorm(NormArgs a) {
  __shared__ double s_part[kNormBlock / kWave];
  const int t = blockIdx.x;
  const float *x = a.x + (size_t)t * a.ld_x;
  double ss = 0.0;
  for (int i = threadIdx.x; i < a.D; i += kNormBlock) {
    const double v = (double)x[i];
    ss = fma(v, v, ss);
  }
  const double w = wave_sum_f64(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = w;
  __syncthreads();
  double total = s_part[0];
#pragma unroll
  for (int k = 1; k < kNormBlock / kWave; ++k) total += s_part[k];
  const double rinv = 1.0 / sqrt(total / (double)a.D + (double)a.eps);
  for (int i = threadIdx.x; i < a.D; i += kNormBlock) {
    const double v = (double)x[i] * rinv * (double)a.gamma[i];
    if (a.out_bf16)
      static_cast<uint16_t *>(a.out)[(size_t)t * a.ld_out + i] = bf16_rne_bits(f32_round_odd_bits(v));
    else
      static_cast<float *>(a.out)[(size_t)t * a.ld_out + i] = (float)v;
  }
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
