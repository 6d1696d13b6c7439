// The f64 wave sum shared by the router GEMV (router.hip) and the rmsnorm (block.hip), and the
// rmsnorm's sum of squares and rounding.  Source: the rmsnorm over strided rows of the "GPU
// resident pipeline" commit of "Commit history of c/backend_cuda.cu"; the formula and rounding are
// described in block.hip.
#pragma once

#include "common.h"

namespace i4moe {

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

// The normalisation's sum of squares is laid out over 16 waves of 64 lanes (1024 threads): lane
// l of wave w sums the columns w * 64 + l + k * 1024 in column order (fma: the square is exact,
// one rounding per add), each wave's lanes are summed with wave_sum_f64, and the 16 wave sums are
// added in wave order.  A workgroup of fewer waves would run the 16 waves' sums in turn (its
// wave v takes waves v, v + nw, ...), giving the same total.
constexpr int kNormWaves = 16;

// The row's 1 / sqrt(sum / D + eps) (all threads of the workgroup; holds two barriers; s_norm is
// workgroup scratch of kNormWaves doubles).
__device__ __forceinline__ double rms_rinv(const float *x, int D, float eps, double *s_norm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int vw = wv; vw < kNormWaves; vw += nw) {
    double ss = 0.0;
    for (int i = vw * kWave + lane; i < D; i += kNormWaves * kWave) {
      const double v = (double)x[i];
      ss = fma(v, v, ss);
    }
    const double w = wave_sum_f64(ss);
    if (lane == 0) s_norm[vw] = w;
  }
  __syncthreads();
  double total = s_norm[0];
#pragma unroll
  for (int k = 1; k < kNormWaves; ++k) total += s_norm[k];
  __syncthreads();  // s_norm may be reused once every thread has its total
  return 1.0 / sqrt(total / (double)D + (double)eps);
}

// One normalised value x * rinv * gamma in f64, rounded once to the output dtype (bfloat16 through
// round-to-odd float32, which with 16 spare bits rounds as the f64 value would).
__device__ __forceinline__ void norm_store(void *out, size_t i, float x, double rinv, float gamma, bool bf16) {
  const double v = (double)x * rinv * (double)gamma;
  if (bf16)
    static_cast<uint16_t *>(out)[i] = bf16_rne_bits(f32_round_odd_bits(v));
  else
    static_cast<float *>(out)[i] = (float)v;
}

}  // namespace i4moe
