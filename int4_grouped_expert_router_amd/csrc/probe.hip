// A measuring aid: the plain-read rate of the expert weights (gfx950).
//
// The bandwidth a projection reaches is reported against HBM peak and against a plain read of
// the same bytes on the same GPU (the figure the pages' grouped kernels are measured by is
// expert-weight bytes per second).  k_read_probe reads every nibble and scale byte of the listed
// experts' tensors and computes nothing: one wave per tile of rows of one tensor (about 16 KB of
// nibbles: 4 rows of 3.5 KB, 16 of 1 KB), whose rows are one contiguous block of the nibble array
// (and one of the scale array), streamed with sixteen 16-byte loads per lane in flight (16 KB
// per wave pass).  The loaded words are folded into one value that is stored
// only if it equals a constant, so the loads stay live and every store stays in bounds whatever
// the data.
#include <hip/hip_ext.h>

#include "common.h"

namespace i4moe {
namespace {

constexpr int kProbeLoads = 16;              // 16-byte loads per lane in flight
constexpr int kFarOffset = 0x7ffffff0;       // past every buffer range: reads zero, no access

__global__ __launch_bounds__(kBlock) void k_read_probe(ProbeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6));
  if (wv >= a.waves) return;
  // wave -> (expert, tensor, tile), expert-major
  int per_e = 0;
  for (int n = 0; n < a.n_tensors; ++n) per_e += a.tiles[n];
  const int ei = wv / per_e;
  int rem = wv - ei * per_e, ni = 0;
  while (ni + 1 < a.n_tensors && rem >= a.tiles[ni]) rem -= a.tiles[ni++];
  const TensorDesc I4MOE_AS4 &d = ((const ExpertRec I4MOE_AS4 *)a.tab)[a.experts[ei]].t[a.tensors[ni]];
  const uint8_t *q = d.q;
  const float *sc = d.s;
  const int O = d.O, row_bytes = d.row_bytes, ng = d.ng;
  const int tr = a.tile_rows[ni];
  const int r0 = rem * tr, r1 = min(r0 + tr, O);
  // the tile's bytes: nibbles [r0, r1) x row_bytes, then scales [r0, r1) x ng x 4
  const int qb = r0 * row_bytes, qe = r1 * row_bytes;
  const int sb = r0 * ng * 4, se = r1 * ng * 4;
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(q), (short)0, qe,
                                                                      0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(sc), (short)0, se,
                                                                      0x00020000);
  uint32_t acc = 0;
  for (int off = qb; off < qe; off += kProbeLoads * kWave * 16) {
    uint32_t v[kProbeLoads][4];
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) {
      const int at = off + 16 * (j * kWave + lane);
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(qr, at < qe ? at : kFarOffset, 0, 2);
      v[j][0] = u[0];
      v[j][1] = u[1];
      v[j][2] = u[2];
      v[j][3] = u[3];
    }
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  for (int off = sb; off < se; off += kProbeLoads * kWave * 4) {
    uint32_t v[kProbeLoads];
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) {
      const int at = off + 4 * (j * kWave + lane);
      v[j] = __builtin_amdgcn_raw_buffer_load_b32(sr, at < se ? at : kFarOffset, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) acc ^= v[j];
  }
  if (acc == 0x9E3779B9u) a.sink[lane] = acc;
}

}  // namespace

hipError_t launch_read_probe(const ProbeArgs &a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  if (a.n_experts < 1 || a.n_experts > kRows || a.n_tensors < 1 || a.n_tensors > 3 || a.waves < 1 || !a.tab || !a.sink)
    return hipErrorInvalidValue;
  for (int n = 0; n < a.n_tensors; ++n)
    if (a.tile_rows[n] < 1 || a.tiles[n] < 1) return hipErrorInvalidValue;
  const dim3 grid((a.waves + kBlock / kWave - 1) / (kBlock / kWave));
  if (t0 || t1)
    hipExtLaunchKernelGGL(k_read_probe, grid, dim3(kBlock), 0, st, t0, t1, 0, a);
  else
    hipLaunchKernelGGL(k_read_probe, grid, dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace i4moe
