// Device-side records shared by the i4moe kernels and the host library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/i4moe.h"

namespace i4moe {

constexpr int kRows = I4MOE_MAX_ROWS;      // expert-token rows per issue
constexpr int kTokens = I4MOE_MAX_TOKENS;
constexpr int kMaxK = I4MOE_MAX_K;
constexpr int kMaxE = I4MOE_MAX_E;
constexpr int kMaxCols = I4MOE_MAX_COLS;
constexpr int kSlots = I4MOE_MAX_SLOTS;
constexpr int kWave = 64;
constexpr int kBlock = 256;                // 4 waves per workgroup

// One uploaded int4 tensor as the kernels see it.  Rows are `row_bytes` apart (C/2 rounded
// up to 16 B, pad bytes 0x88 i.e. weight 0); nibbles stay offset-binary (q encodes q - 8).
struct TensorDesc {
  const uint8_t *q;
  const float *s;      // [O][ng] scales
  int32_t O, C;
  int32_t row_bytes;
  int32_t gs;          // group size; 0 when ng == 1
  int32_t ng;          // scales per row (1 = per-row)
  int32_t pad;
};

// Group record (layout documented with I4MOE_GROUP_WORDS).
struct GroupDev {
  int32_t n_entries, n_rows, S, reserved;
  int32_t entry_expert[kRows];
  int32_t entry_row0[kRows + 1];
  int32_t row_token[kRows];
  int32_t row_expert[kRows];
  float row_weight[kRows];
  int32_t tok_row0[kTokens + 1];
  int32_t red_rows[kRows];
};
static_assert(sizeof(GroupDev) == I4MOE_GROUP_WORDS * 4, "group record layout");

// Packed per-token route record: same layout as i4moe_route_host.
struct RouteTok {
  int32_t n;
  int32_t idx[kMaxK];
  float w[kMaxK];
};
static_assert(sizeof(RouteTok) == sizeof(i4moe_route_host), "route record layout");

struct RouteArgs {
  const float *W;        // [E][D]
  const float *bias;     // [E]
  const void *x;         // [S][D] f32 or bf16
  double *partial;       // [S][E][splits]
  double *logits;        // [S][E]
  unsigned *counter;     // finished-workgroup counter, left at 0 by the last workgroup
  RouteTok *route;       // [S]
  GroupDev *group;
  int E, D, S, K;
  int x_bf16;
  int splits, cols_per_split;
  int norm_topk;
  float topp, routed_scale;
};

struct ProjArgs {
  const GroupDev *group;     // rows to run
  GroupDev *group_copy;      // when non-null, workgroup 0 copies *group here
  const TensorDesc *tA;      // per expert: gate (dual) or down
  const TensorDesc *tB;      // per expert: up (dual only)
  const void *act;           // dual: x [S][act_ld]; down: h [rows][act_ld] f32
  float *out;                // dual: h [rows][out_ld]; down: y [rows][out_ld]
  int act_ld, out_ld;
  int act_bf16;
  int O, C;                  // rows and columns of every tensor in the launch
  int tiles, tile_rows;      // tiles per group row, rows per tile
};

struct TakeArgs {
  const GroupDev *groups[kSlots];
  const float *y[kSlots];
  float *resid;              // [S][D]
  int nslots, y_ld, S, D;
};

// Launchers (defined in the kernel translation units).  They return hipGetLastError().
hipError_t launch_route(const RouteArgs &a, hipStream_t st);
hipError_t launch_dual(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st);
hipError_t launch_down(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st);
hipError_t launch_take(const TakeArgs &a, hipStream_t st);
hipError_t launch_group_store(const GroupDev &g, GroupDev *dst, hipStream_t st);

// Rows per inner step for a launch shape: ~32 weight dwords in flight per lane.
constexpr int rows_per_step(int V, int P, int tensors) {
  return (32 / (tensors * V * P)) < 1 ? 1 : ((32 / (tensors * V * P)) > 8 ? 8 : 32 / (tensors * V * P));
}

}  // namespace i4moe
