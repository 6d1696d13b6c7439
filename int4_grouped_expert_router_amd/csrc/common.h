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
constexpr int kSharedRec = kMaxE;  // the layer's shared expert: the table record after the routed experts' cap
constexpr int kMaxCols = I4MOE_MAX_COLS;
constexpr int kSlots = I4MOE_MAX_SLOTS;
constexpr int kWave = 64;
constexpr int kBlock = 256;                // 4 waves per workgroup

// One uploaded int4 tensor as the kernels see it.  Rows are `row_bytes` apart (C/2 rounded
// up to 16 B, pad bytes 0, i.e. weight 0); every nibble holds q - 8 in 4-bit two's complement
// (the host's offset-binary q converted at upload).
struct TensorDesc {
  const uint8_t *q;
  const float *s;      // [O][ng] scales
  int32_t O, C;
  int32_t row_bytes;
  int32_t gs;          // group size; 0 when ng == 1
  int32_t ng;          // scales per row (1 = per-row)
  int32_t live;        // in a row descriptor's first record: 1 = the row is part of the group
};
static_assert(sizeof(TensorDesc) == 40, "tensor descriptor layout");

// One expert of a layer's table: gate, up and down tensors in a 128-byte record, so a row
// descriptor starts with a straight copy of it.
struct ExpertRec {
  TensorDesc t[3];
  int32_t pad[2];
};
static_assert(sizeof(ExpertRec) == 128, "expert record layout");

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

// Everything a projection wave needs about its group row, in one 128-byte record (t[0].live
// marks the rows of the current group; every row of the buffer is rewritten per group): the
// expert's gate / up / down tensors, the token row of x and the route weight.  In a live row,
// t[1].live is the row's rank among its entry's rows and t[2].live the entry's row count.
struct RowDesc {
  TensorDesc t[3];
  int32_t token;
  float weight;
};
static_assert(sizeof(RowDesc) == 128, "row descriptor layout");

// Packed per-token route record: same layout as i4moe_route_host.
struct RouteTok {
  int32_t n;
  int32_t idx[kMaxK];
  float w[kMaxK];
};
static_assert(sizeof(RouteTok) == sizeof(i4moe_route_host), "route record layout");

// What one route (or one explicit group) hands to issue and take.
struct GroupBuf {
  RowDesc rows[kRows];
  GroupDev g;
  RouteTok route[kTokens];
};

struct RouteArgs {
  const float *W;            // [E][D]
  const float *bias;         // [E]
  const void *x;             // [S][D] f32 or bf16
  double2 *score;            // [S][E]: choice score c = sigma + bias (NaN as -inf), sigma
  double *logits;            // [S][E]
  GroupBuf *out;
  const ExpertRec *table;    // layer expert table [kMaxE], or null (route only)
  int E, D, S, K;
  int x_bf16;
  int splits, cols_per_split;  // GEMV: column splits of an expert row, one wave each
  int epb;                   // GEMV: experts per workgroup (splits * epb <= 16 waves)
  int vec;                   // four-column loads in the GEMV
  int norm_topk;
  float topp, routed_scale;
  // 1: the group gets one more row per token after the routed rows: the layer's shared expert
  // (table record kSharedRec) with weight 1, as one more entry (the route records list only the
  // routed experts)
  int shared_rows;
};

struct ProjArgs {
  const GroupBuf *grp;       // rows to run
  const void *act;           // dual: x [S][act_ld]; down: h [rows][act_ld] f32
  float *out;                // dual: h [rows][out_ld]; down: y [rows][out_ld]
  int act_ld, out_ld;
  int act_bf16;
  int O, C;                  // rows and columns of every tensor in the launch
  int tile_groups, tile_rows;  // workgroups per group row (4 tiles each), rows per tile
  int grid_rows;             // group rows the grid covers (grid = grid_rows * tile_groups)
  // entry_rows > 0 (several tokens): the rows of one expert share each weight pass, at most
  // entry_rows (<= kEntryRows) at a time, and the dynamic LDS holds that many staged rows.
  int entry_rows;
  // mfma_min > 0: entries of at least this many rows belong to the matrix-core kernels and the
  // vector kernels skip them
  int mfma_min;
  RouteArgs ra;              // dual with the fused selection: the route whose scores it ranks
};

constexpr int kEntryRows = 4;  // rows of one expert per weight pass in the vector kernels

// Digit rows for the matrix-core dual projection: rows of f32 or bf16 activations (row stride
// act_ld) as three int8 planes of C64 bytes each (row r at dig + 3 r C64), and each row's E.
struct DigitArgs {
  const void *act;
  int8_t *dig;
  int *E;
  int act_ld, bf16, rows, C, C64;
};

// Matrix-core projection of the entries with at least mfma_min rows (slot k: the k-th such
// entry in entry order).  dual: gate/up + SiLU into h rows, digit rows indexed by token, and the
// digit rows of those h rows (dig_out, E_out, indexed by group row) for the down projection;
// else the down projection into y rows, digit rows indexed by group row.  The columns are split
// into ksplit slices whose partial sums go to part ([ksplit][NT][slots][64][O] floats) and are
// added in slice order by the reduction launch.
struct MfmaArgs {
  const GroupBuf *grp;
  const int8_t *dig;
  const int *E;
  float *out;
  float *part;
  int8_t *dig_out;  // dual: digit rows of h
  int *E_out;       // dual: their exponents
  int out_ld, dig_rows, dual;
  int O, C64;
  int mfma_min, slots, ksplit;
  int row_acc;              // every tensor of the launch is per-row: int32 digit sums over a slice
  int weight_tiles, tiles;  // set by the launcher
};

struct TakeArgs {
  const GroupBuf *groups[kSlots];
  const float *y[kSlots];
  float *resid;              // [S][D]
  int nslots, y_ld, S, D;
  int rows[kSlots];          // row capacity of each slot's group (its live rows are a prefix)
  int in_order;              // 1: one token, and every slot reduces its live rows in row order
};

// rmsnorm of S rows of D float32 values (row stride ld_x) times gamma, into S rows of the
// experts' input dtype (row stride ld_out).
struct NormArgs {
  const float *x;
  const float *gamma;        // [D]
  void *out;                 // float32 or bf16 [S][ld_out]
  int ld_x, ld_out, S, D;
  int out_bf16;
  float eps;
};

// Launchers (defined in the kernel translation units).  They return hipGetLastError().  With
// t0/t1 non-null the launch records the kernel's own start and end into them
// (hipExtLaunchKernel), so an event pair spans the kernel alone.
// parts: kRouteGemv, kRouteSelect or both.  The selection reads the GEMV's scores.
constexpr int kRouteGemv = 1, kRouteSelect = 2;
hipError_t launch_route(const RouteArgs &a, int parts, hipStream_t st, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);
// sel: the dual projection first runs the selection of a.ra itself (one token, E <= 64,
// non-generic spans) and publishes its route, group and row descriptors.
bool dual_sel_ok(const RouteArgs &ra, bool gen);
hipError_t launch_dual(int V, int P, bool gen, bool sel, const ProjArgs &a, int blocks, hipStream_t st,
                       hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_down(int V, int P, bool gen, const ProjArgs &a, int blocks, hipStream_t st, hipEvent_t t0 = nullptr,
                       hipEvent_t t1 = nullptr);
hipError_t launch_take(const TakeArgs &a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Down projection and take in one launch, for one token and one issue of at most kDTRows
// rows whose down rows fit k_rows16 (P passes), kDTTile outputs per workgroup: a.act = h,
// a.grp = the group, a.grid_rows = its rows, a.O = D, a.C = I, a.out = the residual row,
// updated in place.
constexpr int kDTRows = 16, kDTTile = 16;
hipError_t launch_down_take(int P, const ProjArgs &a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Down projection over rows of at most 256 weight dwords (C <= 2048): 16 lanes per row, P
// passes of 4 dwords per lane; f32 activations, per-row or 32-column-aligned group scales.
hipError_t launch_down16(int P, const ProjArgs &a, int blocks, hipStream_t st, hipEvent_t t0 = nullptr,
                         hipEvent_t t1 = nullptr);
int rows16_blocks_per_cu(int P);
// Rows of one expert a launch shape stages per workgroup: at most `want` and kEntryRows, and few
// enough that three workgroups' staged rows fit a CU's LDS.
int entry_rows_fit(int V, int P, bool rows16, int want);
int proj_blocks_per_cu(int V, int P, int NT, bool gen);  // resident 256-thread workgroups per CU
hipError_t launch_group_store(const GroupDev &g, const ExpertRec *table, GroupBuf *dst, hipStream_t st);
hipError_t launch_rmsnorm(const NormArgs &a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_digits8(const DigitArgs &a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_mfma(int NT, MfmaArgs a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// The read probe (a measuring aid): every nibble and scale byte of the listed experts' tensors,
// read with the projections' access shape and no arithmetic.
struct ProbeArgs {
  const ExpertRec *tab;
  uint32_t *sink;            // 64 dwords, written only when the folded loads equal a constant
  int16_t experts[kRows];    // expert indices into tab
  int n_experts;
  int tensors[3], tiles[3], tile_rows[3];  // tensor indices (0 gate, 1 up, 2 down), their tiles, rows per tile
  int n_tensors, waves;
};
hipError_t launch_read_probe(const ProbeArgs &a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Column slices of a matrix-core launch (about two workgroups per CU) and its partial-sum floats.
int mfma_ksplit(int O, int C64, int slots, int n_cu, int rows);
size_t mfma_part_floats(int NT, int O, int slots, int ksplit);

// Rows per pipeline step for a launch shape: about `budget` weight dwords per lane per step.
constexpr int rows_per_step(int V, int P, int tensors, int budget) {
  return (budget / (tensors * V * P)) < 1 ? 1 : ((budget / (tensors * V * P)) > 8 ? 8 : budget / (tensors * V * P));
}

// Raise a kernel's dynamic LDS limit once per device (the attribute belongs to the kernel as
// loaded on the current device); devices past the table raise it on every call.
constexpr int kMaxDevices = 64;
inline hipError_t raise_lds_once(const void *kernel, int bytes, bool (&done)[kMaxDevices]) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked && done[dev]) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && tracked) done[dev] = true;
  return e;
}

// Constant-address-space views: uniform records read with scalar loads.
#define I4MOE_AS4 __attribute__((address_space(4)))
typedef const GroupBuf I4MOE_AS4 *CGroupBuf;
typedef const TensorDesc I4MOE_AS4 *CTensorDesc;

}  // namespace i4moe
