// C ABI of the i4moe library: weight and router memory, route buffers, issue slots, launch
// planning, error conventions and the test hooks.  Declarations and contracts: include/i4moe.h.
//
// Error conventions follow the vendor-neutral-fixes commit ("Commit history of
// c/backend_cuda.cu"): every HIP error is consumed where it is seen so it cannot poison a
// later healthy call, uploaded tensors never look at the caller's host buffers again, and the
// fail-after hook gates compute entry points only.  The take is fatal on failure, as in the
// COLI_CUDA_RESID page: a take that did not run would silently drop routed experts.
#include <sched.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "common.h"
#include "host_tier.h"

using namespace i4moe;

namespace {

struct Tensor {
  uint8_t *q = nullptr;
  float *s = nullptr;
  TensorDesc desc{};
  int fmt = 0;
};

// The layer's shared expert sits in the expert table right after the routed experts' cap.
constexpr int kShared = kSharedRec;

struct Layer {
  int E = 0, D = 0, I = 0;             // router experts; model dim; expert intermediate
  float *W = nullptr, *b = nullptr;    // router
  std::vector<i4moe_tensor> gate, up, down;
  i4moe_tensor shared[3] = {0, 0, 0};  // shared expert: gate, up, down
  bool shared_set = false;
  float *gamma = nullptr;              // rmsnorm weights [D]
  float eps = 0.f;
  ExpertRec *d_tab = nullptr;          // [kMaxE + 1]: gate, up, down descriptors per expert, then the shared one
  std::vector<ExpertRec> h_tab;        // host copy of d_tab
  int route_buf = -1;                  // ring entry holding this layer's latest route
  bool routed = false;
  int route_S = 0, route_K = 0;
  bool route_shared = false;  // the route's group ends with one shared-expert row per token
  std::map<int, std::unique_ptr<HostExpert>> host;  // experts kept on the host (the CPU tier)
  int host_D = 0, host_I = 0;
};

struct SlotInfo {
  int S = 0, D = 0, rows = 0;
  const GroupBuf *grp = nullptr;  // group record + row descriptors this issue ran
  int ring = -1;                  // route ring entry it came from, -1 for an explicit group
  // The down projection of a lone one-token issue waits for the take, which runs it fused
  // with the reduction (k_down_take); anything else that needs y or h first runs it alone.
  bool down_pending = false;
  int down_P = 0, down_blocks = 0;
  ProjArgs down{};
};

constexpr int kRing = 32;  // route buffers: a layer may be re-routed up to 31 times before a take
constexpr int kMfmaMinRows = 8;  // rows of one expert from which the matrix cores pay (measured)

struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};

struct Plan {
  int V = 4, P = 1;
  bool gen = false;
  bool rows16 = false;  // down projection with 16 lanes per row
  int tile_rows = 1, tile_groups = 1, blocks = 1;
};

}  // namespace

struct i4moe_ctx {
  int device = 0;
  hipStream_t stream = nullptr;
  std::string err;
  uint32_t next_handle = 1;
  std::map<uint32_t, Tensor> tensors;
  std::map<int, Layer> layers;

  double2 *d_score = nullptr;  // [kTokens][kMaxE] router scores (choice score, sigma)
  double *d_logits = nullptr;  // [kTokens][kMaxE]

  float *d_xn = nullptr;   // [kTokens][xn_ld] the block's normalised rows (f32 or bf16)
  int xn_ld = 0;
  float *d_h = nullptr;    // [kRows][h_ld]
  int h_ld = 0;
  float *d_y = nullptr;    // [kSlots][kRows][y_ld]
  int y_ld = 0;
  GroupBuf *d_ring = nullptr;       // [kRing] route outputs
  int ring_next = 0;
  GroupBuf *d_slot_bufs = nullptr;  // [kSlots] explicit groups
  SlotInfo slots[kSlots];
  int n_cu = 256;
  double wave_factor = 1.0;
  int entry_mode = 0;      // rows of one expert per weight pass: 0 one, 2..4 up to that many
  int mfma_min = kMfmaMinRows;  // rows from which an entry runs on the matrix cores (0: never)
  int8_t *d_dig = nullptr;      // [kRows][3][kMaxCols] digit rows of the matrix-core projections
  int *d_dig_E = nullptr;       // [kRows] their row exponents
  float *d_part = nullptr;      // partial sums of the matrix-core column slices
  uint32_t *d_sink = nullptr;   // the read probe's 64-dword sink
  size_t part_floats = 0;

  // the CPU tier: worker threads, pinned copies of x and of the host rows' sum, and the events
  // that say when the x copy has landed and when the sum's upload has been read
  int host_threads = 0;
  std::unique_ptr<HostPool> pool;
  std::unique_ptr<HostHelper> helper;  // runs the host rows while the calling thread issues the device group
  void *h_x = nullptr;          // [kTokens][kMaxCols] float32 or bf16, pinned
  float *h_P = nullptr;         // [kTokens][kMaxCols] float32, pinned
  hipEvent_t ev_x = nullptr, ev_p = nullptr;
  bool ev_p_recorded = false;
  int nslots = 0;

  int last_route_S = 0, last_route_E = 0;

  // A one-token device route of which only the GEMV is enqueued.  The next issue of that route
  // runs the selection inside its dual projection (one launch less per layer); anything else
  // that needs the route or the router scratch runs the selection kernel first (flush_sel).
  bool sel_pending = false;
  int sel_layer = -1;
  RouteArgs sel_args{};
  int last_issue_rows = 0, last_issue_I = 0;

  long long fail_after = -1, calls = 0;
  bool poisoned = false;

  void *scratch = nullptr;  // this device's copy of the static route scratch (i4moe_route_noalloc)

  bool profiling = false;
  std::vector<hipEvent_t> ev_pool;
  std::vector<ProfRec> recs;
  double prof_ms[I4MOE_K_COUNT] = {};
  long long prof_n[I4MOE_K_COUNT] = {};
};

namespace {

int fail(i4moe_ctx *c, int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return code;
}

// Consume the pending device error so it cannot leak into the next call.
int hip_fail(i4moe_ctx *c, hipError_t e, const char *what) {
  (void)hipGetLastError();
  return fail(c, e == hipErrorOutOfMemory ? I4MOE_ENOMEM : I4MOE_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool ensure_device(i4moe_ctx *c) {
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess && cur == c->device) return true;
  return hipSetDevice(c->device) == hipSuccess;
}

void dfree(void *p) {
  if (p) (void)hipFree(p);
}

template <class T>
hipError_t dalloc(T **p, size_t bytes) {
  *p = nullptr;
  hipError_t e = hipMalloc(reinterpret_cast<void **>(p), bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
  }
  return e;
}

int gate_compute(i4moe_ctx *c) {
  if (c->poisoned) return fail(c, I4MOE_EPOISONED, "context poisoned by a failed take");
  if (c->fail_after >= 0 && c->calls >= c->fail_after)
    return fail(c, I4MOE_EINJECTED, "injected failure (fail-after %lld)", c->fail_after);
  return I4MOE_OK;
}

hipEvent_t get_event(i4moe_ctx *c) {
  if (!c->ev_pool.empty()) {
    hipEvent_t e = c->ev_pool.back();
    c->ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}

// Launch wrapper: when profiling, hands the launcher an event pair that records the kernel's
// own start and end (the launch itself timestamps them), so host launch gaps are not counted.
template <class F>
hipError_t timed(i4moe_ctx *c, int kernel, F &&f) {
  hipEvent_t a = nullptr, b = nullptr;
  if (c->profiling) {
    a = get_event(c);
    b = get_event(c);
    if (!a || !b) {
      if (a) c->ev_pool.push_back(a);
      if (b) c->ev_pool.push_back(b);
      a = b = nullptr;
    }
  }
  hipError_t e = f(a, b);
  if (a && b) {
    if (e == hipSuccess) {
      c->recs.push_back({kernel, a, b});
    } else {
      c->ev_pool.push_back(a);
      c->ev_pool.push_back(b);
    }
  }
  return e;
}

// Enqueue the selection of the pending route (see i4moe_ctx::sel_pending).
int flush_sel(i4moe_ctx *c) {
  if (!c->sel_pending) return I4MOE_OK;
  hipError_t e = timed(c, I4MOE_K_ROUTE, [&](hipEvent_t t0, hipEvent_t t1) {
    return launch_route(c->sel_args, kRouteSelect, c->stream, t0, t1);
  });
  if (e != hipSuccess) return hip_fail(c, e, "route selection launch");
  c->sel_pending = false;
  return I4MOE_OK;
}

// Enqueue the down projections still waiting for a take (see SlotInfo::down_pending).
int flush_down(i4moe_ctx *c) {
  for (int s = 0; s < c->nslots; ++s) {
    SlotInfo &si = c->slots[s];
    if (!si.down_pending) continue;
    hipError_t e = timed(c, I4MOE_K_DOWN, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_down16(si.down_P, si.down, si.down_blocks, c->stream, t0, t1);
    });
    if (e != hipSuccess) return hip_fail(c, e, "down launch");
    si.down_pending = false;
  }
  return I4MOE_OK;
}

// Everything deferred, before a call that needs the route, h, y or the tensors as they are now.
int flush_all(i4moe_ctx *c) {
  int rc = flush_sel(c);
  return rc ? rc : flush_down(c);
}

void drain_profile(i4moe_ctx *c) {
  for (auto &r : c->recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      c->prof_ms[r.kernel] += ms;
      c->prof_n[r.kernel] += 1;
    } else {
      (void)hipGetLastError();
    }
    c->ev_pool.push_back(r.a);
    c->ev_pool.push_back(r.b);
  }
  c->recs.clear();
}

int round_up(int v, int m) { return (v + m - 1) / m * m; }

// Scratch for S*K <= kRows rows of the largest D and I seen.  Grows only with no issue pending.
int ensure_rows_scratch(i4moe_ctx *c, int D, int I) {
  const int need_h = round_up(I, 64), need_y = round_up(D, 64);
  if (need_h <= c->h_ld && need_y <= c->y_ld) return I4MOE_OK;
  if (c->nslots > 0) return fail(c, I4MOE_EINVAL, "cannot grow issue scratch while %d issue(s) are pending", c->nslots);
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  const int h_ld = need_h > c->h_ld ? need_h : c->h_ld;
  const int y_ld = need_y > c->y_ld ? need_y : c->y_ld;
  float *h = nullptr, *y = nullptr;
  if ((e = dalloc(&h, sizeof(float) * (size_t)kRows * h_ld)) != hipSuccess) return hip_fail(c, e, "hipMalloc(h)");
  if ((e = dalloc(&y, sizeof(float) * (size_t)kSlots * kRows * y_ld)) != hipSuccess) {
    dfree(h);
    return hip_fail(c, e, "hipMalloc(y)");
  }
  dfree(c->d_h);
  dfree(c->d_y);
  c->d_h = h;
  c->d_y = y;
  c->h_ld = h_ld;
  c->y_ld = y_ld;
  return I4MOE_OK;
}

// Digit rows for the matrix-core projections at their cap (1.5 MB), allocated by the first
// issue that uses them.
int ensure_digit_scratch(i4moe_ctx *c) {
  if (c->d_dig) return I4MOE_OK;
  hipError_t e;
  int8_t *d = nullptr;
  int *E = nullptr;
  if ((e = dalloc(&d, (size_t)kRows * 3 * kMaxCols)) != hipSuccess) return hip_fail(c, e, "hipMalloc(digit rows)");
  if ((e = dalloc(&E, sizeof(int) * 2 * kRows)) != hipSuccess) {  // x rows by token, then h rows
    dfree(d);
    return hip_fail(c, e, "hipMalloc(digit exponents)");
  }
  c->d_dig = d;
  c->d_dig_E = E;
  return I4MOE_OK;
}

// Partial sums of the matrix-core column slices; grows (with the stream drained) only.
int ensure_part_scratch(i4moe_ctx *c, size_t floats) {
  if (floats <= c->part_floats) return I4MOE_OK;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  float *p = nullptr;
  if ((e = dalloc(&p, sizeof(float) * floats)) != hipSuccess) return hip_fail(c, e, "hipMalloc(partial sums)");
  dfree(c->d_part);
  c->d_part = p;
  c->part_floats = floats;
  return I4MOE_OK;
}

// Router scratch at its cap (1.5 MB), allocated by the first route.
int ensure_route_scratch(i4moe_ctx *c) {
  if (c->d_score) return I4MOE_OK;
  hipError_t e;
  double2 *p = nullptr;
  double *l = nullptr;
  if ((e = dalloc(&p, sizeof(double2) * kTokens * kMaxE)) != hipSuccess) return hip_fail(c, e, "hipMalloc(scores)");
  if ((e = dalloc(&l, sizeof(double) * kTokens * kMaxE)) != hipSuccess) {
    dfree(p);
    return hip_fail(c, e, "hipMalloc(logits)");
  }
  c->d_score = p;
  c->d_logits = l;
  return I4MOE_OK;
}

int ensure_layer_tables(i4moe_ctx *c, Layer &L) {
  if (L.d_tab) return I4MOE_OK;
  hipError_t e;
  if ((e = dalloc(&L.d_tab, sizeof(ExpertRec) * (kMaxE + 1))) != hipSuccess) return hip_fail(c, e, "hipMalloc(table)");
  L.h_tab.assign(kMaxE + 1, ExpertRec{});
  e = hipMemcpyAsync(L.d_tab, L.h_tab.data(), sizeof(ExpertRec) * (kMaxE + 1), hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "table init");
  return I4MOE_OK;
}

int write_table_entry(i4moe_ctx *c, Layer &L, int expert) {
  hipError_t e =
      hipMemcpyAsync(L.d_tab + expert, &L.h_tab[expert], sizeof(ExpertRec), hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "table update");
  return I4MOE_OK;
}

// Pick the per-lane span V (dwords) and pass count P for rows of C columns, then tile the rows.
//
// Spans of 4 dwords (one aligned 16-byte load per lane) stream best, then 2, then 1; 3-dword
// spans split across 16-byte boundaries and measured slower than any of them, so they are not
// used.  A wider span wins while it wastes at most half of its lanes (lanes past the row load
// nothing).  Tensors whose group size splits a span need the per-byte path, so a span that
// avoids it is preferred.
//
// Tiles: about two workgroups per CU, but never less than kMinWaveBytes of weights per wave
// (short tiles pay the startup latency of a wave for little data).
constexpr int kMinWaveBytes = 12 * 1024;

Plan plan_proj(int C, int O, int max_rows, bool dual, const std::vector<int> &group_sizes, int n_cu,
               double wave_factor) {
  const int RD = (C + 7) / 8;
  Plan best;
  bool have = false;
  for (int pass = 0; pass < 2 && !have; ++pass) {
    for (int V : {4, 2, 1}) {
      const int P = (RD + 64 * V - 1) / (64 * V);
      if (P > 4) continue;
      bool gen = false;
      for (int gs : group_sizes)
        if (gs % (8 * V) != 0) gen = true;
      const double eff = (double)RD / (64.0 * V * P);
      // pass 0: spans that need no per-byte path and use at least half their lanes
      if (pass == 0 && (gen || (eff < 0.5 && V > 1))) continue;
      best.V = V;
      best.P = P;
      best.gen = gen;
      have = true;
      break;
    }
  }
  if (!have) {  // only per-byte spans remain: the narrowest that fits
    best.V = 1;
    best.P = (RD + 63) / 64;
    best.gen = true;
  }
  const int NT = dual ? 2 : 1;
  // Short down rows run 16 lanes per row (four rows per wave instruction): a fully used wave
  // and a 16-lane reduction instead of a 64-lane one.
  if (!dual && RD <= 4 * 64) {
    bool aligned = true;
    for (int gs : group_sizes)
      if (gs % 32 != 0) aligned = false;
    if (aligned) {
      best.rows16 = true;
      best.V = 4;
      best.P = (RD + 63) / 64;
      best.gen = false;
    }
  }
  const int RB = best.rows16 ? 4 : rows_per_step(best.V, best.P, NT, 16);
  const long long units = (long long)max_rows * O;
  // Two workgroups (eight waves) per CU, or fewer if fewer fit: every CU gets the same share
  // and each wave streams several steps, which measured faster than filling every resident
  // slot with shorter tiles.
  const long long resident =
      (long long)(best.rows16 ? rows16_blocks_per_cu(best.P) : proj_blocks_per_cu(best.V, best.P, NT, best.gen)) *
      4 * n_cu;
  const long long per_cu = resident < 8LL * n_cu ? resident : 8LL * n_cu;
  long long target = (long long)(per_cu * wave_factor);
  if (target < 64) target = 64;
  int tr = (int)((units + target - 1) / target);
  const int row_bytes = 4 * RD;
  const int tr_min = (kMinWaveBytes + NT * row_bytes - 1) / (NT * row_bytes);
  if (tr < tr_min) tr = tr_min;
  tr = round_up(tr < RB ? RB : tr, RB);
  if (tr > (kWave / RB) * RB) tr = (kWave / RB) * RB;  // one result per lane of the tile's wave
  best.tile_rows = tr;
  const int tiles = (O + tr - 1) / tr;
  best.tile_groups = (tiles + 3) / 4;
  best.blocks = max_rows * best.tile_groups;
  return best;
}

Layer *find_layer(i4moe_ctx *c, int layer) {
  auto it = c->layers.find(layer);
  return it == c->layers.end() ? nullptr : &it->second;
}

bool all_finite(const float *p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

// ---- Static route scratch for i4moe_route_noalloc: the router's score and logit scratch and the
// group buffer its selection writes, at the route's own limits (I4MOE_MAX_TOKENS tokens of
// I4MOE_MAX_E experts).  Every GPU the library runs on holds one copy until the process ends.
constexpr size_t kScoreBytes = sizeof(double2) * kTokens * kMaxE;       // 1 MiB
constexpr size_t kLogitBytes = sizeof(double) * kTokens * kMaxE;        // 512 KiB
constexpr size_t kGroupBufBytes = (sizeof(GroupBuf) + 255) / 256 * 256;
constexpr size_t kNoAllocScratchBytes = kScoreBytes + kLogitBytes + kGroupBufBytes;
static_assert(kNoAllocScratchBytes == I4MOE_NOALLOC_SCRATCH_BYTES, "documented scratch size");

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

// The device address of `scratch` on each device, looked up once per device with that device
// current (the array's name is only a host-side handle).
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int device, void **out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (device >= 0 && device < kMaxDevices && g_scratch_ptr[device]) {
    *out = g_scratch_ptr[device];
    return hipSuccess;
  }
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
  if (device >= 0 && device < kMaxDevices) g_scratch_ptr[device] = p;
  *out = p;
  return hipSuccess;
}

// Launch geometry of the router GEMV for a layer: at least 256 waves and at most 1024 columns
// per wave (one batch of loads per lane and token group), each split a multiple of 256
// columns; an expert's splits (and up to four experts of one split each) share a workgroup of
// at most 16 waves.
void gemv_geometry(const Layer &L, RouteArgs &a) {
  int splits = (256 + L.E - 1) / L.E;
  if (splits < (L.D + 1023) / 1024) splits = (L.D + 1023) / 1024;
  if (splits > 16) splits = 16;
  const int cps = round_up((L.D + splits - 1) / splits, 256);
  splits = (L.D + cps - 1) / cps;
  a.splits = splits;
  a.cols_per_split = cps;
  a.epb = splits >= 4 ? 1 : 4 / splits;
}

}  // namespace

extern "C" {

int i4moe_ctx_create(int device, i4moe_ctx **out) try {
  if (!out) return I4MOE_EINVAL;
  *out = nullptr;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) {
    (void)hipGetLastError();
    return I4MOE_EDEVICE;
  }
  if (device < 0 || device >= n) return I4MOE_EINVAL;
  if (hipSetDevice(device) != hipSuccess) {
    (void)hipGetLastError();
    return I4MOE_EDEVICE;
  }
  i4moe_ctx *c = new (std::nothrow) i4moe_ctx();
  if (!c) return I4MOE_ENOMEM;
  c->device = device;
  hipError_t e = dalloc(&c->d_ring, sizeof(GroupBuf) * kRing);
  if (e == hipSuccess) e = dalloc(&c->d_slot_bufs, sizeof(GroupBuf) * kSlots);
  if (e == hipSuccess) e = hipMemset(c->d_ring, 0, sizeof(GroupBuf) * kRing);
  if (e == hipSuccess) e = hipMemset(c->d_slot_bufs, 0, sizeof(GroupBuf) * kSlots);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    dfree(c->d_ring);
    dfree(c->d_slot_bufs);
    delete c;
    return e == hipErrorOutOfMemory ? I4MOE_ENOMEM : I4MOE_EDEVICE;
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && ncu > 0)
    c->n_cu = ncu;
  (void)hipGetLastError();
  if (scratch_address(device, &c->scratch) != hipSuccess) {
    (void)hipGetLastError();
    dfree(c->d_ring);
    dfree(c->d_slot_bufs);
    delete c;
    return I4MOE_EDEVICE;
  }
  if (const char *wf = std::getenv("I4MOE_WAVE_FACTOR")) {
    const double v = std::atof(wf);
    if (v >= 0.05 && v <= 64.0) c->wave_factor = v;
  }
  {
    // the cores this process may run on but one (the calling thread issues the device group
    // meanwhile), at most 16
    unsigned hw = std::thread::hardware_concurrency();
    cpu_set_t cs;
    if (sched_getaffinity(0, sizeof cs, &cs) == 0 && CPU_COUNT(&cs) > 0) hw = (unsigned)CPU_COUNT(&cs);
    c->host_threads = hw <= 2 ? 1 : (hw - 1 > 16 ? 16 : (int)hw - 1);
  }
  if (const char *ht = std::getenv("I4MOE_HOST_THREADS")) {
    char *end = nullptr;
    const long v = std::strtol(ht, &end, 10);
    if (end && end != ht && *end == '\0' && v >= 1 && v <= 256) c->host_threads = (int)v;
  }
  if (const char *mm = std::getenv("I4MOE_MFMA_MIN_ROWS")) {
    char *end = nullptr;
    const long v = std::strtol(mm, &end, 10);
    if (end && end != mm && *end == '\0' && (v == 0 || (v >= 2 && v <= kRows))) c->mfma_min = (int)v;
  }
  if (const char *er = std::getenv("I4MOE_ENTRY_ROWS")) {
    char *end = nullptr;
    const long v = std::strtol(er, &end, 10);
    if (end && end != er && *end == '\0' && (v == 0 || (v >= 2 && v <= kEntryRows))) c->entry_mode = (int)v;
  }
  if (const char *fa = std::getenv("I4MOE_FAIL_AFTER")) {
    char *end = nullptr;
    const long long v = std::strtoll(fa, &end, 10);
    if (end && end != fa && *end == '\0' && v >= 0) c->fail_after = v;
  }
  *out = c;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_ctx_destroy(i4moe_ctx *c) try {
  if (!c) return I4MOE_OK;
  ensure_device(c);
  (void)hipStreamSynchronize(c->stream);
  for (auto &kv : c->tensors) {
    dfree(kv.second.q);
    dfree(kv.second.s);
  }
  for (auto &kv : c->layers) {
    Layer &L = kv.second;
    dfree(L.W);
    dfree(L.b);
    dfree(L.gamma);
    dfree(L.d_tab);
  }
  dfree(c->d_xn);
  dfree(c->d_score);
  dfree(c->d_logits);
  dfree(c->d_ring);
  dfree(c->d_slot_bufs);
  dfree(c->d_h);
  dfree(c->d_y);
  dfree(c->d_dig);
  dfree(c->d_dig_E);
  dfree(c->d_part);
  dfree(c->d_sink);
  c->helper.reset();
  c->pool.reset();
  if (c->h_x) (void)hipHostFree(c->h_x);
  if (c->h_P) (void)hipHostFree(c->h_P);
  if (c->ev_x) (void)hipEventDestroy(c->ev_x);
  if (c->ev_p) (void)hipEventDestroy(c->ev_p);
  for (auto &r : c->recs) {
    c->ev_pool.push_back(r.a);
    c->ev_pool.push_back(r.b);
  }
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  (void)hipGetLastError();
  delete c;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_set_stream(i4moe_ctx *c, void *stream) try {
  if (!c) return I4MOE_EINVAL;
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  c->stream = reinterpret_cast<hipStream_t>(stream);
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

const char *i4moe_last_error(const i4moe_ctx *c) try {
  if (!c) return "no context";
  return c->err.c_str();
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return "host memory exhausted";
}

i4moe_tensor i4moe_upload_expert_tensor(i4moe_ctx *c, int fmt, int gs, int O, int C, const uint8_t *packed,
                                        const float *scales) try {
  if (!c) return 0;
  if (fmt != I4MOE_FMT_ROW && fmt != I4MOE_FMT_GROUP) {
    fail(c, I4MOE_EUNSUPPORTED, "unsupported weight format %d (only 2 = per-row and 4 = group-wise int4)", fmt);
    return 0;
  }
  if (fmt == I4MOE_FMT_ROW && gs != 0) {
    fail(c, I4MOE_EINVAL, "per-row tensors take gs = 0 (got %d)", gs);
    return 0;
  }
  if (fmt == I4MOE_FMT_GROUP && (gs < 0 || gs % 2 != 0)) {
    fail(c, I4MOE_EINVAL, "group size must be even and >= 0 (got %d)", gs);
    return 0;
  }
  if (O < 1 || C < 2 || C % 2 != 0) {
    fail(c, I4MOE_EINVAL, "bad tensor shape %d x %d (C must be even)", O, C);
    return 0;
  }
  if (C > kMaxCols) {
    fail(c, I4MOE_EUNSUPPORTED, "C = %d exceeds %d columns", C, kMaxCols);
    return 0;
  }
  if (!packed || !scales) {
    fail(c, I4MOE_EINVAL, "packed and scales must be non-NULL");
    return 0;
  }
  const int row_bytes = round_up(C / 2, 16);
  const size_t qbytes = (size_t)O * row_bytes + 64;
  if (qbytes > (size_t)0x7fff0000) {  // buffer offsets (row * row_bytes, a few rows past the end) stay in int32
    fail(c, I4MOE_EUNSUPPORTED, "tensor too large (%zu bytes)", qbytes);
    return 0;
  }
  const int ng = (fmt == I4MOE_FMT_GROUP && gs > 0) ? (C + gs - 1) / gs : 1;
  if (!ensure_device(c)) {
    hip_fail(c, hipErrorInvalidDevice, "hipSetDevice");
    return 0;
  }
  Tensor t;
  hipError_t e = dalloc(&t.q, qbytes);
  if (e != hipSuccess) {
    hip_fail(c, e, "hipMalloc(weights)");
    return 0;
  }
  if ((e = dalloc(&t.s, sizeof(float) * (size_t)O * ng)) != hipSuccess) {
    dfree(t.q);
    hip_fail(c, e, "hipMalloc(scales)");
    return 0;
  }
  // Nibbles are converted offset->signed here, as the g4 commit's upload does: xor 0x88 turns
  // each nibble q into the 4-bit two's complement of q - 8, which the kernels' integer dot
  // products take as it is.  Rows are padded to 16 bytes (and the tail slack filled) with
  // zeros, i.e. weight 0.
  std::unique_ptr<uint8_t[]> dev(new (std::nothrow) uint8_t[qbytes]);
  if (!dev) {
    dfree(t.q);
    dfree(t.s);
    fail(c, I4MOE_ENOMEM, "host staging for a %zu-byte tensor", qbytes);
    return 0;
  }
  std::memset(dev.get(), 0, qbytes);
  for (int o = 0; o < O; ++o) {
    const uint8_t *src = packed + (size_t)o * (C / 2);
    uint8_t *dst = dev.get() + (size_t)o * row_bytes;
    for (int b = 0; b < C / 2; ++b) dst[b] = src[b] ^ 0x88u;
  }
  e = hipMemcpyAsync(t.q, dev.get(), qbytes, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(t.s, scales, sizeof(float) * (size_t)O * ng, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    dfree(t.q);
    dfree(t.s);
    hip_fail(c, e, "upload copy");
    return 0;
  }
  t.fmt = fmt;
  t.desc.q = t.q;
  t.desc.s = t.s;
  t.desc.O = O;
  t.desc.C = C;
  t.desc.row_bytes = row_bytes;
  t.desc.gs = ng > 1 ? gs : 0;
  t.desc.ng = ng;
  t.desc.live = 0;
  const uint32_t h = c->next_handle++;
  c->tensors[h] = t;
  return h;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return 0;
}

int i4moe_tensor_free(i4moe_ctx *c, i4moe_tensor h) try {
  if (!c) return I4MOE_EINVAL;
  auto it = c->tensors.find(h);
  if (it == c->tensors.end()) return fail(c, I4MOE_EINVAL, "unknown tensor handle %u", h);
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  for (auto &kv : c->layers) {
    Layer &L = kv.second;
    std::vector<i4moe_tensor> *v[3] = {&L.gate, &L.up, &L.down};
    for (size_t x = 0; x < L.gate.size(); ++x) {
      bool hit = false;
      for (int w = 0; w < 3; ++w) hit = hit || (*v[w])[x] == h;
      if (!hit) continue;
      for (int w = 0; w < 3; ++w) (*v[w])[x] = 0;
      L.h_tab[x] = ExpertRec{};
      // the layer's route copied the old records into its row descriptors: it must be
      // recomputed before an issue may consume it
      L.routed = false;
      int rc = write_table_entry(c, L, (int)x);
      if (rc) return rc;
    }
    if (L.shared_set && (L.shared[0] == h || L.shared[1] == h || L.shared[2] == h)) {
      L.shared[0] = L.shared[1] = L.shared[2] = 0;
      L.shared_set = false;
      L.h_tab[kShared] = ExpertRec{};
      int rc = write_table_entry(c, L, kShared);
      if (rc) return rc;
    }
  }
  dfree(it->second.q);
  dfree(it->second.s);
  c->tensors.erase(it);
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_set_expert(i4moe_ctx *c, int layer, int expert, i4moe_tensor gate, i4moe_tensor up, i4moe_tensor down) try {
  if (!c) return I4MOE_EINVAL;
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  if (layer < 0 || expert < 0 || expert >= kMaxE) return fail(c, I4MOE_EINVAL, "bad layer %d / expert %d", layer, expert);
  auto tg = c->tensors.find(gate), tu = c->tensors.find(up), td = c->tensors.find(down);
  if (tg == c->tensors.end() || tu == c->tensors.end() || td == c->tensors.end())
    return fail(c, I4MOE_EINVAL, "unknown tensor handle");
  const TensorDesc &G = tg->second.desc, &U = tu->second.desc, &Dn = td->second.desc;
  const int I = G.O, D = G.C;
  if (U.O != I || U.C != D || Dn.O != D || Dn.C != I)
    return fail(c, I4MOE_EINVAL, "expert shapes: gate %dx%d, up %dx%d, down %dx%d (need I x D, I x D, D x I)", G.O, G.C,
                U.O, U.C, Dn.O, Dn.C);
  Layer &L = c->layers[layer];
  if ((L.D && L.D != D) || (L.I && L.I != I))
    return fail(c, I4MOE_EINVAL, "layer %d has D=%d I=%d, expert has D=%d I=%d", layer, L.D, L.I, D, I);
  if (L.E && expert >= L.E) return fail(c, I4MOE_EINVAL, "expert %d >= router E=%d", expert, L.E);
  ensure_device(c);
  int rc = ensure_rows_scratch(c, D, I);
  if (rc) return rc;
  if ((rc = ensure_layer_tables(c, L))) return rc;
  L.D = D;
  L.I = I;
  if ((int)L.gate.size() <= expert) {
    L.gate.resize(expert + 1, 0);
    L.up.resize(expert + 1, 0);
    L.down.resize(expert + 1, 0);
  }
  L.gate[expert] = gate;
  L.up[expert] = up;
  L.down[expert] = down;
  L.h_tab[expert].t[0] = G;
  L.h_tab[expert].t[1] = U;
  L.h_tab[expert].t[2] = Dn;
  // A device route copies the expert records into its row descriptors when it runs, so a
  // route taken before this change would still name the old tensors (and the issue would
  // plan its launch from the new ones): the layer has to be routed again.
  L.routed = false;
  return write_table_entry(c, L, expert);
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_upload_router(i4moe_ctx *c, int layer, int E, int D, const float *W, const float *bias) try {
  if (!c) return I4MOE_EINVAL;
  if (layer < 0 || E < 1 || E > kMaxE || D < 1 || !W) return fail(c, I4MOE_EINVAL, "bad router arguments");
  if ((size_t)E * D > ((size_t)1 << 28)) return fail(c, I4MOE_EUNSUPPORTED, "router too large");
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  Layer &L = c->layers[layer];
  bool any_expert = false;
  for (i4moe_tensor g : L.gate) any_expert = any_expert || g != 0;
  if (any_expert && L.D != D) return fail(c, I4MOE_EINVAL, "router D=%d but layer experts have D=%d", D, L.D);
  if ((int)L.gate.size() > E) {
    for (size_t x = E; x < L.gate.size(); ++x)
      if (L.gate[x]) return fail(c, I4MOE_EINVAL, "expert %zu is set but router E=%d", x, E);
  }
  if (!all_finite(W, (size_t)E * D) || (bias && !all_finite(bias, E)))
    return fail(c, I4MOE_EINVAL, "router weights and bias must be finite");
  ensure_device(c);
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  float *dW = nullptr, *db = nullptr;
  if ((e = dalloc(&dW, sizeof(float) * (size_t)E * D)) != hipSuccess) return hip_fail(c, e, "hipMalloc(router)");
  if ((e = dalloc(&db, sizeof(float) * E)) != hipSuccess) {
    dfree(dW);
    return hip_fail(c, e, "hipMalloc(bias)");
  }
  std::vector<float> zeros;
  if (!bias) {
    zeros.assign(E, 0.f);
    bias = zeros.data();
  }
  e = hipMemcpyAsync(dW, W, sizeof(float) * (size_t)E * D, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipMemcpyAsync(db, bias, sizeof(float) * E, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    dfree(dW);
    dfree(db);
    return hip_fail(c, e, "router copy");
  }
  dfree(L.W);
  dfree(L.b);
  L.W = dW;
  L.b = db;
  L.E = E;
  L.D = D;
  L.routed = false;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

// The compute entry points are the fault hook's gate and call count around these bodies; a
// composite call (i4moe_moe_block) gates and counts once around several of them.
// with_shared: the route's group also gets the layer's shared expert, one row per token after the
// routed rows (i4moe_moe_block).
static int route_impl(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S, int K, float topp, int norm_topk,
                      float routed_scale, i4moe_route_host *host_out, bool with_shared = false) {
  int rc = I4MOE_OK;
  Layer *L = find_layer(c, layer);
  if (!L || !L->W) return fail(c, I4MOE_EINVAL, "layer %d has no router", layer);
  if (!x_dev) return fail(c, I4MOE_EINVAL, "x_dev is NULL");
  if (dtype != I4MOE_DTYPE_F32 && dtype != I4MOE_DTYPE_BF16) return fail(c, I4MOE_EINVAL, "bad dtype %d", dtype);
  if (S < 1 || S > kTokens) return fail(c, I4MOE_EINVAL, "S=%d outside 1..%d", S, kTokens);
  if (K < 1 || K > L->E || K > kMaxK) return fail(c, I4MOE_EINVAL, "K=%d outside 1..min(E=%d, %d)", K, L->E, kMaxK);
  if (S * K > kRows) return fail(c, I4MOE_EINVAL, "S*K=%d exceeds the %d-row cap", S * K, kRows);
  if (with_shared && (!L->shared_set || S * K + S > kRows))
    return fail(c, I4MOE_EINVAL, "no shared expert, or S*(K+1)=%d exceeds the %d-row cap", S * (K + 1), kRows);
  if (!std::isfinite(topp) || !std::isfinite(routed_scale)) return fail(c, I4MOE_EINVAL, "topp and scale must be finite");
  ensure_device(c);
  const int ring = c->ring_next;
  for (int s = 0; s < c->nslots; ++s)
    if (c->slots[s].ring == ring)
      return fail(c, I4MOE_EINVAL, "%d routes since a pending issue; take before routing again", kRing);
  // the previous route's selection reads the scores this route overwrites
  if ((rc = flush_sel(c))) return rc;
  if ((rc = ensure_route_scratch(c))) return rc;
  RouteArgs a{};
  a.W = L->W;
  a.bias = L->b;
  a.x = x_dev;
  a.score = c->d_score;
  a.logits = c->d_logits;
  a.out = c->d_ring + ring;
  a.table = L->d_tab;
  a.E = L->E;
  a.D = L->D;
  a.S = S;
  a.K = K;
  a.x_bf16 = dtype == I4MOE_DTYPE_BF16;
  gemv_geometry(*L, a);
  a.vec = (L->D % 4 == 0) && reinterpret_cast<uintptr_t>(L->W) % 16 == 0 &&
          reinterpret_cast<uintptr_t>(x_dev) % (dtype == I4MOE_DTYPE_F32 ? 16 : 8) == 0;
  a.norm_topk = norm_topk ? 1 : 0;
  a.topp = topp;
  a.routed_scale = routed_scale;
  a.shared_rows = with_shared ? 1 : 0;
  // Without a host copy a one-token route defers its selection to the issue that consumes it.
  const bool defer = !host_out && dual_sel_ok(a, false);
  const int parts = defer ? kRouteGemv : kRouteGemv | kRouteSelect;
  hipError_t e = timed(c, I4MOE_K_ROUTE, [&](hipEvent_t t0, hipEvent_t t1) {
    return launch_route(a, parts, c->stream, t0, t1);
  });
  if (e != hipSuccess) return hip_fail(c, e, "route launch");
  if (defer) {
    c->sel_pending = true;
    c->sel_layer = layer;
    c->sel_args = a;
  }
  c->ring_next = (ring + 1) % kRing;
  L->route_buf = ring;
  L->routed = true;
  L->route_S = S;
  L->route_K = K;
  L->route_shared = with_shared;
  c->last_route_S = S;
  c->last_route_E = L->E;
  if (host_out) {
    e = hipMemcpyAsync(host_out, c->d_ring[ring].route, sizeof(RouteTok) * S, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "route copy back");
  }
  return I4MOE_OK;
}

int i4moe_route(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S, int K, float topp, int norm_topk,
                float routed_scale, i4moe_route_host *host_out) try {
  if (!c) return I4MOE_EINVAL;
  int rc = gate_compute(c);
  if (rc) return rc;
  rc = route_impl(c, layer, x_dev, dtype, S, K, topp, norm_topk, routed_scale, host_out);
  if (rc == I4MOE_OK) c->calls++;
  return rc;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_route_noalloc(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S, int K, float topp, int norm_topk,
                        float routed_scale, i4moe_route_host *route_dev) try {
  if (!c) return I4MOE_EINVAL;
  int rc = gate_compute(c);
  if (rc) return rc;
  Layer *L = find_layer(c, layer);
  if (!L || !L->W) return fail(c, I4MOE_EINVAL, "layer %d has no router", layer);
  if (!x_dev || !route_dev) return fail(c, I4MOE_EINVAL, "x_dev and route_dev must be device pointers");
  if (reinterpret_cast<uintptr_t>(route_dev) % 4 != 0) return fail(c, I4MOE_EINVAL, "route_dev must be 4-byte aligned");
  if (dtype != I4MOE_DTYPE_F32 && dtype != I4MOE_DTYPE_BF16) return fail(c, I4MOE_EINVAL, "bad dtype %d", dtype);
  // the static scratch holds the scores of at most kTokens tokens of kMaxE experts and one group
  if (S < 1 || S > kTokens)
    return fail(c, I4MOE_EUNSUPPORTED, "S=%d outside 1..%d (the static route scratch holds %d tokens)", S, kTokens, kTokens);
  if (L->E > kMaxE) return fail(c, I4MOE_EUNSUPPORTED, "E=%d exceeds the static route scratch (%d experts)", L->E, kMaxE);
  if (K < 1 || K > L->E || K > kMaxK) return fail(c, I4MOE_EINVAL, "K=%d outside 1..min(E=%d, %d)", K, L->E, kMaxK);
  if (S * K > kRows)
    return fail(c, I4MOE_EUNSUPPORTED, "S*K=%d exceeds the %d rows of the static route scratch", S * K, kRows);
  if (!std::isfinite(topp) || !std::isfinite(routed_scale)) return fail(c, I4MOE_EINVAL, "topp and scale must be finite");
  if (!c->scratch) return fail(c, I4MOE_EDEVICE, "static route scratch has no device address");
  ensure_device(c);
  // Every part of the route's working memory comes from this device's static scratch, addressed
  // through the pointer looked up at context creation: scores, logits, then the group buffer the
  // selection writes.  Each is fully written by this call's kernels before it is read, so
  // nothing needs clearing.
  uint8_t *base = static_cast<uint8_t *>(c->scratch);
  RouteArgs a{};
  a.W = L->W;
  a.bias = L->b;
  a.x = x_dev;
  a.score = reinterpret_cast<double2 *>(base);
  a.logits = reinterpret_cast<double *>(base + kScoreBytes);
  a.out = reinterpret_cast<GroupBuf *>(base + kScoreBytes + kLogitBytes);
  a.table = nullptr;  // routes only: no row descriptors
  a.E = L->E;
  a.D = L->D;
  a.S = S;
  a.K = K;
  a.x_bf16 = dtype == I4MOE_DTYPE_BF16;
  gemv_geometry(*L, a);
  a.vec = (L->D % 4 == 0) && reinterpret_cast<uintptr_t>(L->W) % 16 == 0 &&
          reinterpret_cast<uintptr_t>(x_dev) % (dtype == I4MOE_DTYPE_F32 ? 16 : 8) == 0;
  a.norm_topk = norm_topk ? 1 : 0;
  a.topp = topp;
  a.routed_scale = routed_scale;
  hipError_t e = launch_route(a, kRouteGemv | kRouteSelect, c->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(route_dev, a.out->route, sizeof(RouteTok) * S, hipMemcpyDeviceToDevice, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "route launch");
  c->calls++;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

// allow_shared: the group may name the layer's shared expert (kShared).
static int issue_impl(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S, const i4moe_group *group,
                      bool allow_shared) {
  int rc = I4MOE_OK;
  Layer *L = find_layer(c, layer);
  if (!L || !L->D || !L->I || !L->d_tab) return fail(c, I4MOE_EINVAL, "layer %d has no experts", layer);
  if (!x_dev) return fail(c, I4MOE_EINVAL, "x_dev is NULL");
  if (dtype != I4MOE_DTYPE_F32 && dtype != I4MOE_DTYPE_BF16) return fail(c, I4MOE_EINVAL, "bad dtype %d", dtype);
  if (S < 1 || S > kTokens) return fail(c, I4MOE_EINVAL, "S=%d outside 1..%d", S, kTokens);
  if (reinterpret_cast<uintptr_t>(x_dev) % (dtype == I4MOE_DTYPE_F32 ? 8 : 4) != 0)
    return fail(c, I4MOE_EINVAL, "x_dev must be %d-byte aligned", dtype == I4MOE_DTYPE_F32 ? 8 : 4);
  if (c->nslots >= kSlots) return fail(c, I4MOE_EINVAL, "%d issues pending; take before issuing more", kSlots);
  if (c->nslots > 0 && (c->slots[0].S != S || c->slots[0].D != L->D))
    return fail(c, I4MOE_EINVAL, "pending issues have S=%d D=%d; this issue has S=%d D=%d", c->slots[0].S,
                c->slots[0].D, S, L->D);
  ensure_device(c);

  // The experts this issue may touch decide the kernel variant.
  std::vector<int> gs_in, gs_dn;
  auto note = [&](int e) {
    const TensorDesc &g = L->h_tab[e].t[0], &u = L->h_tab[e].t[1], &d = L->h_tab[e].t[2];
    if (g.ng > 1) gs_in.push_back(g.gs);
    if (u.ng > 1) gs_in.push_back(u.gs);
    if (d.ng > 1) gs_dn.push_back(d.gs);
  };
  const int s = c->nslots;
  int max_rows = 0;
  const GroupBuf *grp = nullptr;
  int ring = -1;
  GroupDev hg;
  if (!group) {
    if (!L->routed) return fail(c, I4MOE_EINVAL, "layer %d has no device route; call i4moe_route first", layer);
    if (L->route_S != S) return fail(c, I4MOE_EINVAL, "route has S=%d, issue has S=%d", L->route_S, S);
    if ((int)L->gate.size() < L->E) return fail(c, I4MOE_EINVAL, "layer %d: experts 0..%d must all be set", layer, L->E - 1);
    for (int e = 0; e < L->E; ++e) {
      if (!L->gate[e]) return fail(c, I4MOE_EINVAL, "layer %d: expert %d is not set", layer, e);
      note(e);
    }
    if (L->route_shared) {
      if (!L->shared_set) return fail(c, I4MOE_EINVAL, "layer %d: the route's shared expert is gone", layer);
      note(kShared);
    }
    max_rows = S * L->route_K + (L->route_shared ? S : 0);
    ring = L->route_buf;
    grp = c->d_ring + ring;
  } else {
    const int n = group->n_rows;
    if (n < 1 || n > kRows || !group->expert || !group->token || !group->weight)
      return fail(c, I4MOE_EINVAL, "explicit group needs 1..%d rows and non-NULL arrays", kRows);
    std::memset(&hg, 0, sizeof hg);
    int order[kRows];
    int n_ent = 0, ent_of[kRows];
    for (int r = 0; r < n; ++r) {
      const int e = group->expert[r], t = group->token[r];
      const bool shared = allow_shared && e == kShared && L->shared_set;
      if (!shared && (e < 0 || e >= (int)L->gate.size() || !L->gate[e]))
        return fail(c, I4MOE_EINVAL, "group row %d: expert %d is not set", r, e);
      if (t < 0 || t >= S) return fail(c, I4MOE_EINVAL, "group row %d: token %d outside 0..%d", r, t, S - 1);
      if (!std::isfinite(group->weight[r])) return fail(c, I4MOE_EINVAL, "group row %d: weight not finite", r);
      int j = 0;
      while (j < n_ent && hg.entry_expert[j] != e) ++j;
      if (j == n_ent) hg.entry_expert[n_ent++] = e;
      ent_of[r] = j;
      note(e);
    }
    // rows entry-major, listed order inside an entry
    int pos = 0;
    for (int j = 0; j < n_ent; ++j) {
      hg.entry_row0[j] = pos;
      for (int r = 0; r < n; ++r)
        if (ent_of[r] == j) order[r] = pos++;
    }
    hg.entry_row0[n_ent] = pos;
    for (int r = 0; r < n; ++r) {
      hg.row_token[order[r]] = group->token[r];
      hg.row_expert[order[r]] = group->expert[r];
      hg.row_weight[order[r]] = group->weight[r];
    }
    // reduce order per token: listed order
    int q = 0;
    for (int t = 0; t < S; ++t) {
      hg.tok_row0[t] = q;
      for (int r = 0; r < n; ++r)
        if (group->token[r] == t) hg.red_rows[q++] = order[r];
    }
    hg.tok_row0[S] = q;
    hg.n_entries = n_ent;
    hg.n_rows = n;
    hg.S = S;
    max_rows = n;
    grp = c->d_slot_bufs + s;
  }

  const Plan pd = plan_proj(L->D, L->I, max_rows, true, gs_in, c->n_cu, c->wave_factor);
  const Plan pn = plan_proj(L->I, L->D, max_rows, false, gs_dn, c->n_cu, c->wave_factor);
  ProjArgs ad{};
  ad.grp = grp;
  ad.act = x_dev;
  ad.act_ld = L->D;
  ad.act_bf16 = dtype == I4MOE_DTYPE_BF16;
  ad.out = c->d_h;
  ad.out_ld = c->h_ld;
  ad.O = L->I;
  ad.C = L->D;
  ad.tile_groups = pd.tile_groups;
  ad.grid_rows = max_rows;
  ad.tile_rows = pd.tile_rows;
  ProjArgs an{};
  an.grp = grp;
  an.act = c->d_h;
  an.act_ld = c->h_ld;
  an.act_bf16 = 0;
  an.out = c->d_y + (size_t)s * kRows * c->y_ld;
  an.out_ld = c->y_ld;
  an.O = L->D;
  an.C = L->I;
  an.tile_groups = pn.tile_groups;
  an.grid_rows = max_rows;
  an.tile_rows = pn.tile_rows;
  // Several tokens: the rows of one expert may share each weight pass (I4MOE_ENTRY_ROWS).  Not
  // by default: measured on the small-batch shape at 1 to 64 rows per expert, the shared passes
  // were slower than one row per workgroup at every row count (rows of one expert that run
  // together re-read its weights mostly from L2 and the Infinity Cache, while a workgroup running
  // nr rows does nr times the dot products per weight byte); from 8 rows the matrix cores win.
  if (S > 1 && c->entry_mode > 0) {
    int most = S;  // a device route gives an expert at most one row per token
    if (group) {
      most = 0;
      for (int j = 0; j < hg.n_entries; ++j) most = std::max(most, hg.entry_row0[j + 1] - hg.entry_row0[j]);
    }
    const int want = std::min(most, c->entry_mode);
    const int ed = entry_rows_fit(pd.V, pd.P, false, want);
    const int en = entry_rows_fit(pn.V, pn.P, pn.rows16, want);
    if (ed > 1 && !pd.gen) ad.entry_rows = ed;
    if (en > 1 && (pn.rows16 || !pn.gen)) an.entry_rows = en;
  }

  // Entries of at least mfma_min rows run on the matrix cores (every tensor of the issue per-row
  // or with group sizes that are multiples of 64); the vector kernels then take the chunked path,
  // which skips those entries.
  int mfma_min = 0, mfma_slots = 0, ks_dual = 1, ks_down = 1;
  bool vec_rows = true;  // some entry runs on the vector kernels (always possible for a device route)
  if (S > 1 && c->mfma_min > 0) {
    bool fmt_ok = true;
    for (int gs : gs_in) fmt_ok = fmt_ok && gs % 64 == 0;
    for (int gs : gs_dn) fmt_ok = fmt_ok && gs % 64 == 0;
    int most = S, n_big = max_rows / c->mfma_min;  // a device route: at most one row per token
    if (group) {
      most = n_big = 0;
      for (int j = 0; j < hg.n_entries; ++j) {
        const int n = hg.entry_row0[j + 1] - hg.entry_row0[j];
        most = std::max(most, n);
        if (n >= c->mfma_min) ++n_big;
      }
      vec_rows = n_big < hg.n_entries;
    }
    if (fmt_ok && most >= c->mfma_min && n_big > 0) {
      mfma_min = c->mfma_min;
      mfma_slots = n_big;
      ks_dual = mfma_ksplit(L->I, round_up(L->D, 64), n_big, c->n_cu, most);
      ks_down = mfma_ksplit(L->D, round_up(L->I, 64), n_big, c->n_cu, most);
      if ((rc = ensure_digit_scratch(c))) return rc;
      if ((rc = ensure_part_scratch(c, std::max(mfma_part_floats(2, L->I, n_big, ks_dual),
                                                 mfma_part_floats(1, L->D, n_big, ks_down)))))
        return rc;
      ad.mfma_min = an.mfma_min = mfma_min;
      if (ad.entry_rows == 0) ad.entry_rows = 1;
      if (an.entry_rows == 0) an.entry_rows = 1;
    } else {
      vec_rows = true;
    }
  }

  // This layer's latest route still owes its selection: run it inside the dual projection
  // when that variant can, else as its own kernel first.
  bool sel = false;
  if (!group && c->sel_pending && c->sel_layer == layer && c->sel_args.out == grp) {
    if (dual_sel_ok(c->sel_args, pd.gen)) {
      sel = true;
      ad.ra = c->sel_args;
    } else if ((rc = flush_sel(c))) {
      return rc;
    }
  }
  // a waiting down projection reads h, which this issue's dual projection overwrites
  if ((rc = flush_down(c))) return rc;
  // A lone one-token issue of a device route leaves its down projection to the take.
  const bool defer_down = S == 1 && !group && s == 0 && pn.rows16 && max_rows <= kDTRows;
  hipError_t e = hipSuccess;
  if (group) e = launch_group_store(hg, L->d_tab, c->d_slot_bufs + s, c->stream);
  // matrix-core launches of one projection: the dual's digit rows of x, the projection of the
  // big entries (after the vector kernels of the same projection) and its reduction, which for
  // the dual also writes the digit rows of h that the down projection reads
  auto mfma = [&](bool dual) -> hipError_t {
    DigitArgs da{};
    da.act = x_dev;
    da.dig = c->d_dig;
    da.E = c->d_dig_E;
    da.act_ld = L->D;
    da.bf16 = dtype == I4MOE_DTYPE_BF16;
    da.rows = S;
    da.C = L->D;
    da.C64 = round_up(L->D, 64);
    MfmaArgs ma{};
    ma.grp = grp;
    ma.dig = c->d_dig;
    ma.E = dual ? c->d_dig_E : c->d_dig_E + kRows;
    ma.out = dual ? c->d_h : an.out;
    ma.out_ld = dual ? c->h_ld : c->y_ld;
    ma.dig_out = dual ? c->d_dig : nullptr;
    ma.E_out = dual ? c->d_dig_E + kRows : nullptr;
    ma.dig_rows = dual ? S : max_rows;
    ma.dual = dual ? 1 : 0;
    ma.O = dual ? L->I : L->D;
    ma.C64 = dual ? da.C64 : round_up(L->I, 64);
    ma.mfma_min = mfma_min;
    ma.slots = mfma_slots;
    ma.ksplit = dual ? ks_dual : ks_down;
    ma.row_acc = (dual ? gs_in : gs_dn).empty() ? 1 : 0;
    ma.part = c->d_part;
    return timed(c, I4MOE_K_MFMA, [&](hipEvent_t t0, hipEvent_t t1) {
      // the event pair spans the projection's launches
      if (!dual) return launch_mfma(1, ma, c->stream, t0, t1);
      hipError_t r = launch_digits8(da, c->stream, t0, nullptr);
      return r != hipSuccess ? r : launch_mfma(2, ma, c->stream, nullptr, t1);
    });
  };
  if (e == hipSuccess && vec_rows) e = timed(c, I4MOE_K_DUAL, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_dual(pd.V, pd.P, pd.gen, sel, ad, pd.blocks, c->stream, t0, t1);
    });
  if (e == hipSuccess && sel) c->sel_pending = false;
  if (e == hipSuccess && mfma_min) e = mfma(true);
  if (e == hipSuccess && !defer_down && vec_rows) e = timed(c, I4MOE_K_DOWN, [&](hipEvent_t t0, hipEvent_t t1) {
      return pn.rows16 ? launch_down16(pn.P, an, pn.blocks, c->stream, t0, t1)
                       : launch_down(pn.V, pn.P, pn.gen, an, pn.blocks, c->stream, t0, t1);
    });
  if (e == hipSuccess && mfma_min) e = mfma(false);
  if (e != hipSuccess) return hip_fail(c, e, "issue launch");
  c->slots[s].down_pending = defer_down;
  if (defer_down) {
    c->slots[s].down_P = pn.P;
    c->slots[s].down_blocks = pn.blocks;
    c->slots[s].down = an;
  }
  c->slots[s].S = S;
  c->slots[s].D = L->D;
  c->slots[s].rows = max_rows;
  c->slots[s].grp = grp;
  c->slots[s].ring = ring;
  c->nslots = s + 1;
  c->last_issue_rows = max_rows;
  c->last_issue_I = L->I;
  return s;
}

int i4moe_expert_group_issue(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S, const i4moe_group *group) try {
  if (!c) return I4MOE_EINVAL;
  int rc = gate_compute(c);
  if (rc) return rc;
  rc = issue_impl(c, layer, x_dev, dtype, S, group, false);
  if (rc >= 0) c->calls++;
  return rc;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

// A failure here poisons the context (the routed experts would be dropped silently).
static int take_impl(i4moe_ctx *c, float *residual_dev, int S) {
  int rc = I4MOE_OK;
  if (c->nslots == 0) return I4MOE_OK;
  if (!residual_dev || S != c->slots[0].S) {
    c->poisoned = true;
    return fail(c, I4MOE_EINVAL, "take: residual NULL or S=%d differs from the issued S=%d", S, c->slots[0].S);
  }
  ensure_device(c);
  if (c->nslots == 1 && c->slots[0].down_pending && c->slots[0].ring >= 0 && S == 1) {
    // the lone slot's down projection and the take in one launch
    SlotInfo &si = c->slots[0];
    ProjArgs dt = si.down;
    dt.out = residual_dev;
    hipError_t e = timed(c, I4MOE_K_TAKE, [&](hipEvent_t t0, hipEvent_t t1) {
      return launch_down_take(si.down_P, dt, c->stream, t0, t1);
    });
    if (e != hipSuccess) {
      c->poisoned = true;
      return hip_fail(c, e, "take launch");
    }
    si.down_pending = false;
    c->nslots = 0;
    return I4MOE_OK;
  }
  if ((rc = flush_down(c))) {
    c->poisoned = true;
    return rc;
  }
  TakeArgs a{};
  // Device routes at S = 1 hold distinct experts, one row each in route order, live rows first:
  // the take can then read everything without first reading the reduce order.
  a.in_order = S == 1 ? 1 : 0;
  for (int s = 0; s < c->nslots; ++s) {
    a.groups[s] = c->slots[s].grp;
    a.y[s] = c->d_y + (size_t)s * kRows * c->y_ld;
    a.rows[s] = c->slots[s].rows;
    if (c->slots[s].ring < 0) a.in_order = 0;  // explicit groups reduce in their listed order
  }
  a.resid = residual_dev;
  a.nslots = c->nslots;
  a.y_ld = c->y_ld;
  a.S = S;
  a.D = c->slots[0].D;
  hipError_t e = timed(c, I4MOE_K_TAKE, [&](hipEvent_t t0, hipEvent_t t1) { return launch_take(a, c->stream, t0, t1); });
  if (e != hipSuccess) {
    c->poisoned = true;
    return hip_fail(c, e, "take launch");
  }
  c->nslots = 0;
  return I4MOE_OK;
}

int i4moe_expert_group_take(i4moe_ctx *c, float *residual_dev, int S) try {
  if (!c) return I4MOE_EINVAL;
  if (c->poisoned) return fail(c, I4MOE_EPOISONED, "context poisoned by a failed take");
  int rc = gate_compute(c);
  if (rc) {
    c->poisoned = true;
    return rc;
  }
  rc = take_impl(c, residual_dev, S);
  if (rc == I4MOE_OK) c->calls++;
  return rc;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_set_shared_expert(i4moe_ctx *c, int layer, i4moe_tensor gate, i4moe_tensor up, i4moe_tensor down) try {
  if (!c) return I4MOE_EINVAL;
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  if (layer < 0) return fail(c, I4MOE_EINVAL, "bad layer %d", layer);
  auto tg = c->tensors.find(gate), tu = c->tensors.find(up), td = c->tensors.find(down);
  if (tg == c->tensors.end() || tu == c->tensors.end() || td == c->tensors.end())
    return fail(c, I4MOE_EINVAL, "unknown tensor handle");
  const TensorDesc &G = tg->second.desc, &U = tu->second.desc, &Dn = td->second.desc;
  const int I = G.O, D = G.C;
  if (U.O != I || U.C != D || Dn.O != D || Dn.C != I)
    return fail(c, I4MOE_EINVAL, "shared expert shapes: gate %dx%d, up %dx%d, down %dx%d (need I x D, I x D, D x I)",
                G.O, G.C, U.O, U.C, Dn.O, Dn.C);
  Layer &L = c->layers[layer];
  if ((L.D && L.D != D) || (L.I && L.I != I))
    return fail(c, I4MOE_EINVAL, "layer %d has D=%d I=%d, shared expert has D=%d I=%d", layer, L.D, L.I, D, I);
  int rc = ensure_rows_scratch(c, D, I);
  if (rc) return rc;
  if ((rc = ensure_layer_tables(c, L))) return rc;
  L.D = D;
  L.I = I;
  L.shared[0] = gate;
  L.shared[1] = up;
  L.shared[2] = down;
  L.shared_set = true;
  L.h_tab[kShared].t[0] = G;
  L.h_tab[kShared].t[1] = U;
  L.h_tab[kShared].t[2] = Dn;
  return write_table_entry(c, L, kShared);
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_upload_norm(i4moe_ctx *c, int layer, int D, const float *gamma, float eps) try {
  if (!c) return I4MOE_EINVAL;
  if (layer < 0 || D < 1 || !gamma) return fail(c, I4MOE_EINVAL, "bad norm arguments");
  if (!std::isfinite(eps) || eps < 0.f) return fail(c, I4MOE_EINVAL, "eps must be finite and >= 0");
  if (!all_finite(gamma, (size_t)D)) return fail(c, I4MOE_EINVAL, "gamma must be finite");
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  Layer &L = c->layers[layer];
  if (L.D && L.D != D) return fail(c, I4MOE_EINVAL, "norm D=%d but layer %d has D=%d", D, layer, L.D);
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  float *g = nullptr;
  if ((e = dalloc(&g, sizeof(float) * D)) != hipSuccess) return hip_fail(c, e, "hipMalloc(gamma)");
  e = hipMemcpyAsync(g, gamma, sizeof(float) * D, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    dfree(g);
    return hip_fail(c, e, "norm copy");
  }
  dfree(L.gamma);
  L.gamma = g;
  L.eps = eps;
  if (!L.D) L.D = D;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

// The block's normalised rows, [kTokens][D] of float32 (bf16 uses half of it).  Grows only with
// no issue pending (an issue may still read the old buffer).
static int ensure_xn(i4moe_ctx *c, int D) {
  const int need = round_up(D, 64);
  if (need <= c->xn_ld) return I4MOE_OK;
  if (c->nslots > 0) return fail(c, I4MOE_EINVAL, "cannot grow the block scratch while %d issue(s) are pending", c->nslots);
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  float *p = nullptr;
  if ((e = dalloc(&p, sizeof(float) * (size_t)kTokens * need)) != hipSuccess) return hip_fail(c, e, "hipMalloc(xn)");
  dfree(c->d_xn);
  c->d_xn = p;
  c->xn_ld = need;
  return I4MOE_OK;
}

static int rmsnorm_impl(i4moe_ctx *c, const Layer &L, const float *x_dev, int ld_x, int S, void *out_dev, int ld_out,
                        int out_dtype) {
  NormArgs a{};
  a.x = x_dev;
  a.gamma = L.gamma;
  a.out = out_dev;
  a.ld_x = ld_x;
  a.ld_out = ld_out;
  a.S = S;
  a.D = L.D;
  a.out_bf16 = out_dtype == I4MOE_DTYPE_BF16;
  a.eps = L.eps;
  hipError_t e = launch_rmsnorm(a, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "rmsnorm launch");
  return I4MOE_OK;
}

int i4moe_rmsnorm(i4moe_ctx *c, int layer, const float *x_dev, int ld_x, int S, void *out_dev, int ld_out,
                  int out_dtype) try {
  if (!c) return I4MOE_EINVAL;
  int rc = gate_compute(c);
  if (rc) return rc;
  Layer *L = find_layer(c, layer);
  if (!L || !L->gamma) return fail(c, I4MOE_EINVAL, "layer %d has no norm weights", layer);
  if (!x_dev || !out_dev) return fail(c, I4MOE_EINVAL, "x_dev and out_dev must be device pointers");
  if (out_dtype != I4MOE_DTYPE_F32 && out_dtype != I4MOE_DTYPE_BF16) return fail(c, I4MOE_EINVAL, "bad dtype %d", out_dtype);
  if (S < 1 || S > kTokens) return fail(c, I4MOE_EINVAL, "S=%d outside 1..%d", S, kTokens);
  if (ld_x < L->D || ld_out < L->D) return fail(c, I4MOE_EINVAL, "row strides %d, %d below D=%d", ld_x, ld_out, L->D);
  if (reinterpret_cast<uintptr_t>(x_dev) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(out_dev) % (out_dtype == I4MOE_DTYPE_F32 ? 4 : 2) != 0)
    return fail(c, I4MOE_EINVAL, "misaligned rows");
  ensure_device(c);
  rc = rmsnorm_impl(c, *L, x_dev, ld_x, S, out_dev, ld_out, out_dtype);
  if (rc == I4MOE_OK) c->calls++;
  return rc;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

// The shared expert's group: one row per token, weight 1, listed in token order.
static int shared_issue_impl(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S) {
  Layer *L = find_layer(c, layer);
  if (!L || !L->shared_set) return fail(c, I4MOE_EINVAL, "layer %d has no shared expert", layer);
  if (S < 1 || S > kTokens) return fail(c, I4MOE_EINVAL, "S=%d outside 1..%d", S, kTokens);
  int32_t ex[kTokens], tok[kTokens];
  float w[kTokens];
  for (int t = 0; t < S; ++t) {
    ex[t] = kShared;
    tok[t] = t;
    w[t] = 1.f;
  }
  const i4moe_group g{S, ex, tok, w};
  return issue_impl(c, layer, x_dev, dtype, S, &g, true);
}

int i4moe_shared_expert_issue(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S) try {
  if (!c) return I4MOE_EINVAL;
  int rc = gate_compute(c);
  if (rc) return rc;
  rc = shared_issue_impl(c, layer, x_dev, dtype, S);
  if (rc >= 0) c->calls++;
  return rc;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_moe_block(i4moe_ctx *c, int layer, float *residual_dev, int S, int act_dtype, int K, float topp,
                    int norm_topk, float routed_scale) try {
  if (!c) return I4MOE_EINVAL;
  if (c->poisoned) return fail(c, I4MOE_EPOISONED, "context poisoned by a failed take");
  int rc = gate_compute(c);
  if (rc) return rc;
  Layer *L = find_layer(c, layer);
  if (!L || !L->W || !L->gamma || !L->I || !L->d_tab)
    return fail(c, I4MOE_EINVAL, "layer %d needs a router, norm weights and experts", layer);
  if (!residual_dev || reinterpret_cast<uintptr_t>(residual_dev) % 16 != 0)
    return fail(c, I4MOE_EINVAL, "residual_dev must be a 16-byte aligned device pointer");
  if (act_dtype != I4MOE_DTYPE_F32 && act_dtype != I4MOE_DTYPE_BF16) return fail(c, I4MOE_EINVAL, "bad dtype %d", act_dtype);
  if (S < 1 || S > kTokens) return fail(c, I4MOE_EINVAL, "S=%d outside 1..%d", S, kTokens);
  if (K < 1 || K > L->E || K > kMaxK || S * K > kRows)
    return fail(c, I4MOE_EINVAL, "K=%d with S=%d outside the route's limits", K, S);
  // the shared expert rides in the routed group when its rows fit beside the routed ones
  const bool merge = L->shared_set && S * K + S <= kRows;
  if (c->nslots + (L->shared_set && !merge ? 2 : 1) > kSlots) return fail(c, I4MOE_EINVAL, "no free issue slots");
  if (c->nslots > 0 && (c->slots[0].S != S || c->slots[0].D != L->D))
    return fail(c, I4MOE_EINVAL, "pending issues have another S or D");
  if ((int)L->gate.size() < L->E) return fail(c, I4MOE_EINVAL, "layer %d: experts 0..%d must all be set", layer, L->E - 1);
  for (int e = 0; e < L->E; ++e)
    if (!L->gate[e]) return fail(c, I4MOE_EINVAL, "layer %d: expert %d is not set", layer, e);
  ensure_device(c);
  if ((rc = ensure_xn(c, L->D))) return rc;
  // From the first launch on, a failure leaves the residual without its experts: poison, as a
  // failed take does.
  // the normalised rows are packed [S][D] (what the route and the issues read)
  rc = rmsnorm_impl(c, *L, residual_dev, L->D, S, c->d_xn, L->D, act_dtype);
  // the shared expert rides in the routed group as one more row per token (weight 1, after the
  // routed rows): one issue and one slot, the same sums as a separate shared issue taken after it,
  // which is what runs when the rows do not fit one group
  if (!rc) rc = route_impl(c, layer, c->d_xn, act_dtype, S, K, topp, norm_topk, routed_scale, nullptr, merge);
  if (!rc) {
    const int s = issue_impl(c, layer, c->d_xn, act_dtype, S, nullptr, false);
    if (s < 0) rc = s;
  }
  if (!rc && L->shared_set && !merge) {
    const int s = shared_issue_impl(c, layer, c->d_xn, act_dtype, S);
    if (s < 0) rc = s;
  }
  if (!rc) rc = take_impl(c, residual_dev, S);
  if (rc) {
    c->poisoned = true;
    return rc;
  }
  c->calls++;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_set_fail_after(i4moe_ctx *c, long long n) try {
  if (!c) return I4MOE_EINVAL;
  c->fail_after = n < 0 ? -1 : n;
  c->calls = 0;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

size_t i4moe_debug_size(i4moe_ctx *c, int what, int index) try {
  if (!c) return 0;
  switch (what) {
    case I4MOE_TAP_LOGITS:
      return sizeof(double) * (size_t)c->last_route_S * c->last_route_E;
    case I4MOE_TAP_ROUTE: {
      Layer *L = find_layer(c, index);
      return (L && L->routed) ? sizeof(RouteTok) * L->route_S : 0;
    }
    case I4MOE_TAP_GROUP: {
      Layer *L = find_layer(c, index);
      return (L && L->routed) ? sizeof(GroupDev) : 0;
    }
    case I4MOE_TAP_H:
      return sizeof(float) * (size_t)c->last_issue_rows * c->last_issue_I;
    case I4MOE_TAP_Y:
      return (index >= 0 && index < c->nslots) ? sizeof(float) * (size_t)c->slots[index].rows * c->slots[index].D : 0;
    default:
      return 0;
  }
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return 0;
}

int i4moe_debug_read(i4moe_ctx *c, int what, int index, void *host_dst, size_t bytes) try {
  if (!c || !host_dst) return I4MOE_EINVAL;
  const size_t need = i4moe_debug_size(c, what, index);
  if (need == 0 || bytes != need) return fail(c, I4MOE_EINVAL, "tap %d/%d: need %zu bytes, got %zu", what, index, need, bytes);
  ensure_device(c);
  if (int rc = flush_all(c)) return rc;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "hipStreamSynchronize");
  if (what == I4MOE_TAP_LOGITS) {
    e = hipMemcpy(host_dst, c->d_logits, bytes, hipMemcpyDeviceToHost);
  } else if (what == I4MOE_TAP_ROUTE) {
    e = hipMemcpy(host_dst, c->d_ring[find_layer(c, index)->route_buf].route, bytes, hipMemcpyDeviceToHost);
  } else if (what == I4MOE_TAP_GROUP) {
    e = hipMemcpy(host_dst, &c->d_ring[find_layer(c, index)->route_buf].g, bytes, hipMemcpyDeviceToHost);
  } else if (what == I4MOE_TAP_H) {
    e = hipMemcpy2D(host_dst, sizeof(float) * c->last_issue_I, c->d_h, sizeof(float) * c->h_ld,
                    sizeof(float) * c->last_issue_I, c->last_issue_rows, hipMemcpyDeviceToHost);
  } else {
    const SlotInfo &si = c->slots[index];
    e = hipMemcpy2D(host_dst, sizeof(float) * si.D, c->d_y + (size_t)index * kRows * c->y_ld, sizeof(float) * c->y_ld,
                    sizeof(float) * si.D, si.rows, hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) return hip_fail(c, e, "tap copy");
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

// ---- the CPU tier ----------------------------------------------------------------------------

static int host_tensor_copy(i4moe_ctx *c, const i4moe_host_tensor *h, const char *what, HostTensor &t) {
  if (!h) return fail(c, I4MOE_EINVAL, "%s: NULL tensor", what);
  if (h->fmt != I4MOE_FMT_ROW && h->fmt != I4MOE_FMT_GROUP)
    return fail(c, I4MOE_EUNSUPPORTED, "%s: unsupported weight format %d", what, h->fmt);
  if ((h->fmt == I4MOE_FMT_ROW && h->gs != 0) || (h->fmt == I4MOE_FMT_GROUP && (h->gs < 0 || h->gs % 2 != 0)))
    return fail(c, I4MOE_EINVAL, "%s: bad group size %d for format %d", what, h->gs, h->fmt);
  if (h->O < 1 || h->C < 2 || h->C % 2 != 0 || h->C > kMaxCols)
    return fail(c, I4MOE_EINVAL, "%s: bad shape %d x %d", what, h->O, h->C);
  if (!h->packed || !h->scales) return fail(c, I4MOE_EINVAL, "%s: packed and scales must be non-NULL", what);
  t.O = h->O;
  t.C = h->C;
  t.gs = h->fmt == I4MOE_FMT_GROUP ? h->gs : 0;
  t.ng = t.gs > 0 ? (h->C + t.gs - 1) / t.gs : 1;
  if (!all_finite(h->scales, (size_t)t.O * t.ng)) return fail(c, I4MOE_EINVAL, "%s: scales must be finite", what);
  try {
    t.packed.assign(h->packed, h->packed + (size_t)t.O * (t.C / 2));
    t.scales.assign(h->scales, h->scales + (size_t)t.O * t.ng);
  } catch (const std::bad_alloc &) {
    return fail(c, I4MOE_ENOMEM, "%s: host memory", what);
  }
  return I4MOE_OK;
}

int i4moe_host_rows(int S, int D, int I, int n_rows, const int32_t *token, const float *weight,
                    const i4moe_host_tensor *gate, const i4moe_host_tensor *up, const i4moe_host_tensor *down,
                    const float *x, float *P, int threads) try {
  if (S < 1 || D < 2 || I < 2 || n_rows < 0 || threads < 1 || threads > 256 || !x || !P) return I4MOE_EINVAL;
  if (n_rows > 0 && (!token || !weight || !gate || !up || !down)) return I4MOE_EINVAL;
  std::vector<HostExpert> ex;
  std::vector<HostRow> rows;
  try {
    ex.resize(n_rows);
    rows.reserve(n_rows);
  } catch (const std::bad_alloc &) {
    return I4MOE_ENOMEM;
  }
  // the same checks as i4moe_set_host_expert, without a context to report them on
  auto copy = [](const i4moe_host_tensor &h, int O, int C, HostTensor &t) -> int {
    if (h.O != O || h.C != C || h.C % 2 != 0 || h.C > kMaxCols || !h.packed || !h.scales) return I4MOE_EINVAL;
    if (h.fmt != I4MOE_FMT_ROW && h.fmt != I4MOE_FMT_GROUP) return I4MOE_EUNSUPPORTED;
    if ((h.fmt == I4MOE_FMT_ROW && h.gs != 0) || (h.fmt == I4MOE_FMT_GROUP && (h.gs < 0 || h.gs % 2 != 0)))
      return I4MOE_EINVAL;
    t.O = O;
    t.C = C;
    t.gs = h.fmt == I4MOE_FMT_GROUP ? h.gs : 0;
    t.ng = t.gs > 0 ? (C + t.gs - 1) / t.gs : 1;
    if (!all_finite(h.scales, (size_t)O * t.ng)) return I4MOE_EINVAL;
    try {
      t.packed.assign(h.packed, h.packed + (size_t)O * (C / 2));
      t.scales.assign(h.scales, h.scales + (size_t)O * t.ng);
    } catch (const std::bad_alloc &) {
      return I4MOE_ENOMEM;
    }
    return I4MOE_OK;
  };
  auto same = [](const i4moe_host_tensor &a, const i4moe_host_tensor &b) {
    return a.fmt == b.fmt && a.gs == b.gs && a.O == b.O && a.C == b.C && a.packed == b.packed && a.scales == b.scales;
  };
  for (int r = 0; r < n_rows; ++r) {
    if (token[r] < 0 || token[r] >= S || !std::isfinite(weight[r])) return I4MOE_EINVAL;
    // rows that name the same three tensors are one expert: one copy, computed together
    int first = 0;
    while (first < r && !(same(gate[first], gate[r]) && same(up[first], up[r]) && same(down[first], down[r]))) ++first;
    if (first == r) {
      int rc;
      if ((rc = copy(gate[r], I, D, ex[r].gate)) || (rc = copy(up[r], I, D, ex[r].up)) ||
          (rc = copy(down[r], D, I, ex[r].down)))
        return rc;
    }
    rows.push_back(HostRow{token[r], &ex[first], weight[r]});
  }
  try {
    HostPool pool(threads);
    host_rows_forward(pool, rows, x, D, I, P);
  } catch (const std::exception &) {
    return I4MOE_ENOMEM;
  }
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_host_int_path(void) { return host_int_path_available() ? 1 : 0; }

int i4moe_set_host_expert(i4moe_ctx *c, int layer, int expert, const i4moe_host_tensor *gate,
                          const i4moe_host_tensor *up, const i4moe_host_tensor *down) try {
  if (!c) return I4MOE_EINVAL;
  if (layer < 0 || expert < 0 || expert >= kMaxE) return fail(c, I4MOE_EINVAL, "bad layer %d / expert %d", layer, expert);
  std::unique_ptr<HostExpert> he(new (std::nothrow) HostExpert());
  if (!he) return fail(c, I4MOE_ENOMEM, "host memory");
  int rc;
  if ((rc = host_tensor_copy(c, gate, "gate", he->gate)) || (rc = host_tensor_copy(c, up, "up", he->up)) ||
      (rc = host_tensor_copy(c, down, "down", he->down)))
    return rc;
  const int I = he->gate.O, D = he->gate.C;
  if (he->up.O != I || he->up.C != D || he->down.O != D || he->down.C != I)
    return fail(c, I4MOE_EINVAL, "host expert shapes: need gate I x D, up I x D, down D x I");
  Layer &L = c->layers[layer];
  if ((L.D && L.D != D) || (L.I && L.I != I) || (L.host_D && L.host_D != D) || (L.host_I && L.host_I != I))
    return fail(c, I4MOE_EINVAL, "layer %d: host expert D=%d I=%d differs from the layer's", layer, D, I);
  if (L.E && expert >= L.E) return fail(c, I4MOE_EINVAL, "expert %d >= router E=%d", expert, L.E);
  L.host_D = D;
  L.host_I = I;
  L.host[expert] = std::move(he);
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

static int tier_buffers(i4moe_ctx *c) {
  hipError_t e = hipSuccess;
  const size_t bytes = sizeof(float) * (size_t)kTokens * kMaxCols;
  if (!c->h_x && (e = hipHostMalloc(&c->h_x, bytes, hipHostMallocDefault)) != hipSuccess) {
    c->h_x = nullptr;
    return hip_fail(c, e, "hipHostMalloc(x)");
  }
  if (!c->h_P && (e = hipHostMalloc(reinterpret_cast<void **>(&c->h_P), bytes, hipHostMallocDefault)) != hipSuccess) {
    c->h_P = nullptr;
    return hip_fail(c, e, "hipHostMalloc(host rows)");
  }
  if (!c->ev_x && (e = hipEventCreateWithFlags(&c->ev_x, hipEventDisableTiming)) != hipSuccess) {
    c->ev_x = nullptr;
    return hip_fail(c, e, "hipEventCreate");
  }
  if (!c->ev_p && (e = hipEventCreateWithFlags(&c->ev_p, hipEventDisableTiming)) != hipSuccess) {
    c->ev_p = nullptr;
    return hip_fail(c, e, "hipEventCreate");
  }
  try {  // thread creation can throw
    if (!c->pool) c->pool.reset(new HostPool(c->host_threads));
    if (!c->helper) c->helper.reset(new HostHelper());
  } catch (const std::exception &) {
    return fail(c, I4MOE_ENOMEM, "host worker threads");
  }
  return I4MOE_OK;
}

int i4moe_tiered_issue(i4moe_ctx *c, int layer, const void *x_dev, int dtype, int S, const i4moe_route_host *routes,
                       i4moe_tier_times *times) try {
  if (!c) return I4MOE_EINVAL;
  using clk = std::chrono::steady_clock;
  const auto t_start = clk::now();
  int rc = gate_compute(c);
  if (rc) return rc;
  Layer *L = find_layer(c, layer);
  if (!L) return fail(c, I4MOE_EINVAL, "layer %d has no experts", layer);
  if (!x_dev || !routes) return fail(c, I4MOE_EINVAL, "x_dev and routes must be non-NULL");
  if (dtype != I4MOE_DTYPE_F32 && dtype != I4MOE_DTYPE_BF16) return fail(c, I4MOE_EINVAL, "bad dtype %d", dtype);
  if (S < 1 || S > kTokens) return fail(c, I4MOE_EINVAL, "S=%d outside 1..%d", S, kTokens);
  const int D = L->D ? L->D : L->host_D, I = L->I ? L->I : L->host_I;
  if (!D || !I) return fail(c, I4MOE_EINVAL, "layer %d has no experts", layer);

  // the rows of each tier, in route order (token-major, selection order)
  std::vector<int32_t> de, dt;
  std::vector<float> dw;
  std::vector<HostRow> hrows;
  for (int t = 0; t < S; ++t) {
    const i4moe_route_host &r = routes[t];
    if (r.n < 0 || r.n > kMaxK) return fail(c, I4MOE_EINVAL, "route %d: n=%d outside 0..%d", t, r.n, kMaxK);
    for (int k = 0; k < r.n; ++k) {
      const int e = r.idx[k];
      const float w = r.w[k];
      if (!std::isfinite(w)) return fail(c, I4MOE_EINVAL, "route %d: weight %d not finite", t, k);
      if (e >= 0 && e < (int)L->gate.size() && L->gate[e]) {
        de.push_back(e);
        dt.push_back(t);
        dw.push_back(w);
        continue;
      }
      auto it = L->host.find(e);
      if (it == L->host.end()) return fail(c, I4MOE_EINVAL, "route %d: expert %d is neither on the device nor on the host", t, e);
      hrows.push_back(HostRow{t, it->second.get(), w});
    }
  }
  const bool dev = !de.empty(), host = !hrows.empty();
  if ((int)de.size() > kRows) return fail(c, I4MOE_EINVAL, "%zu device rows exceed the %d-row cap", de.size(), kRows);
  if (c->nslots + (dev ? 1 : 0) + (host ? 1 : 0) > kSlots)
    return fail(c, I4MOE_EINVAL, "%d issues pending; take before issuing more", c->nslots);
  if (c->nslots > 0 && (c->slots[0].S != S || c->slots[0].D != D))
    return fail(c, I4MOE_EINVAL, "pending issues have S=%d D=%d; this issue has S=%d D=%d", c->slots[0].S,
                c->slots[0].D, S, D);
  if (host && reinterpret_cast<uintptr_t>(x_dev) % (dtype == I4MOE_DTYPE_F32 ? 4 : 2) != 0)
    return fail(c, I4MOE_EINVAL, "x_dev misaligned");
  ensure_device(c);
  if ((rc = ensure_rows_scratch(c, D, I))) return rc;
  if ((rc = ensure_layer_tables(c, *L))) return rc;
  if (host && (rc = tier_buffers(c))) return rc;
  if ((rc = flush_all(c))) return rc;

  // x to the host first, so the CPU can start while the device group's kernels run
  const size_t esz = dtype == I4MOE_DTYPE_F32 ? 4 : 2;
  hipError_t e = hipSuccess;
  if (host) {
    e = hipMemcpyAsync(c->h_x, x_dev, esz * S * D, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipEventRecord(c->ev_x, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "copy of x to the host");
  }
  // The host rows start on the helper thread as soon as x has landed, while this thread issues
  // the device group (its host-side work and launches overlap them too).
  hipError_t host_err = hipSuccess;
  bool host_oom = false;
  auto t_x = clk::now(), t_cpu = t_x;
  if (host) {
    // the previous tiered issue's upload of the host sum must have read it
    if (c->ev_p_recorded && (e = hipEventSynchronize(c->ev_p)) != hipSuccess) return hip_fail(c, e, "wait for upload");
    c->pool->warm();  // the workers poll while x is on its way
    c->helper->post([&, S, D, I] {
      host_err = hipEventSynchronize(c->ev_x);
      t_x = clk::now();
      if (host_err != hipSuccess) return;
      try {  // host allocations can throw; nothing may escape the helper thread
        std::vector<float> xf((size_t)S * D);
        if (dtype == I4MOE_DTYPE_F32) {
          std::memcpy(xf.data(), c->h_x, sizeof(float) * xf.size());
        } else {
          const uint16_t *xb = static_cast<const uint16_t *>(c->h_x);
          for (size_t i = 0; i < xf.size(); ++i) {
            const uint32_t u = (uint32_t)xb[i] << 16;
            std::memcpy(&xf[i], &u, 4);
          }
        }
        std::memset(c->h_P, 0, sizeof(float) * (size_t)S * D);
        host_rows_forward(*c->pool, hrows, xf.data(), D, I, c->h_P);
      } catch (const std::exception &) {
        host_oom = true;
      }
      t_cpu = clk::now();
    });
  }
  int issued = 0;
  if (dev) {
    i4moe_group g{(int32_t)de.size(), de.data(), dt.data(), dw.data()};
    const int s = issue_impl(c, layer, x_dev, dtype, S, &g, false);
    if (s < 0) {
      if (host) c->helper->wait();
      return s;
    }
    ++issued;
  }
  const auto t_issued = clk::now();
  if (host) {
    c->helper->wait();
    if (host_err != hipSuccess) {
      if (dev) c->poisoned = true;  // the device slot is issued but the host rows would be lost
      return hip_fail(c, host_err, "wait for x");
    }
    if (host_oom) {
      if (dev) c->poisoned = true;
      return fail(c, I4MOE_ENOMEM, "host rows: host memory");
    }
    // the host slot: one row per token, weight 1, holding the token's sum of host rows
    const int s = c->nslots;
    GroupDev hg;
    std::memset(&hg, 0, sizeof hg);
    hg.n_entries = 1;
    hg.entry_expert[0] = 0;
    hg.entry_row0[0] = 0;
    hg.entry_row0[1] = S;
    for (int t = 0; t < S; ++t) {
      hg.row_token[t] = t;
      hg.row_expert[t] = 0;
      hg.row_weight[t] = 1.f;
      hg.tok_row0[t] = t;
      hg.red_rows[t] = t;
    }
    hg.tok_row0[S] = S;
    hg.n_rows = S;
    hg.S = S;
    GroupBuf *gb = c->d_slot_bufs + s;
    e = launch_group_store(hg, L->d_tab, gb, c->stream);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(c->d_y + (size_t)s * kRows * c->y_ld, sizeof(float) * c->y_ld, c->h_P, sizeof(float) * D,
                           sizeof(float) * D, S, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipEventRecord(c->ev_p, c->stream);
    if (e != hipSuccess) {
      c->poisoned = true;  // the device slot is issued but the host rows would be lost
      return hip_fail(c, e, "upload of the host rows");
    }
    c->ev_p_recorded = true;
    SlotInfo &si = c->slots[s];
    si = SlotInfo{};
    si.S = S;
    si.D = D;
    si.rows = S;
    si.grp = gb;
    si.ring = -1;
    c->nslots = s + 1;
    ++issued;
  }
  c->calls++;
  if (times) {
    auto ms = [](clk::time_point a, clk::time_point b) { return std::chrono::duration<double, std::milli>(b - a).count(); };
    const auto t_end = clk::now();
    times->issue_ms = ms(t_start, t_issued);
    times->x_wait_ms = host ? ms(t_start, t_x) : 0.0;
    times->cpu_ms = host ? ms(t_x, t_cpu) : 0.0;
    times->total_ms = ms(t_start, t_end);
    times->device_rows = (int32_t)de.size();
    times->host_rows = (int32_t)hrows.size();
  }
  return issued;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_read_probe(i4moe_ctx *c, int layer, int tensor_mask, int n_experts, const int32_t *experts) try {
  if (!c) return I4MOE_EINVAL;
  Layer *L = find_layer(c, layer);
  if (!L || !L->D || !L->I || !L->d_tab) return fail(c, I4MOE_EINVAL, "layer %d has no experts", layer);
  if (tensor_mask < 1 || tensor_mask > 7) return fail(c, I4MOE_EINVAL, "tensor_mask %d outside 1..7", tensor_mask);
  if (n_experts < 1 || n_experts > kRows || !experts)
    return fail(c, I4MOE_EINVAL, "read probe needs 1..%d experts and a non-NULL list", kRows);
  ProbeArgs a{};
  for (int i = 0; i < n_experts; ++i) {
    const int e = experts[i];
    if (e < 0 || e >= (int)L->gate.size() || !L->gate[e])
      return fail(c, I4MOE_EINVAL, "read probe: expert %d is not set", e);
    a.experts[i] = (int16_t)e;
  }
  ensure_device(c);
  if (!c->d_sink) {
    const hipError_t e = dalloc(&c->d_sink, 64 * sizeof(uint32_t));
    if (e != hipSuccess) return hip_fail(c, e, "hipMalloc(read probe sink)");
  }
  // tiles of about one wave pass of nibbles: 16 loads of 16 bytes per lane
  constexpr int kProbePassBytes = 16 * 16 * kWave;
  a.tab = L->d_tab;
  a.sink = c->d_sink;
  a.n_experts = n_experts;
  int per_e = 0;
  for (int n = 0; n < 3; ++n)
    if (tensor_mask & (1 << n)) {
      const int O = n < 2 ? L->I : L->D, C = n < 2 ? L->D : L->I;
      const int row_bytes = (C / 2 + 15) / 16 * 16;
      const int tr = std::max(1, std::min(64, kProbePassBytes / row_bytes));
      a.tensors[a.n_tensors] = n;
      a.tile_rows[a.n_tensors] = tr;
      a.tiles[a.n_tensors] = (O + tr - 1) / tr;
      per_e += a.tiles[a.n_tensors++];
    }
  a.waves = n_experts * per_e;
  const hipError_t e = timed(c, I4MOE_K_PROBE, [&](hipEvent_t t0, hipEvent_t t1) {
    return launch_read_probe(a, c->stream, t0, t1);
  });
  return e != hipSuccess ? hip_fail(c, e, "read probe launch") : I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_set_profiling(i4moe_ctx *c, int on) try {
  if (!c) return I4MOE_EINVAL;
  ensure_device(c);
  (void)hipStreamSynchronize(c->stream);
  drain_profile(c);
  for (int k = 0; k < I4MOE_K_COUNT; ++k) {
    c->prof_ms[k] = 0;
    c->prof_n[k] = 0;
  }
  c->profiling = on != 0;
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

int i4moe_profile_query(i4moe_ctx *c, int kernel, double *total_ms, long long *launches) try {
  if (!c || kernel < 0 || kernel >= I4MOE_K_COUNT) return I4MOE_EINVAL;
  ensure_device(c);
  drain_profile(c);
  if (total_ms) *total_ms = c->prof_ms[kernel];
  if (launches) *launches = c->prof_n[kernel];
  return I4MOE_OK;
} catch (...) {  // nothing thrown (host allocation, thread start) crosses the C ABI
  return I4MOE_ENOMEM;
}

}  // extern "C"
