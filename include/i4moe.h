/*
 * i4moe -- decode-time int4 grouped MoE expert path for AMD Instinct MI355X (gfx950).
 *
 * One MoE layer at decode is three calls on one HIP stream:
 *
 *   i4moe_route                  device router: E x D logits GEMV, sigmoid, bias-augmented
 *                                top-K with strict tie-break, top-p, norm_topk, routed_scale,
 *                                and the expert group (which experts run on which token rows)
 *   i4moe_expert_group_issue     grouped W4A16 experts over that group: dual gate/up
 *                                projection with the SiLU-gated product fused in, then the
 *                                down projection into a per-issue slot
 *   i4moe_expert_group_take      per token, the per-expert weighted sum in route order, the
 *                                slots in issue order, added into the residual; no atomics
 *
 * Sources (web pages on the colibri int4 MoE engine):
 *   [LOG-g4]  "Commit history of c/backend_cuda.cu", commit opening "The grouped MoE kernels
 *             were per-row-only": fmt=4 group-wise int4, gs, O*ceil(C/gs) scales, gs even,
 *             gs=0 per-row, fmt=2 and fmt=4 members in one launch, reject unknown formats,
 *             upload_g carrying gs, handle 0 = not uploaded.
 *   [LOG-tc]  same page, commit gating the TC_W4A16 branch: the grouped 3-launch decode path
 *             (dual gate/up, silu, down).
 *   [LOG-rt]  same page, commit "First increment of the #431 plan": the device router and its
 *             packed route result (~68 B at K=8).
 *   [LOG-fix] same page, "Three vendor-neutral fixes": cached tensors usable with stale host
 *             pointers, sticky device errors consumed, a fail-after-N fault hook on compute
 *             entry points only.
 *   [PR342]   "cuda: COLI_GROUP_ASYNC=1 - overlap the CPU expert rows with the GPU groups at
 *             decode", section "What": issue/take split, S<=4 small-batch groups.
 *   [PR434]   "cuda: COLI_CUDA_RESID=1 - expert-group results stay on device", section "What":
 *             per-expert weighting and fixed-order reduce, per-issue slots reserved at the
 *             64-expert cap, take in issue order without atomics, failed take is fatal.
 *
 * Conventions for every call
 *   - Return value: I4MOE_OK (0) or a negative I4MOE_E* code; i4moe_last_error() gives the
 *     message of the most recent failure on that context.  A failed call enqueues nothing
 *     unless stated otherwise, and no device error is left pending for a later call.
 *   - Device pointers ("_dev") are plain HIP device addresses (e.g. torch tensor data_ptr()).
 *     Host pointers are read during the call only; the caller may free or overwrite them as
 *     soon as the call returns.
 *   - A NULL context is refused before any HIP call: I4MOE_EINVAL, or 0 from the calls that
 *     return a handle or a size (i4moe_ctx_destroy(NULL) is a no-op).
 *   - A context is bound to one device and one stream and is not thread-safe.
 *   - Compute calls (route, issue, take) only enqueue work; they never synchronise the host
 *     unless a host output is requested.
 */
#ifndef I4MOE_H
#define I4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Limits. */
#define I4MOE_MAX_ROWS   64    /* expert-token rows in one issue: the 64-expert cap [PR434] */
#define I4MOE_MAX_TOKENS 64    /* tokens S per call */
#define I4MOE_MAX_K      64    /* top-K */
#define I4MOE_MAX_E      1024  /* routed experts per layer */
#define I4MOE_MAX_COLS   8192  /* columns C of an int4 tensor (D for gate/up, I for down) */
#define I4MOE_MAX_SLOTS  16    /* issues pending before a take */

/* Weight formats: the pages' own codes [LOG-g4]. */
enum { I4MOE_FMT_ROW = 2, I4MOE_FMT_GROUP = 4 };

/* Activation dtypes. */
enum { I4MOE_DTYPE_F32 = 0, I4MOE_DTYPE_BF16 = 1 };

/* Status codes.  No C++ exception leaves a function of this interface: a host allocation or a
 * worker thread that cannot be had returns I4MOE_ENOMEM (0 from the functions that return a
 * handle or a size). */
enum {
  I4MOE_OK = 0,
  I4MOE_EINVAL = -1,       /* bad argument, shape, handle or state                      */
  I4MOE_ENOMEM = -2,       /* device or host allocation failed                            */
  I4MOE_EDEVICE = -3,      /* a HIP call or kernel launch failed                          */
  I4MOE_EUNSUPPORTED = -4, /* well-formed request outside what the kernels decode       */
  I4MOE_EINJECTED = -5,    /* failure injected by the fail-after hook                     */
  I4MOE_EPOISONED = -6     /* an earlier take failed; compute calls refuse until destroy */
};

typedef struct i4moe_ctx i4moe_ctx;
typedef uint32_t i4moe_tensor;  /* 0 = invalid / not uploaded [LOG-g4] */

/* Per-token route result, host side.  n = experts kept after top-p; idx[0..K) are the K
 * selections in selection order; w[0..n) the final float32 weights, w[n..K) = 0.
 * On the device the same record is the packed route [LOG-rt]. */
typedef struct {
  int32_t n;
  int32_t idx[I4MOE_MAX_K];
  float w[I4MOE_MAX_K];
} i4moe_route_host;

/* Explicit group for issue (host arrays of n_rows entries): each row runs expert[r] on token
 * row token[r] of x and is weighted by weight[r].  Per token, rows are summed in the order
 * listed.  An expert with at least 8 rows in the group runs on the matrix cores
 * (I4MOE_MFMA_MIN_ROWS at i4moe_ctx_create), the others on the vector kernels, one row per
 * workgroup (or up to 4 rows per weight pass with I4MOE_ENTRY_ROWS). */
typedef struct {
  int32_t n_rows;
  const int32_t *expert;
  const int32_t *token;
  const float *weight;
} i4moe_group;

/* ---- context ---------------------------------------------------------------------------- */

/* Create a context on HIP device `device`, bound to the null stream.  The fault hook starts
 * from the environment variable I4MOE_FAIL_AFTER when it holds a non-negative integer.
 * I4MOE_WAVE_FACTOR (0.05 .. 64, default 1) scales the number of waves the projections aim
 * for per CU; it changes how output rows are tiled over waves, never the results (each row
 * is still reduced by one wave in a fixed order).
 * I4MOE_ENTRY_ROWS (2..4; unset or 0: one row per workgroup) lets up to that many rows of one
 * expert (S > 1) share each pass over its weights in the vector kernels.  Off by default: it
 * measured slower than one row per workgroup at every row count (rows of one expert running
 * together re-read its weights mostly from cache).  It changes only the order of additions: a
 * group-wise tensor's results are the same bits either way, a per-row tensor's may differ in the
 * last bits (both within the documented tolerance of the f64 result).
 * I4MOE_MFMA_MIN_ROWS (0 = off, else 2 .. 64; default 8, the crossover measured on MI355X; the
 * pages report ~16 on their GPU) is the row count from which an expert's rows in one issue run on
 * the matrix cores (int8 products of digit rows, exact like the vector kernels; gate/up/down of
 * every expert of the issue per-row or with group sizes that are multiples of 64); smaller
 * entries keep the vector kernels.
 * Errors: EINVAL (bad device, out == NULL), EDEVICE, ENOMEM. */
int i4moe_ctx_create(int device, i4moe_ctx **out);

/* Synchronise the stream and free everything the context owns.  NULL is a no-op. */
int i4moe_ctx_destroy(i4moe_ctx *ctx);

/* Bind the stream later compute calls enqueue on (a hipStream_t; NULL = null stream). */
int i4moe_set_stream(i4moe_ctx *ctx, void *hip_stream);

/* Message of the most recent failure on ctx (static text if ctx is NULL).  Never NULL. */
const char *i4moe_last_error(const i4moe_ctx *ctx);

/* ---- weights ---------------------------------------------------------------------------- */

/* Upload one int4 tensor of O rows x C columns [LOG-g4].
 *   fmt    I4MOE_FMT_ROW (gs must be 0) or I4MOE_FMT_GROUP (gs even, >= 0; gs = 0 is per-row)
 *   packed O * C/2 bytes, row-major; byte c/2 of a row holds column c in its low nibble when
 *          c is even, in its high nibble when c is odd; nibble q encodes the integer q - 8
 *   scales float32: O of them (per-row) or O * ceil(C/gs) row-major [o][group] (group-wise);
 *          the last group of a row may be narrower than gs and has its own scale
 * C must be even and <= I4MOE_MAX_COLS; O >= 1.  Synchronous: the data is on the device when
 * the call returns and the host buffers may then be freed or reused.
 * Returns a handle > 0, or 0 on failure (EINVAL / EUNSUPPORTED / ENOMEM / EDEVICE in
 * i4moe_last_error); a failed upload leaves nothing allocated. */
i4moe_tensor i4moe_upload_expert_tensor(i4moe_ctx *ctx, int fmt, int gs, int O, int C,
                                        const uint8_t *packed, const float *scales);

/* Release a tensor.  Synchronises the stream first.  Experts still bound to it become unset. */
int i4moe_tensor_free(i4moe_ctx *ctx, i4moe_tensor t);

/* Bind expert `expert` of layer `layer` to three uploaded tensors: gate and up are I x D,
 * down is D x I, with D and I equal across the layer (and D equal to the router's D when one
 * is uploaded).  Formats may differ between experts and between the three tensors. */
int i4moe_set_expert(i4moe_ctx *ctx, int layer, int expert, i4moe_tensor gate, i4moe_tensor up,
                     i4moe_tensor down);

/* Upload the router of `layer`: W is E x D float32 row-major, bias E float32 (NULL = zeros)
 * [LOG-rt].  Values must be finite.  E <= I4MOE_MAX_E.  Synchronous. */
int i4moe_upload_router(i4moe_ctx *ctx, int layer, int E, int D, const float *W, const float *bias);

/* ---- compute ---------------------------------------------------------------------------- */

/* Route S tokens of x_dev ([S][D], dtype F32 or BF16, row-major, device) with the router of
 * `layer` [LOG-rt]:
 *   l = W x (f64 accumulation of exact products), sigma = 1/(1+exp(-l)), score = sigma + bias,
 *   K rounds of "first strictly greater" over ascending expert index, weights sigma of the
 *   chosen, top-p over the K in selection order (active when 0 < topp < 1), then division by
 *   their sum when norm_topk != 0, then times routed_scale, rounded once to float32.
 * The route and the expert group (distinct experts in first-appearance order, token-major)
 * stay in the layer's device route buffer for i4moe_expert_group_issue.  If host_out != NULL
 * it receives S records and the call synchronises the stream (one small copy back).
 * With S == 1, E <= 64 and host_out == NULL only the logits GEMV is enqueued here; the
 * selection runs inside the dual projection of the issue that consumes this route, or as its
 * own kernel on the context's stream when another call needs the route or the router scratch
 * first (a route, a tap, a stream switch, a change of the layer's experts or router).  The
 * results are bitwise the same either way.
 * Limits: 1 <= S <= I4MOE_MAX_TOKENS, 1 <= K <= min(E, I4MOE_MAX_K), S*K <= I4MOE_MAX_ROWS.
 * Fault-hook gated.  Non-finite activations give an unspecified (but in-range) route. */
int i4moe_route(i4moe_ctx *ctx, int layer, const void *x_dev, int dtype, int S, int K, float topp,
                int norm_topk, float routed_scale, i4moe_route_host *host_out);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the route of i4moe_route, by the same kernels with the
 * same bits, with every byte of its working memory (scores, logits, the selection's group
 * buffer) in a static device array of I4MOE_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends.  Its address is looked up once per device when a context is created there; this call
 * allocates nothing, also on its first use.
 *   route_dev  device memory for S records (i4moe_route_host layout), written on the stream;
 *              the layer's own device route (the one i4moe_expert_group_issue consumes) is left
 *              as it was, and the host is not synchronised.
 * Limits are those of the scratch: S <= I4MOE_MAX_TOKENS, E <= I4MOE_MAX_E, S*K <= I4MOE_MAX_ROWS
 * (I4MOE_EUNSUPPORTED beyond them, with nothing enqueued); other errors as i4moe_route.
 * Every context on a GPU shares that GPU's scratch: calls whose kernels overlap on one GPU (on
 * two streams) race and must be ordered by the caller; calls on one stream are ordered already.
 * Fault-hook gated; no profiling events are recorded for it. */
#define I4MOE_NOALLOC_SCRATCH_BYTES (1048576 + 524288 + 43264)
int i4moe_route_noalloc(i4moe_ctx *ctx, int layer, const void *x_dev, int dtype, int S, int K, float topp,
                        int norm_topk, float routed_scale, i4moe_route_host *route_dev);

/* Run the experts of one group over x_dev ([S][D], F32 or BF16) and keep the per-row outputs
 * in the next free slot.  group == NULL consumes the device group of `layer` written by the
 * latest i4moe_route of that layer (no host round trip); the route of that layer must not be
 * recomputed before this issue has executed on the stream.  Otherwise the explicit group is
 * used (rows <= I4MOE_MAX_ROWS, experts set, tokens < S).  Every expert the group may name
 * must be set; with group == NULL that is every expert 0..E-1 of the layer.
 * Returns the slot index (>= 0) or a negative code with nothing enqueued, so the caller can
 * fall back to another path [PR342].  x_dev must stay valid until the issue has executed.
 * A lone one-token issue of a device route (no other slot pending, at most 8 rows, I <= 2048)
 * enqueues only the dual projection: the take then runs the down projection and the
 * reduction in one kernel.  A y tap, another issue, a stream switch or a change of the
 * layer's experts runs the down projection on its own first; the results are bitwise the same.
 * The first issue whose entries reach the matrix cores (I4MOE_MFMA_MIN_ROWS) allocates their
 * scratch (digit rows, column-slice partial sums; the latter grows for larger shapes), which
 * synchronises the stream: under graph capture, run one issue of the same shape eagerly first.
 * Fault-hook gated. */
int i4moe_expert_group_issue(i4moe_ctx *ctx, int layer, const void *x_dev, int dtype, int S,
                             const i4moe_group *group);

/* For every token t < S and column i < D of the issued slots:
 *   residual_dev[t][i] += sum over slots in issue order of
 *                         (sum over the slot's rows of token t, in route order, of w * y)
 * in float32 with a fixed order and no atomics [PR434], then frees all slots.  residual_dev is
 * [S][D] float32 on the device, updated in place on the stream.  All pending slots must have
 * been issued for the same D and with S equal to this S.  With no slot pending it is a no-op.
 * On failure (including an injected one) the context is poisoned: routed experts would be
 * dropped silently, so every later compute call returns I4MOE_EPOISONED [PR434]. */
int i4moe_expert_group_take(i4moe_ctx *ctx, float *residual_dev, int S);

/* ---- the steps around the routed experts --------------------------------------------------- */
/* Sources, same page ("Commit history of c/backend_cuda.cu"):
 *   [LOG-pipe] the "GPU resident pipeline" commit: device primitives rmsnorm over strided rows,
 *              silu-mul, residual add and a fixed-order row merge without atomics, checked
 *              against the engine's CPU math.
 *   [LOG-mla]  the "CUDA batch MLA attention, ..., W4A16 kernels" commit: W4A16 kernels for the
 *              shared expert beside the per-device expert groups. */

/* Bind the shared expert of `layer` (gate and up I x D, down D x I, as i4moe_set_expert) [LOG-mla].
 * It runs on every token with weight 1; it is not part of the router's E experts. */
int i4moe_set_shared_expert(i4moe_ctx *ctx, int layer, i4moe_tensor gate, i4moe_tensor up, i4moe_tensor down);

/* Upload the rmsnorm weights of `layer`: gamma is D float32 (finite), eps >= 0.  Synchronous. */
int i4moe_upload_norm(i4moe_ctx *ctx, int layer, int D, const float *gamma, float eps);

/* rmsnorm of S rows of x_dev (float32, row stride ld_x >= D) into out_dev (row stride ld_out >= D,
 * out_dtype F32 or BF16) [LOG-pipe]:
 *   out[t][i] = round( x[t][i] / sqrt(sum_i x[t][i]^2 / D + eps) * gamma[i] )
 * in f64 (exact squares, a fixed summation order), rounded once from the f64 value to the output
 * dtype (round to nearest, ties to even; bf16 directly, not through a float32 rounding).
 * Limits: 1 <= S <= I4MOE_MAX_TOKENS.  Fault-hook gated. */
int i4moe_rmsnorm(i4moe_ctx *ctx, int layer, const float *x_dev, int ld_x, int S, void *out_dev, int ld_out,
                  int out_dtype);

/* Issue the layer's shared expert over the S rows of x_dev ([S][D], F32 or BF16): one group row per
 * token, weight 1, into the next free slot, reduced by the next take after the slots issued before
 * it [LOG-mla].  Returns the slot index, or a negative code with nothing enqueued.  Fault-hook gated. */
int i4moe_shared_expert_issue(i4moe_ctx *ctx, int layer, const void *x_dev, int dtype, int S);

/* One whole MoE block on the residual stream, on the device, in one call: for the S float32 rows
 * of residual_dev ([S][D], 16-byte aligned, updated in place),
 *   a   = i4moe_rmsnorm of the rows into act_dtype (context scratch)
 *   route a (as i4moe_route with K, topp, norm_topk, routed_scale), issue the routed experts and,
 *   if one is bound, the shared expert, and take:
 *   residual[t] += (sum over the routed rows of t, route order, of w * y) + y_shared
 * The shared expert runs as one more row per token of the routed group (weight 1, after the routed
 * rows) when S * (K + 1) <= I4MOE_MAX_ROWS, in the same launches and the same take slot, else as
 * its own issue after the routed one: the same bits either way.  Needs the layer's router, norm weights and
 * every routed expert.  Fault-hook gated as one compute call.  A failure after the first launch
 * poisons the context, as a failed take does.  The first call on a context allocates its scratch
 * for the normalised rows; later calls with the same or a smaller D allocate nothing. */
int i4moe_moe_block(i4moe_ctx *ctx, int layer, float *residual_dev, int S, int act_dtype, int K, float topp,
                    int norm_topk, float routed_scale);

/* ---- test hooks ----------------------------------------------------------------------------- */

/* Fault hook [LOG-fix]: after n more successful compute calls (route, issue, take), every
 * compute call fails with I4MOE_EINJECTED without enqueuing anything; n < 0 disables it.
 * Uploads, binds and queries are never gated. */
int i4moe_set_fail_after(i4moe_ctx *ctx, long long n);

/* Debug taps for tests; each synchronises the stream and copies to host_dst (bytes must
 * equal the size stated).
 *   I4MOE_TAP_LOGITS  index ignored: f64 [S][E] logits of the latest route
 *   I4MOE_TAP_ROUTE   index = layer: i4moe_route_host [S] of that layer's latest route
 *   I4MOE_TAP_GROUP   index = layer: int32 [I4MOE_GROUP_WORDS] device group record of the layer
 *                     (layout below)
 *   I4MOE_TAP_H       index ignored: f32 [rows][I] SiLU-gated products of the latest issue
 *   I4MOE_TAP_Y       index = slot: f32 [rows][D] down-projection rows of that pending slot */
enum { I4MOE_TAP_LOGITS = 1, I4MOE_TAP_ROUTE = 2, I4MOE_TAP_GROUP = 3, I4MOE_TAP_H = 4, I4MOE_TAP_Y = 5 };
int i4moe_debug_read(i4moe_ctx *ctx, int what, int index, void *host_dst, size_t bytes);

/* Size in bytes a tap needs for the given layer/slot right now (0 if unavailable). */
size_t i4moe_debug_size(i4moe_ctx *ctx, int what, int index);

/* Group record layout (int32 words; row_weight holds float32 bit patterns):
 *   [0] n_entries  [1] n_rows  [2] S  [3] reserved
 *   entry_expert[64], entry_row0[65], row_token[64], row_expert[64], row_weight[64],
 *   tok_row0[65], red_rows[64]
 * Rows of entry j are entry_row0[j] .. entry_row0[j+1]-1 (an expert's rows are its tokens in
 * ascending order); rows of token t in reduce order (route order) are
 * red_rows[tok_row0[t] .. tok_row0[t+1]-1]. */
#define I4MOE_GROUP_WORDS (4 + 64 + 65 + 64 + 64 + 64 + 65 + 64)

/* ---- the CPU tier [PR342] ------------------------------------------------------------------ */

/* One int4 tensor in host memory, in the layout of i4moe_upload_expert_tensor. */
typedef struct {
  int32_t fmt, gs, O, C;
  const uint8_t *packed;
  const float *scales;
} i4moe_host_tensor;

/* Keep expert `expert` of `layer` on the host (gate and up I x D, down D x I, formats and layout
 * as i4moe_upload_expert_tensor; D and I equal to the layer's device experts' when there are
 * any).  The library copies the three tensors into host memory it owns, so the buffers may be
 * freed when the call returns.  A host expert is computed on the CPU by i4moe_tiered_issue; an
 * expert also bound on the device (i4moe_set_expert) runs on the device. */
int i4moe_set_host_expert(i4moe_ctx *ctx, int layer, int expert, const i4moe_host_tensor *gate,
                          const i4moe_host_tensor *up, const i4moe_host_tensor *down);

/* Host wall-clock split of one tiered issue, in milliseconds (cf. the overlap window of [PR342]),
 * each from the start of the call: until the device group is enqueued (issue_ms), until x has
 * reached the host (x_wait_ms); then the CPU rows themselves (cpu_ms) and the whole call. */
typedef struct {
  double issue_ms, x_wait_ms, cpu_ms, total_ms;
  int32_t device_rows, host_rows;
} i4moe_tier_times;

/* The experts of a host route (S records, e.g. from i4moe_route with host_out) split by tier
 * [PR342]: the rows (t, k < n_t) whose expert is bound on the device run as one explicit group on
 * the GPU (a slot, as i4moe_expert_group_issue); the rows whose expert is kept on the host are
 * computed on the CPU while that group runs, and their weighted sum per token (rows in route
 * order, float32) goes to the next slot as one row per token with weight 1.  A weight row's dot
 * product on the CPU: on a host with AVX-512 VNNI, when every host tensor is per-row or has a
 * group size that is a multiple of 64 (see i4moe_host_int_path), the activation row (x, or a row
 * of the gated product h) is taken in 24-bit fixed point with a power-of-two exponent of its own
 * and each group's sum is an exact integer, scaled in float32 lanes (gs 64) or in double
 * (other group sizes, per-row); otherwise each group's products are summed in float32, then
 * scaled.  SiLU and the gated product are float32 either way.  i4moe_expert_group_take then
 * joins both slots in issue order (the device slot first), so the sum order is fixed and the
 * result bitwise reproducible [PR434].
 * x_dev ([S][D], F32 or BF16) is copied to the host on the stream before the device group's
 * kernels are enqueued; the CPU rows start on a helper thread of the context when that copy has
 * landed, while the calling thread enqueues the device group, and the call returns when the CPU
 * rows are done and their sum is enqueued for upload (the device group may still be running).
 * Uses up to 2 slots; returns the number of slots issued (0 when no token has an expert), or a
 * negative code.  Every expert the routes name must be bound on the device or kept on the host.
 * On failure nothing is left pending except possibly the copy of x.  times may be NULL.
 * Host threads: I4MOE_HOST_THREADS at context creation (1..256; default the host's cores but
 * one, at most 16).  Fault-hook gated (one compute call). */
int i4moe_tiered_issue(i4moe_ctx *ctx, int layer, const void *x_dev, int dtype, int S,
                       const i4moe_route_host *routes, i4moe_tier_times *times);

/* The CPU tier's arithmetic alone (host only, no device and no context; what i4moe_tiered_issue
 * runs for its host rows) [PR342]: for r < n_rows, in order,
 *   P[token[r]][d] += weight[r] * (down[r] . (silu(gate[r] . x_t) * (up[r] . x_t)))[d]
 * with x: S x D float32 rows and P: S x D float32 (accumulated into), gate/up/down[r] host tensors
 * (I x D, I x D, D x I, layouts as i4moe_upload_expert_tensor), with the arithmetic described at
 * i4moe_tiered_issue.  threads >= 1 workers (the results do not depend on the count).  Rows
 * whose three descriptors are equal (same pointers, format and shape) are one expert: its tensors
 * are copied once and, on the integer path, each weight row is read once for all of them, as for
 * an expert that several tokens of a tiered issue route to (the results are the same bits as
 * row by row).
 * Non-finite values in x give unspecified outputs.
 * Errors: EINVAL (bad shapes, tokens, NULL pointers, non-finite scales or weights), ENOMEM. */
int i4moe_host_rows(int S, int D, int I, int n_rows, const int32_t *token, const float *weight,
                    const i4moe_host_tensor *gate, const i4moe_host_tensor *up, const i4moe_host_tensor *down,
                    const float *x, float *P, int threads);

/* 1 when the CPU tier's dot products take the integer path on this host (AVX-512 F, BW, VL and
 * VNNI present and I4MOE_HOST_INT is not "0" in the environment), else 0.  The integer path
 * handles two 64-column blocks per 512-bit instruction where the groups allow (per-row, gs 64,
 * gs a multiple of 128; I4MOE_HOST_INT=256 keeps it at 256 bits); both widths give the same
 * bits.  Tensors whose group size is not a multiple of 64 take the float32 path on any host.
 * The environment is read at every call, here and in the CPU tier. */
int i4moe_host_int_path(void);

/* ---- profiling ---------------------------------------------------------------------------- */

/* Kernel families timed when profiling is on.  A selection run inside the dual projection
 * (see i4moe_route) is timed as part of I4MOE_K_DUAL, a down projection run inside the take
 * (see i4moe_expert_group_issue) as part of I4MOE_K_TAKE.  I4MOE_K_MFMA: the matrix-core
 * projections of experts with many rows, with the digit rows they read. */
enum {
  I4MOE_K_ROUTE = 0, I4MOE_K_DUAL = 1, I4MOE_K_DOWN = 2, I4MOE_K_TAKE = 3, I4MOE_K_MFMA = 4, I4MOE_K_PROBE = 5,
  I4MOE_K_COUNT = 6
};

/* on != 0: bracket every later kernel launch with a pair of HIP events on the context's
 * stream; on == 0 stops.  Switching resets the accumulated figures. */
int i4moe_set_profiling(i4moe_ctx *ctx, int on);

/* Synchronise, then report the total device milliseconds and launch count accumulated for one
 * kernel family since profiling was switched on. */
int i4moe_profile_query(i4moe_ctx *ctx, int kernel, double *total_ms, long long *launches);

/* A measuring aid: the plain-read rate of the expert weights, against which the projections'
 * bandwidth is reported (expert-weight bytes per second, the figure the pages' grouped kernels
 * are measured by [LOG-tc, PR651]).  One launch on the context's stream that reads every nibble
 * and scale byte of the listed experts' tensors of the layer (tensor_mask bit 0 gate, 1 up,
 * 2 down; n_experts 1..I4MOE_MAX_ROWS indices into the layer's table, each bound on the device)
 * and computes nothing: one wave per tile of a tensor's rows (about 16 KB of nibbles), read
 * as one contiguous block of nibbles and one of scales with sixteen 16-byte loads per lane in
 * flight; it writes nothing the caller reads.  Timed as I4MOE_K_PROBE when profiling is on.
 * Errors: EINVAL (bad layer, mask, list or expert), ENOMEM (its 256-byte scratch, allocated on
 * the first call). */
int i4moe_read_probe(i4moe_ctx *ctx, int layer, int tensor_mask, int n_experts, const int32_t *experts);

#ifdef __cplusplus
}
#endif
#endif /* I4MOE_H */
