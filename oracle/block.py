"""The steps around the routed experts of one MoE block, in f64.  TEST INFRASTRUCTURE.

Sources: the "GPU resident pipeline" commit of "Commit history of c/backend_cuda.cu" lists the
device primitives of the layer's data plane (rmsnorm over strided rows, silu-mul, residual add,
a fixed-order row merge without atomics); the "CUDA batch MLA attention, ..., W4A16 kernels"
commit of the same page runs the shared expert as a W4A16 MLP beside the routed expert groups.

For token t of the residual stream r (float32 [S, D]):

    n_t   = r_t / sqrt(mean_i r_t[i]^2 + eps) * gamma       rmsnorm                 [LOG-pipe]
    a_t   = round(n_t) to the expert input dtype              (bf16 or f32)
    out_t = r_t + sum_{k < n} w_k * y_k(a_t) + y_shared(a_t)  routed experts, shared expert, residual add

Readings (the pages name these steps but give no formula):
* rmsnorm is the usual root-mean-square normalisation: the mean of the squares over the D
  columns, eps added inside the square root, then the per-column weight gamma;
* the normalised row is rounded once, directly from its exact value, to the dtype the experts
  read (round to nearest, ties to even) -- no intermediate float32 rounding for bf16;
* the shared expert is one more gate/up/down expert, run on every token with weight 1 (it has no
  routing weight), and its output joins the routed sum and the residual.
"""

from __future__ import annotations

import math

import numpy as np

from . import experts, router


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """f64 [S, D]: each row divided by the square root of (its mean square + eps), times gamma.
    The sum of squares is correctly rounded (math.fsum); eps and gamma are float32 values."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    e = float(np.float32(eps))
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        ms = math.fsum(float(v) * float(v) for v in x[t]) / x.shape[1]
        out[t] = x[t] / math.sqrt(ms + e) * g
    return out


def round_bf16(v: float) -> float:
    """v rounded to the nearest bfloat16 value (8 significant bits, exponent range of float32),
    ties to even, as a float.  Written from the definition: the spacing of bf16 values around v
    is 2^(e-8) for v in [2^(e-1), 2^e), and never finer than the subnormal spacing 2^-133."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)                 # v = m * 2^e, 0.5 <= |m| < 1
    q = max(e - 8, -133)                 # exponent of the last kept bit
    scaled = math.ldexp(v, -q)           # exact: a power-of-two scaling
    r = math.ldexp(float(round(scaled)), q)  # round() on floats is round-half-even
    if abs(r) >= 2.0 ** 128:             # rounded past the largest finite bf16
        return math.copysign(math.inf, v)
    return r


def bf16_bits(v: float) -> int:
    """The 16-bit pattern of a value that is already a bfloat16 (the top half of its float32)."""
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0]) >> 16


def round_activations(n: np.ndarray, dtype: str):
    """The expert input: float32 (numpy's correctly rounded conversion) or the bf16 bit patterns."""
    if dtype == "f32":
        return np.asarray(n, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        flat = [bf16_bits(round_bf16(float(v))) for v in np.asarray(n, dtype=np.float64).ravel()]
        return np.array(flat, dtype=np.uint16).reshape(np.shape(n))
    raise ValueError(dtype)


def moe_block(residual, gamma, eps: float, act_dtype: str, W, bias, expert_of, K: int, topp: float,
              norm_topk: bool, routed_scale: float, shared=None):
    """The whole block on the residual rows.  Returns (a, routes, delta, out): the rounded expert
    input, the routes, the f64 sum of the routed and shared outputs, and residual + delta."""
    r = np.atleast_2d(np.asarray(residual, dtype=np.float32))
    a = round_activations(rmsnorm(r, gamma, eps), act_dtype)
    a64 = router.widen_activations(a, act_dtype)
    routes = router.route(W, bias, a64, K, topp, norm_topk, routed_scale)
    delta, _ = experts.layer_delta(routes, expert_of, a64)
    if shared is not None:
        for t in range(a64.shape[0]):
            delta[t] += experts.expert_forward(shared.gate, shared.up, shared.down, a64[t])[3]
    return a, routes, delta, r.astype(np.float64) + delta
