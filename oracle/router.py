"""Device-router semantics in f64, written from [LOG-rt].  TEST INFRASTRUCTURE.

Per token t the router computes (all in f64, inputs widened exactly):

1. logits  l_e = sum_i W_r[e, i] * x_t[i]         (E x D GEMV; correctly rounded via math.fsum)
2. sigma_e = 1 / (1 + exp(-l_e))                    (sigmoid)
3. score   c_e = sigma_e + b_e                      (bias-augmented, used only for choosing)
4. top-K by choice: K rounds, each taking the first e (ascending) among the
   not-yet-chosen whose score is strictly greater than the best so far
5. w_k = sigma_{idx_k}                              (weight from the raw, unbiased logit)
6. route-level top-p, if 0 < p < 1: keep the shortest prefix (in selection
   order, at least one) whose running sum reaches p * sum_{k<K} w_k
7. norm_topk: w_k /= sum_{j<n} w_j                  (running sum in selection order)
8. w_k *= routed_scale; the route carries float32(w_k)

Readings (pages silent or terse): the bias only enters the choice (step 3, since
weights come "from the raw logit"); top-p is applied to the K selected in
selection order with ">="; truncation precedes norm, which precedes the scale;
routed_scale applies with norm off too; no epsilon in the norm.  Weights of
dropped selections (k >= n) are reported as 0.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List

import numpy as np


def widen_activations(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact f64 values of device activations: float32 as is, bf16 bit patterns by a 16-bit shift."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def router_logits(W: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """f64 [S, E]; each entry is the correctly rounded dot product (f32*f32 products are exact in f64)."""
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    x64 = np.atleast_2d(x64)
    S, E = x64.shape[0], W64.shape[0]
    out = np.empty((S, E), dtype=np.float64)
    for t in range(S):
        prod = W64 * x64[t][None, :]
        for e in range(E):
            out[t, e] = math.fsum(prod[e].tolist())
    return out


def sigmoid(l: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(l, dtype=np.float64)))


def choice_scores(sig: np.ndarray, bias: np.ndarray) -> np.ndarray:
    return np.asarray(sig, dtype=np.float64) + np.asarray(bias, dtype=np.float32).astype(np.float64)


def select_topk(c: np.ndarray, K: int) -> List[int]:
    """K rounds of a strict-'>' ascending scan over the unchosen experts [LOG-rt]."""
    E = len(c)
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    taken = [False] * E
    out = []
    for _ in range(K):
        best = -1
        for e in range(E):
            if taken[e]:
                continue
            if best < 0 or c[e] > c[best]:
                best = e
        taken[best] = True
        out.append(best)
    return out


def topp_count(w: List[float], p: float) -> int:
    """Kept count n for route-level top-p over the selected weights, selection order."""
    K = len(w)
    if not (0.0 < p < 1.0):
        return K
    total = 0.0
    for v in w:
        total += v
    thr = p * total
    run = 0.0
    for m in range(1, K + 1):
        run += w[m - 1]
        if run >= thr:
            return m
    return K


def finish_weights(w_sel: List[float], topp: float, norm_topk: bool, routed_scale: float):
    """Steps 6-8.  Returns (n, f64 weights of length K with zeros past n)."""
    K = len(w_sel)
    p = float(np.float32(topp))
    n = topp_count(w_sel, p)
    kept = list(w_sel[:n])
    if norm_topk:
        den = 0.0
        for v in kept:
            den += v
        kept = [v / den for v in kept]
    scale = float(np.float32(routed_scale))
    kept = [v * scale for v in kept]
    return n, kept + [0.0] * (K - n)


@dataclass
class RouteResult:
    n: int
    idx: List[int]            # K selections, selection order
    w64: List[float]          # final f64 weights (0 past n)
    w32: np.ndarray           # float32(w64): what the route carries
    logits: np.ndarray        # f64 [E]
    sigma: np.ndarray         # f64 [E]
    scores: np.ndarray        # f64 [E]


def route_token(logits_t: np.ndarray, bias: np.ndarray, K: int, topp: float,
                norm_topk: bool, routed_scale: float) -> RouteResult:
    sig = sigmoid(logits_t)
    c = choice_scores(sig, bias)
    idx = select_topk(c, K)
    w_sel = [float(sig[e]) for e in idx]
    n, w64 = finish_weights(w_sel, topp, norm_topk, routed_scale)
    return RouteResult(n=n, idx=idx, w64=w64, w32=np.asarray(w64, dtype=np.float32),
                       logits=np.asarray(logits_t, dtype=np.float64), sigma=sig, scores=c)


def route(W, bias, x64, K: int, topp: float, norm_topk: bool, routed_scale: float) -> List[RouteResult]:
    """All S tokens; the S rows share one GEMV, each token is routed on its own ([LOG-pipe], batched router)."""
    L = router_logits(W, x64)
    return [route_token(L[t], bias, K, topp, norm_topk, routed_scale) for t in range(L.shape[0])]
