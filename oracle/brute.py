"""Pure-Python loop formulations for tiny inputs.  TEST INFRASTRUCTURE.

A second, deliberately different route to the same definitions, used to pin the
numpy oracle: weights are decoded one at a time from the packed bytes with
integer operations, dot products are ``math.fsum`` over Python floats, and the
top-K is taken from a full sort on (-score, index) instead of a scan.
"""

from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np


def weight(packed, scales, fmt: int, gs: int, O: int, C: int, o: int, c: int) -> float:
    byte = int(np.asarray(packed, dtype=np.uint8).reshape(O, C // 2)[o, c // 2])
    q = (byte & 0xF) if c % 2 == 0 else (byte >> 4)
    s = np.asarray(scales, dtype=np.float32).reshape(-1)
    if fmt == 4 and gs > 0:
        ng = (C + gs - 1) // gs
        sc = float(s[o * ng + c // gs])
    else:
        sc = float(s[o])
    return (q - 8) * sc


def matvec(t, v: Sequence[float]) -> List[float]:
    return [math.fsum(weight(t.packed, t.scales, t.fmt, t.gs, t.O, t.C, o, c) * float(v[c])
                      for c in range(t.C)) for o in range(t.O)]


def silu(z: float) -> float:
    return z * (1.0 / (1.0 + math.exp(-z))) if z > -700 else 0.0 * z


def logits(W, x: Sequence[float]) -> List[float]:
    W = np.asarray(W, dtype=np.float32)
    return [math.fsum(float(W[e, i]) * float(x[i]) for i in range(W.shape[1])) for e in range(W.shape[0])]


def topk_by_sort(scores: Sequence[float], K: int) -> List[int]:
    order = sorted(range(len(scores)), key=lambda e: (-scores[e], e))
    return order[:K]


def route(W, bias, x, K: int, topp: float, norm_topk: bool, routed_scale: float):
    L = logits(W, x)
    sig = [1.0 / (1.0 + math.exp(-v)) for v in L]
    sc = [sig[e] + float(np.float32(bias[e])) for e in range(len(L))]
    idx = topk_by_sort(sc, K)
    w = [sig[e] for e in idx]
    p = float(np.float32(topp))
    n = K
    if 0.0 < p < 1.0:
        total = 0.0
        for v in w:
            total += v
        acc = 0.0
        for m in range(K):
            acc += w[m]
            if acc >= p * total:
                n = m + 1
                break
    w = w[:n]
    if norm_topk:
        d = 0.0
        for v in w:
            d += v
        w = [v / d for v in w]
    w = [v * float(np.float32(routed_scale)) for v in w]
    return n, idx, w


def expert(gate, up, down, x: Sequence[float]) -> List[float]:
    g = matvec(gate, x)
    u = matvec(up, x)
    h = [silu(a) * b for a, b in zip(g, u)]
    return matvec(down, h)
