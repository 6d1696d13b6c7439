"""Grouped expert MLP, group build and the residual join, in f64.  TEST INFRASTRUCTURE.

For a token t and a kept selection k (expert e = idx_k, weight w_k):

    g = G_e x_t,  u = U_e x_t                 dual gate/up projection  [LOG-tc], [LOG-g4]
    h = silu(g) * u,  silu(z) = z / (1 + exp(-z))                       [LOG-tc] ("silu" launch), [LOG-pipe]
    y = Dn_e h                                 down projection
    delta_t = sum_{k < n_t} w_k * y            per-expert weighting + reduce  [PR434]
    out_t   = residual_t + delta_t             take joins the residual        [PR434]

w_k is the float32 weight the route carries.  The f64 sum has no order to
respect; the GPU's fixed order (k ascending, then slots in issue order) is
checked separately for run-to-run identity.

Group build (S > 1, the small-batch decode of [PR342]): the distinct experts of
all tokens' kept selections in first-appearance order (token-major, k-minor);
each expert's rows are its tokens in ascending order.  Reading: the pages name
the union but not its order; first appearance is the plainest deterministic one.
"""

from __future__ import annotations

from typing import Callable, Dict, List, Tuple

import numpy as np

from . import int4, router


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_forward(gate, up, down, x_t: np.ndarray):
    """(g, u, h, y) in f64 for one token row through one expert (tensors: fmt, gs, O, C, packed, scales)."""
    g = int4.matvec_rows(gate, x_t)
    u = int4.matvec_rows(up, x_t)
    h = silu(g) * u
    y = int4.matvec_rows(down, h)
    return g, u, h, y


def build_group(routes: List[router.RouteResult]):
    """Integer group structure the device builds from the S routes.

    Returns dict with
      entries:     distinct experts, first-appearance order
      entry_rows:  per entry, list of (token, k) in ascending token order
      rows:        flattened (expert, token, k) in entry order (the row numbering)
      token_rows:  per token, row indices for k = 0..n_t-1 (the reduce order)
    """
    entries: List[int] = []
    where: Dict[int, int] = {}
    entry_rows: List[List[Tuple[int, int]]] = []
    for t, r in enumerate(routes):
        for k in range(r.n):
            e = r.idx[k]
            if e not in where:
                where[e] = len(entries)
                entries.append(e)
                entry_rows.append([])
            entry_rows[where[e]].append((t, k))
    rows = []
    row_of = {}
    for j, e in enumerate(entries):
        for (t, k) in entry_rows[j]:
            row_of[(t, k)] = len(rows)
            rows.append((e, t, k))
    token_rows = [[row_of[(t, k)] for k in range(r.n)] for t, r in enumerate(routes)]
    return {"entries": entries, "entry_rows": entry_rows, "rows": rows, "token_rows": token_rows}


def layer_delta(routes: List[router.RouteResult], expert_of: Callable, x64: np.ndarray):
    """delta [S, D] in f64 plus the per-row intermediates {(t, k): (g, u, h, y)}."""
    x64 = np.atleast_2d(x64)
    S, D = x64.shape
    delta = np.zeros((S, D), dtype=np.float64)
    inter = {}
    for t, r in enumerate(routes):
        for k in range(r.n):
            ew = expert_of(r.idx[k])
            g, u, h, y = expert_forward(ew.gate, ew.up, ew.down, x64[t])
            inter[(t, k)] = (g, u, h, y)
            delta[t] += float(r.w32[k]) * y
    return delta, inter


def moe_layer(W, bias, x64, expert_of: Callable, K: int, topp: float, norm_topk: bool,
              routed_scale: float, residual=None):
    """Route, run the kept experts, join the residual.  Returns (routes, group, delta, out)."""
    routes = router.route(W, bias, x64, K, topp, norm_topk, routed_scale)
    group = build_group(routes)
    delta, _ = layer_delta(routes, expert_of, x64)
    out = None
    if residual is not None:
        out = np.asarray(residual, dtype=np.float32).astype(np.float64) + delta
    return routes, group, delta, out
