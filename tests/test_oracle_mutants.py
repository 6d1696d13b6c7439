"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch every one.

A mutant replaces one oracle function with a subtly wrong version: a swapped
nibble, a dropped offset, a wrong group index, a transposed operand, a bias in
the weights, a non-strict tie-break, a mis-ordered top-p / norm / scale, a
wrong activation, a dropped residual.  If some mutant survived every pin, the
pins would not be pinning that part of the oracle.
"""

import math

import numpy as np
import pytest

from oracle import block, experts, int4, router
from pins_oracle import PINS

_orig_unpack = int4.unpack_nibbles
_orig_scale = int4.scale_matrix
_orig_deq_rows = int4.dequantize_rows
_orig_matvec = int4.matvec_rows
_orig_route_token = router.route_token
_orig_select = router.select_topk
_orig_topp = router.topp_count
_orig_finish = router.finish_weights
_orig_logits = router.router_logits
_orig_build = experts.build_group
_orig_moe = experts.moe_layer
_orig_layer_delta = experts.layer_delta


def m_swap_nibbles(p, O, C):
    q = _orig_unpack(p, O, C)
    out = q.copy()
    out[:, 0::2], out[:, 1::2] = q[:, 1::2], q[:, 0::2]
    return out


def m_no_offset(packed, scales, fmt, gs, O, C, rows):
    rows = np.asarray(rows)
    p = np.asarray(packed, dtype=np.uint8).reshape(O, C // 2)[rows]
    q = _orig_unpack(p, len(rows), C).astype(np.float64)
    return q * _orig_scale(scales, fmt, gs, O, C, rows)


def m_offset7(packed, scales, fmt, gs, O, C, rows):
    return _orig_deq_rows(packed, scales, fmt, gs, O, C, rows) + _orig_scale(scales, fmt, gs, O, C, rows)


def m_group_index(scales, fmt, gs, O, C, rows=None):
    rows = np.arange(O) if rows is None else np.asarray(rows)
    ng = int4.n_groups(fmt, gs, C)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(O, ng)[rows]
    if ng == 1:
        return np.repeat(s, C, axis=1)
    return s[:, np.minimum((np.arange(C) + 1) // gs, ng - 1)]


def m_tail_scale(scales, fmt, gs, O, C, rows=None):
    # the tail group reuses the previous group's scale
    rows = np.arange(O) if rows is None else np.asarray(rows)
    ng = int4.n_groups(fmt, gs, C)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(O, ng)[rows]
    if ng == 1:
        return np.repeat(s, C, axis=1)
    g = np.arange(C) // gs
    if C % gs:
        g = np.where(g == ng - 1, max(ng - 2, 0), g)
    return s[:, g]


def m_row_scale_by_col(scales, fmt, gs, O, C, rows=None):
    rows = np.arange(O) if rows is None else np.asarray(rows)
    if int4.n_groups(fmt, gs, C) == 1:
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        return np.tile(s[np.arange(C) % O], (len(rows), 1))
    return _orig_scale(scales, fmt, gs, O, C, rows)


def m_transpose(t, v, rows=None, block=1024):
    if t.O == t.C:
        W = int4.dequantize(t.packed, t.scales, t.fmt, t.gs, t.O, t.C).T
        rows = np.arange(t.O) if rows is None else np.asarray(rows)
        return W[rows] @ np.asarray(v, dtype=np.float64)
    return _orig_matvec(t, v, rows, block)


def m_biased_weights(logits_t, bias, K, topp, norm_topk, routed_scale):
    r = _orig_route_token(logits_t, bias, K, topp, norm_topk, routed_scale)
    w_sel = [float(router.sigmoid(r.logits[e] + float(bias[e]))) for e in r.idx]
    n, w64 = router.finish_weights(w_sel, topp, norm_topk, routed_scale)
    r.n, r.w64, r.w32 = n, w64, np.asarray(w64, dtype=np.float32)
    return r


def m_weights_from_score(logits_t, bias, K, topp, norm_topk, routed_scale):
    r = _orig_route_token(logits_t, bias, K, topp, norm_topk, routed_scale)
    w_sel = [float(r.scores[e]) for e in r.idx]
    n, w64 = router.finish_weights(w_sel, topp, norm_topk, routed_scale)
    r.n, r.w64, r.w32 = n, w64, np.asarray(w64, dtype=np.float32)
    return r


def m_tie_last(c, K):
    taken = [False] * len(c)
    out = []
    for _ in range(K):
        best = -1
        for e in range(len(c)):
            if not taken[e] and (best < 0 or c[e] >= c[best]):
                best = e
        taken[best] = True
        out.append(best)
    return out


def m_topp_strict(w, p):
    K = len(w)
    if not (0.0 < p < 1.0):
        return K
    total = sum(w)
    run = 0.0
    for m in range(1, K + 1):
        run += w[m - 1]
        if run > p * total:
            return m
    return K


def m_norm_over_K(w_sel, topp, norm_topk, routed_scale):
    K = len(w_sel)
    p = float(np.float32(topp))
    n = router.topp_count(w_sel, p)
    den = sum(w_sel) if norm_topk else 1.0
    kept = [v / den * float(np.float32(routed_scale)) for v in w_sel[:n]]
    return n, kept + [0.0] * (K - n)


def m_scale_first(w_sel, topp, norm_topk, routed_scale):
    s = float(np.float32(routed_scale))
    return _orig_finish([v * s for v in w_sel], topp, norm_topk, 1.0)


def m_no_scale_when_unnormed(w_sel, topp, norm_topk, routed_scale):
    return _orig_finish(w_sel, topp, norm_topk, routed_scale if norm_topk else 1.0)


def m_naive_logits(W, x64):
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    x64 = np.atleast_2d(x64)
    out = np.empty((x64.shape[0], W64.shape[0]))
    for t in range(x64.shape[0]):
        for e in range(W64.shape[0]):
            acc = 0.0
            for v in (W64[e] * x64[t])[::-1]:
                acc += v
            out[t, e] = acc
    return out


def m_first_token_only(W, x64):
    x64 = np.atleast_2d(x64)
    L = _orig_logits(W, x64[:1])
    return np.repeat(L, x64.shape[0], axis=0)


def m_silu_no_sigma(z):
    return np.asarray(z, dtype=np.float64)


def m_silu_sigma_only(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def m_swap_gate_up(gate, up, down, x_t):
    return _orig_expert(up, gate, down, x_t)


_orig_expert = experts.expert_forward


def m_sorted_entries(routes):
    g = _orig_build(routes)
    order = sorted(range(len(g["entries"])), key=lambda j: g["entries"][j])
    entries = [g["entries"][j] for j in order]
    entry_rows = [g["entry_rows"][j] for j in order]
    rows, row_of = [], {}
    for j, e in enumerate(entries):
        for (t, k) in entry_rows[j]:
            row_of[(t, k)] = len(rows)
            rows.append((e, t, k))
    token_rows = [[row_of[(t, k)] for k in range(r.n)] for t, r in enumerate(routes)]
    return {"entries": entries, "entry_rows": entry_rows, "rows": rows, "token_rows": token_rows}


def _group_from_entries(routes, entries, entry_rows):
    rows, row_of = [], {}
    for j, e in enumerate(entries):
        for (t, k) in entry_rows[j]:
            row_of[(t, k)] = len(rows)
            rows.append((e, t, k))
    token_rows = [[row_of[(t, k)] for k in range(r.n)] for t, r in enumerate(routes)]
    return {"entries": entries, "entry_rows": entry_rows, "rows": rows, "token_rows": token_rows}


def m_group_ignores_topp(routes):
    # every one of the K selections becomes a row, also those the top-p cut dropped
    full = [router.RouteResult(n=len(r.idx), idx=r.idx, w64=r.w64, w32=r.w32, logits=r.logits, sigma=r.sigma,
                               scores=r.scores) for r in routes]
    g = _orig_build(full)
    return _group_from_entries(routes, g["entries"], g["entry_rows"])


def m_entry_rows_by_rank(routes):
    # an entry's rows ordered by selection rank (then token) instead of by token
    g = _orig_build(routes)
    entry_rows = [sorted(er, key=lambda tk: (tk[1], tk[0])) for er in g["entry_rows"]]
    return _group_from_entries(routes, g["entries"], entry_rows)


def m_drop_residual(W, bias, x64, expert_of, K, topp, norm_topk, routed_scale, residual=None):
    routes, group, delta, out = _orig_moe(W, bias, x64, expert_of, K, topp, norm_topk, routed_scale, residual)
    return routes, group, delta, (delta.copy() if out is not None else None)


def m_f64_weights(routes, expert_of, x64):
    for r in routes:
        r.w32 = np.asarray(r.w64, dtype=np.float64)
    return _orig_layer_delta(routes, expert_of, x64)


_orig_check = int4.check_format


def m_check_accepts_odd_gs(fmt, gs, O, C):
    # only the format code is checked
    if fmt not in (int4.FMT_ROW, int4.FMT_GROUP):
        raise ValueError(f"unsupported fmt {fmt}")


def m_dequant_unchecked(packed, scales, fmt, gs, O, C, rows):
    # decodes whatever it is handed
    rows = np.asarray(rows)
    p = np.asarray(packed, dtype=np.uint8).reshape(O, C // 2)[rows]
    q = _orig_unpack(p, len(rows), C).astype(np.float64) - 8.0
    return q * _orig_scale(scales, fmt, gs, O, C, rows)


_orig_rmsnorm = block.rmsnorm
_orig_round_bf16 = block.round_bf16
_orig_block = block.moe_block


def m_rms_no_eps(x, gamma, eps):
    return _orig_rmsnorm(x, gamma, 0.0)


def m_rms_eps_outside(x, gamma, eps):
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        ms = math.fsum(float(v) * float(v) for v in x[t]) / x.shape[1]
        out[t] = x[t] / (math.sqrt(ms) + float(np.float32(eps))) * g
    return out


def m_rms_mean_over_d_minus_1(x, gamma, eps):
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        ms = math.fsum(float(v) * float(v) for v in x[t]) / (x.shape[1] - 1)
        out[t] = x[t] / math.sqrt(ms + float(np.float32(eps))) * g
    return out


def m_round_via_f32(v):
    # double rounding: to float32 first, then to bf16
    f = float(np.float32(v))
    return _orig_round_bf16(f)


def m_round_half_up(v):
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)
    q = max(e - 8, -133)
    scaled = math.ldexp(v, -q)
    return math.ldexp(math.floor(abs(scaled) + 0.5) * (1 if v > 0 else -1), q)


def m_shared_half_weight(residual, gamma, eps, act_dtype, W, bias, expert_of, K, topp, norm_topk, routed_scale,
                         shared=None):
    a, routes, delta, out = _orig_block(residual, gamma, eps, act_dtype, W, bias, expert_of, K, topp, norm_topk,
                                        routed_scale, shared=None)
    a64 = router.widen_activations(a, act_dtype)
    if shared is not None:
        for t in range(a64.shape[0]):
            delta[t] += 0.5 * experts.expert_forward(shared.gate, shared.up, shared.down, a64[t])[3]
    r = np.atleast_2d(np.asarray(residual, dtype=np.float32)).astype(np.float64)
    return a, routes, delta, r + delta


def m_shared_on_raw_residual(residual, gamma, eps, act_dtype, W, bias, expert_of, K, topp, norm_topk, routed_scale,
                             shared=None):
    a, routes, delta, out = _orig_block(residual, gamma, eps, act_dtype, W, bias, expert_of, K, topp, norm_topk,
                                        routed_scale, shared=None)
    r = np.atleast_2d(np.asarray(residual, dtype=np.float32)).astype(np.float64)
    if shared is not None:
        for t in range(r.shape[0]):
            delta[t] += experts.expert_forward(shared.gate, shared.up, shared.down, r[t])[3]
    return a, routes, delta, r + delta


MUTANTS = {
    "rmsnorm_without_eps": (block, "rmsnorm", m_rms_no_eps),
    "rmsnorm_eps_outside_sqrt": (block, "rmsnorm", m_rms_eps_outside),
    "rmsnorm_mean_over_d_minus_1": (block, "rmsnorm", m_rms_mean_over_d_minus_1),
    "bf16_double_rounding": (block, "round_bf16", m_round_via_f32),
    "bf16_ties_away": (block, "round_bf16", m_round_half_up),
    "shared_expert_half_weight": (block, "moe_block", m_shared_half_weight),
    "shared_expert_on_raw_residual": (block, "moe_block", m_shared_on_raw_residual),
    "check_accepts_odd_gs": (int4, "check_format", m_check_accepts_odd_gs),
    "dequant_unchecked": (int4, "dequantize_rows", m_dequant_unchecked),
    "swap_nibbles": (int4, "unpack_nibbles", m_swap_nibbles),
    "no_offset": (int4, "dequantize_rows", m_no_offset),
    "offset7": (int4, "dequantize_rows", m_offset7),
    "group_index_off_by_one": (int4, "scale_matrix", m_group_index),
    "tail_group_shares_scale": (int4, "scale_matrix", m_tail_scale),
    "row_scale_by_column": (int4, "scale_matrix", m_row_scale_by_col),
    "transposed_operand": (int4, "matvec_rows", m_transpose),
    "bias_in_weights": (router, "route_token", m_biased_weights),
    "weights_from_score": (router, "route_token", m_weights_from_score),
    "tie_break_last": (router, "select_topk", m_tie_last),
    "topp_strict": (router, "topp_count", m_topp_strict),
    "norm_over_K": (router, "finish_weights", m_norm_over_K),
    "scale_before_norm": (router, "finish_weights", m_scale_first),
    "scale_only_when_normed": (router, "finish_weights", m_no_scale_when_unnormed),
    "naive_reverse_sum_logits": (router, "router_logits", m_naive_logits),
    "first_token_logits": (router, "router_logits", m_first_token_only),
    "silu_without_sigma": (experts, "silu", m_silu_no_sigma),
    "silu_sigma_only": (experts, "silu", m_silu_sigma_only),
    "gate_up_swapped": (experts, "expert_forward", m_swap_gate_up),
    "entries_sorted": (experts, "build_group", m_sorted_entries),
    "group_ignores_topp": (experts, "build_group", m_group_ignores_topp),
    "entry_rows_by_rank": (experts, "build_group", m_entry_rows_by_rank),
    "residual_dropped": (experts, "moe_layer", m_drop_residual),
    "f64_route_weights": (experts, "layer_delta", m_f64_weights),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pname, pin in PINS.items():
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pname)
    assert caught, f"mutant {name} survived every pin"
