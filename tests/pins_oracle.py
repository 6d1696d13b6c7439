"""Pins of the f64 oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
brute-force loop, a closed form, an invariant, a library routine or the
hand-worked example in tests/golden.  ``test_oracle_pins.py`` runs them;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and checks
that at least one pin catches each.
"""

from __future__ import annotations

import json
import math
import os
from types import SimpleNamespace

import numpy as np

import oracle
from oracle import brute, experts, int4, router

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def T(fmt, gs, O, C, packed, scales):
    return SimpleNamespace(fmt=fmt, gs=gs, O=O, C=C, packed=np.asarray(packed, dtype=np.uint8).reshape(O, C // 2),
                           scales=np.asarray(scales, dtype=np.float32))


def rand_tensor(rng, fmt, gs, O, C):
    ng = -(-C // gs) if (fmt == 4 and gs > 0) else 1
    return T(fmt, gs, O, C, rng.integers(0, 256, (O, C // 2), dtype=np.uint8),
             rng.lognormal(math.log(0.01), 0.5, O * ng).astype(np.float32))


def pack_test(q):
    """Test-local packer written from the layout rule: column c -> byte c//2, even c in the low nibble."""
    q = np.asarray(q, dtype=np.uint8)
    O, C = q.shape
    out = np.zeros((O, C // 2), dtype=np.uint8)
    for o in range(O):
        for c in range(C):
            shift = 0 if c % 2 == 0 else 4
            out[o, c // 2] |= np.uint8(int(q[o, c]) << shift)
    return out


# ---------------------------------------------------------------- int4 decoding

def pin_check_format():
    """The format rules of the g4 commit ("Commit history of c/backend_cuda.cu"): only fmt 2
    (per-row) and fmt 4 (group-wise) decode, a group size is even so that no packed byte holds two
    groups, gs = 0 is per-row, and anything else is refused rather than decoded.  Odd C (half a
    byte) and empty shapes are refused by the reading of a byte-packed row."""
    for fmt, gs, O, C in [(2, 0, 4, 8), (4, 0, 4, 8), (4, 2, 4, 8), (4, 64, 3, 200), (4, 256, 1, 64)]:
        int4.check_format(fmt, gs, O, C)
    bad = [(3, 0, 4, 8), (1, 0, 4, 8), (0, 0, 4, 8), (5, 64, 4, 8),   # no other format codes
           (4, 3, 4, 8), (4, 63, 4, 200), (4, -2, 4, 8),              # odd or negative group size
           (2, 64, 4, 8), (2, 2, 4, 8),                                # a per-row tensor has no groups
           (2, 0, 4, 7), (4, 2, 4, 9), (2, 0, 0, 8), (4, 2, 4, 0)]     # half bytes, empty shapes
    for args in bad:
        try:
            int4.check_format(*args)
        except ValueError:
            continue
        raise AssertionError(f"check_format accepted {args}")
    # the decoder applies the rules: an unknown format or an odd group size never decodes
    p = np.full((4, 4), 0x88, np.uint8)
    for fmt, gs, s in [(3, 0, np.ones(4, np.float32)), (4, 3, np.ones(12, np.float32))]:
        try:
            int4.dequantize(p, s, fmt, gs, 4, 8)
        except ValueError:
            continue
        raise AssertionError(f"dequantize decoded fmt={fmt} gs={gs}")


def pin_nibble_roundtrip():
    rng = np.random.default_rng(11)
    for (O, C) in [(1, 2), (3, 10), (7, 64), (2, 200)]:
        q = rng.integers(0, 16, (O, C), dtype=np.uint8)
        assert np.array_equal(int4.unpack_nibbles(pack_test(q), O, C), q)
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = int4.unpack_nibbles(allb, 1, 512)
    assert np.array_equal(pack_test(q), allb)
    # byte 0x8F: column 0 holds 15 (weight +7), column 1 holds 8 (weight 0)
    assert list(int4.unpack_nibbles(np.array([[0x8F]], np.uint8), 1, 2)[0]) == [15, 8]


def pin_dequant_vs_brute():
    rng = np.random.default_rng(12)
    cases = [(2, 0, 3, 8), (4, 64, 3, 200), (4, 64, 2, 2000), (4, 6, 4, 22), (4, 2, 3, 10),
             (4, 0, 3, 16), (4, 300, 2, 200), (4, 64, 5, 128)]
    for fmt, gs, O, C in cases:
        t = rand_tensor(rng, fmt, gs, O, C)
        W = int4.dequantize(t.packed, t.scales, fmt, gs, O, C)
        cols = range(C) if C <= 64 else sorted(set(rng.integers(0, C, 40).tolist()) | {0, C - 1, 63, 64, C - 16})
        for o in range(O):
            for c in cols:
                assert W[o, c] == brute.weight(t.packed, t.scales, fmt, gs, O, C, o, c), (fmt, gs, o, c)


def pin_group_degenerate_cases():
    rng = np.random.default_rng(13)
    O, C = 5, 96
    p = rng.integers(0, 256, (O, C // 2), dtype=np.uint8)
    s_row = rng.lognormal(-4.6, 0.5, O).astype(np.float32)
    W_row = int4.dequantize(p, s_row, 2, 0, O, C)
    # gs = 0 degrades to per-row
    assert np.array_equal(int4.dequantize(p, s_row, 4, 0, O, C), W_row)
    # gs >= C: a single group per row
    assert np.array_equal(int4.dequantize(p, s_row, 4, 128, O, C), W_row)
    # every group of a row sharing that row's scale is per-row
    ng = -(-C // 64)
    assert np.array_equal(int4.dequantize(p, np.repeat(s_row, ng), 4, 64, O, C), W_row)


def pin_matvec_closed_forms():
    rng = np.random.default_rng(14)
    O, C = 4, 40
    s = np.array([0.5, 1.0, 2.0, 0.25], np.float32)
    x = rng.standard_normal(C)
    zero = T(2, 0, O, C, np.full((O, C // 2), 0x88), s)
    assert np.all(int4.matvec_rows(zero, x) == 0.0)
    ones = T(2, 0, O, C, np.full((O, C // 2), 0x99), s)
    assert np.allclose(int4.matvec_rows(ones, x), s.astype(np.float64) * math.fsum(x), rtol=1e-13, atol=1e-13)
    # 0x0F: even columns +7, odd columns -8
    alt = T(2, 0, O, C, np.full((O, C // 2), 0x0F), s)
    e0 = np.zeros(C); e0[0] = 1.0
    e1 = np.zeros(C); e1[1] = 1.0
    assert np.array_equal(int4.matvec_rows(alt, e0), 7.0 * s.astype(np.float64))
    assert np.array_equal(int4.matvec_rows(alt, e1), -8.0 * s.astype(np.float64))
    assert np.array_equal(int4.matvec_rows(alt, np.ones(C)), -0.5 * C * s.astype(np.float64))
    # one-hot input picks one column of a random group-wise tensor: tail group column
    t = rand_tensor(rng, 4, 16, 3, 40)
    ec = np.zeros(40); ec[37] = 1.0
    col = [brute.weight(t.packed, t.scales, 4, 16, 3, 40, o, 37) for o in range(3)]
    assert np.array_equal(int4.matvec_rows(t, ec), np.array(col))


def pin_matvec_vs_fsum():
    rng = np.random.default_rng(15)
    for fmt, gs, O, C in [(2, 0, 6, 24), (4, 8, 5, 36), (4, 64, 3, 200), (2, 0, 12, 12), (4, 4, 10, 10)]:
        t = rand_tensor(rng, fmt, gs, O, C)
        v = rng.standard_normal(C)
        ref = np.array(brute.matvec(t, v.tolist()))
        got = int4.matvec_rows(t, v)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max()), (fmt, gs, O, C)


# ---------------------------------------------------------------- activation / silu

def pin_silu():
    assert experts.silu(0.0) == 0.0
    for z in [0.1, 0.5, 1.0, 2.0, 3.7, 10.0, 25.0]:
        assert abs((experts.silu(z) - experts.silu(-z)) - z) <= 4e-16 * max(1.0, z)
        assert abs(experts.silu(z) - z / (1.0 + math.exp(-z))) <= 1e-15 * z
    assert abs(experts.silu(50.0) - 50.0) < 1e-18 * 1e6
    assert abs(experts.silu(-50.0)) < 1e-19
    assert experts.silu(-1000.0) == 0.0


def pin_widen_bf16():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F7F], np.uint16)
    v = router.widen_activations(bits, "bf16")
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 3.140625
    assert v[3] == 2.0 ** -133
    assert v[4] == (2 - 2.0 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------- router

def pin_logits():
    rng = np.random.default_rng(16)
    W = rng.normal(0, 0.02, (6, 64)).astype(np.float32)
    x = rng.standard_normal((2, 64)).astype(np.float32).astype(np.float64)
    L = router.router_logits(W, x)
    for t in range(2):
        assert L[t].tolist() == brute.logits(W, x[t].tolist())
        assert np.allclose(L[t], W.astype(np.float64) @ x[t], rtol=1e-12, atol=1e-15)
    onehot = np.zeros((1, 64)); onehot[0, 5] = 1.0
    assert np.array_equal(router.router_logits(W, onehot)[0], W[:, 5].astype(np.float64))


def pin_topk_vs_sort():
    rng = np.random.default_rng(17)
    for E in [1, 2, 5, 8, 64, 256]:
        c = rng.standard_normal(E)
        for K in sorted({1, min(2, E), min(8, E), E}):
            assert router.select_topk(c, K) == brute.topk_by_sort(c.tolist(), K)
            assert router.select_topk(c, K) == np.lexsort((np.arange(E), -c))[:K].tolist()
    c = np.array([0.3, 0.7, 0.7, 0.1, 0.7, 0.3])
    assert router.select_topk(c, 6) == [1, 2, 4, 0, 5, 3]
    assert sorted(router.select_topk(rng.standard_normal(17), 17)) == list(range(17))


def pin_topp_hand():
    w = [0.5, 0.25, 0.125, 0.125]
    assert router.finish_weights(w, 0.75, False, 1.0)[0] == 2
    assert router.finish_weights(w, 0.7, False, 1.0)[0] == 2
    assert router.finish_weights(w, 0.8, False, 1.0)[0] == 3
    assert router.finish_weights(w, 0.5, False, 1.0)[0] == 1
    assert router.finish_weights(w, 1.0, False, 1.0)[0] == 4
    assert router.finish_weights(w, 0.0, False, 1.0)[0] == 4
    assert router.finish_weights(w, 1e-30, False, 1.0)[0] == 1
    n, ww = router.finish_weights(w, 0.8, True, 1.0)
    assert n == 3 and ww == [0.5 / 0.875, 0.25 / 0.875, 0.125 / 0.875, 0.0]


def pin_norm_and_scale():
    rng = np.random.default_rng(18)
    for scale in [1.0, 2.5, 0.3]:
        w = rng.uniform(0.05, 1.0, 8).tolist()
        n, ww = router.finish_weights(w, 0.0, True, scale)
        assert n == 8 and abs(math.fsum(ww) - float(np.float32(scale))) <= 1e-14 * scale
        n, ww = router.finish_weights(w, 0.0, False, scale)
        assert ww == [v * float(np.float32(scale)) for v in w]


def pin_bias_only_in_choice():
    # l = [0, 0.1]; bias favours expert 0, whose weight must still be sigma(0) = 0.5
    W = np.array([[0.0, 0.0], [0.1, 0.0]], np.float32)
    x = np.array([[1.0, 0.0]])
    b = np.array([0.1, 0.0], np.float32)
    r = router.route(W, b, x, 1, 0.0, False, 1.0)[0]
    assert r.idx == [0] and r.n == 1 and r.w64[0] == 0.5


def pin_route_vs_brute():
    rng = np.random.default_rng(19)
    for trial in range(40):
        E = int(rng.choice([4, 8, 16]))
        D = 32
        K = int(rng.integers(1, min(E, 8) + 1))
        W = rng.normal(0, 0.3, (E, D)).astype(np.float32)
        b = rng.normal(0, 0.1, E).astype(np.float32)
        x = rng.standard_normal((2, D)).astype(np.float32).astype(np.float64)
        topp = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
        norm = bool(rng.integers(0, 2))
        scale = float(rng.choice([1.0, 2.5, 0.75]))
        rs = router.route(W, b, x, K, topp, norm, scale)
        for t in range(2):
            n, idx, w = brute.route(W, b, x[t].tolist(), K, topp, norm, scale)
            assert rs[t].n == n and rs[t].idx == idx, trial
            assert np.allclose(rs[t].w64[:n], w, rtol=1e-15, atol=0)
            assert all(v == 0.0 for v in rs[t].w64[n:])


# ---------------------------------------------------------------- groups and the whole layer

def pin_group_build_hand():
    mk = lambda idx: router.RouteResult(n=len(idx), idx=idx, w64=[0.0] * len(idx),
                                        w32=np.zeros(len(idx), np.float32), logits=None, sigma=None, scores=None)
    g = experts.build_group([mk([3, 1]), mk([1, 5]), mk([5, 3])])
    assert g["entries"] == [3, 1, 5]
    assert g["entry_rows"] == [[(0, 0), (2, 1)], [(0, 1), (1, 0)], [(1, 1), (2, 0)]]
    assert g["rows"] == [(3, 0, 0), (3, 2, 1), (1, 0, 1), (1, 1, 0), (5, 1, 1), (5, 2, 0)]
    assert g["token_rows"] == [[0, 2], [3, 4], [5, 1]]
    r = mk([2, 7, 4])
    r.n = 2
    g = experts.build_group([r])
    assert g["entries"] == [2, 7] and g["token_rows"] == [[0, 1]]


def pin_group_build_invariants():
    """Random routes with repeated experts and top-p cuts: the rows are exactly the kept
    (token, k) pairs, each under its own expert; entries follow first appearance in token-major
    order; an entry's rows are contiguous with ascending tokens; a token's reduce list names
    its own rows in route order."""
    rng = np.random.default_rng(77)
    for trial in range(300):
        S, K, E = int(rng.integers(1, 9)), int(rng.integers(1, 9)), int(rng.integers(8, 20))
        routes = []
        for _ in range(S):
            idx = [int(e) for e in rng.choice(E, size=K, replace=False)]
            n = int(rng.integers(1, K + 1))
            routes.append(router.RouteResult(n=n, idx=idx, w64=[0.0] * K, w32=np.zeros(K, np.float32),
                                             logits=None, sigma=None, scores=None))
        g = experts.build_group(routes)
        kept = {(t, k) for t, r in enumerate(routes) for k in range(r.n)}
        assert sorted((t, k) for _, t, k in g["rows"]) == sorted(kept), trial
        assert all(e == routes[t].idx[k] for e, t, k in g["rows"]), trial
        first = {}
        for t, k in sorted(kept):
            first.setdefault(routes[t].idx[k], (t, k))
        assert g["entries"] == sorted(first, key=lambda e: first[e]), trial
        row_entries = [e for e, _, _ in g["rows"]]
        assert [e for j, e in enumerate(row_entries) if j == 0 or row_entries[j - 1] != e] == g["entries"], trial
        for e in g["entries"]:
            toks = [t for x, t, _ in g["rows"] if x == e]
            assert toks == sorted(set(toks)), trial
        for t, r in enumerate(routes):
            assert [g["rows"][i][1:] for i in g["token_rows"][t]] == [(t, k) for k in range(r.n)], trial


def identity_expert(D, diag_nibble=9, scale=1.0):
    q = np.full((D, D), 8, np.uint8)
    np.fill_diagonal(q, diag_nibble)
    t = T(2, 0, D, D, pack_test(q), np.full(D, scale, np.float32))
    return SimpleNamespace(gate=t, up=t, down=t)


def pin_layer_closed_form():
    D = 6
    rng = np.random.default_rng(20)
    x = rng.standard_normal((1, D)).astype(np.float32).astype(np.float64)
    r = rng.standard_normal((1, D)).astype(np.float32)
    W = rng.normal(0, 0.5, (1, D)).astype(np.float32)
    b = np.zeros(1, np.float32)
    ex = identity_expert(D)
    # one expert, norm on: weight = routed_scale exactly; y = silu(x) * x elementwise
    _, _, delta, out = experts.moe_layer(W, b, x, lambda e: ex, 1, 0.0, True, 2.5, residual=r)
    y = np.array([v / (1.0 + math.exp(-v)) * v for v in x[0]])
    assert np.allclose(delta[0], 2.5 * y, rtol=1e-14, atol=0)
    assert np.allclose(out[0], r[0].astype(np.float64) + 2.5 * y, rtol=1e-14, atol=1e-15)
    # norm off, scale 1: the weight is float32(sigma(l)) -- the route carries float32
    _, _, delta, _ = experts.moe_layer(W, b, x, lambda e: ex, 1, 0.0, False, 1.0)
    l = math.fsum((W[0].astype(np.float64) * x[0]).tolist())
    w32 = float(np.float32(1.0 / (1.0 + math.exp(-l))))
    assert np.allclose(delta[0], w32 * y, rtol=1e-14, atol=0)


def pin_layer_linearity():
    rng = np.random.default_rng(21)
    D, I, E = 16, 8, 4
    ex = {e: SimpleNamespace(gate=rand_tensor(rng, 2, 0, I, D), up=rand_tensor(rng, 4, 4, I, D),
                             down=rand_tensor(rng, 4, 6, D, I)) for e in range(E)}
    W = rng.normal(0, 0.3, (E, D)).astype(np.float32)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    x = rng.standard_normal((2, D)).astype(np.float32).astype(np.float64)
    _, _, d1, _ = experts.moe_layer(W, b, x, lambda e: ex[e], 2, 0.0, True, 1.0)
    ex2 = {e: SimpleNamespace(gate=v.gate, up=v.up,
                              down=T(4, 6, D, I, v.down.packed, v.down.scales * 2)) for e, v in ex.items()}
    _, _, d2, _ = experts.moe_layer(W, b, x, lambda e: ex2[e], 2, 0.0, True, 1.0)
    assert np.array_equal(d2, 2 * d1)
    ex3 = {e: SimpleNamespace(gate=v.gate, up=T(4, 4, I, D, v.up.packed, v.up.scales * 4),
                              down=v.down) for e, v in ex.items()}
    _, _, d3, _ = experts.moe_layer(W, b, x, lambda e: ex3[e], 2, 0.0, True, 1.0)
    assert np.array_equal(d3, 4 * d1)


def pin_layer_vs_brute():
    rng = np.random.default_rng(22)
    D, I, E, K, S = 12, 6, 5, 2, 2
    ex = {}
    for e in range(E):
        fmt, gs = [(2, 0), (4, 4), (4, 6)][e % 3]
        ex[e] = SimpleNamespace(gate=rand_tensor(rng, fmt, gs, I, D), up=rand_tensor(rng, fmt, gs, I, D),
                                down=rand_tensor(rng, fmt, gs, D, I))
    W = rng.normal(0, 0.3, (E, D)).astype(np.float32)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    x = rng.standard_normal((S, D)).astype(np.float32).astype(np.float64)
    routes, _, delta, _ = experts.moe_layer(W, b, x, lambda e: ex[e], K, 0.9, True, 2.5)
    for t in range(S):
        n, idx, w = brute.route(W, b, x[t].tolist(), K, 0.9, True, 2.5)
        ref = [0.0] * D
        for k in range(n):
            y = brute.expert(ex[idx[k]].gate, ex[idx[k]].up, ex[idx[k]].down, x[t].tolist())
            ref = [a + float(np.float32(w[k])) * v for a, v in zip(ref, y)]
        assert np.allclose(delta[t], ref, rtol=1e-11, atol=1e-14 * max(map(abs, ref)))


def load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    exs = []
    for e in g["experts"]:
        def t(name, O, C):
            pk = np.array([[int(h, 16) for h in row] for row in e[name]["packed"]], np.uint8)
            return T(e["fmt"], e["gs"], O, C, pk, e[name]["scales"])
        exs.append(SimpleNamespace(gate=t("gate", g["I"], g["D"]), up=t("up", g["I"], g["D"]),
                                   down=t("down", g["D"], g["I"])))
    return g, exs


def pin_worked_example():
    g, exs = load_worked_example()
    x = np.array([g["x"]])
    W = np.array(g["router_W"], np.float32)
    b = np.array(g["router_b"], np.float32)
    r = np.array([g["residual"]], np.float32)
    s = lambda z: z / (1.0 + math.exp(-z))
    # Hand derivation.  All three logits are 0, so sigma = 1/2 and the scores are
    # 1/2 + b = [0.5, 0.75, 0.25]: top-2 = [1, 0], weights 1/2 each, norm -> 1/2,
    # times 2.5 -> 1.25.  Expert 1 (per-row): g = [x0, x2] = [1, 2],
    # u = [-x1, 2*0.5*x3] = [1, 0.5], h = [s(1), 0.5 s(2)],
    # y = 0.5*[2h0, 2h1, h0+h1, -h0].  Expert 0 (gs=2): g = [(x0+x1) + 0.5(x2+x3), 2 x2]
    # = [1.25, 4], u = [2 x0, 0.25*4*x3] = [2, 0.5], h = [2 s(1.25), 0.5 s(4)],
    # y = [h0, h1, h0-h1, 0].
    h1 = [s(1.0), 0.5 * s(2.0)]
    y1 = [h1[0], h1[1], 0.5 * (h1[0] + h1[1]), -0.5 * h1[0]]
    h0 = [2.0 * s(1.25), 0.5 * s(4.0)]
    y0 = [h0[0], h0[1], h0[0] - h0[1], 0.0]
    routes, group, delta, out = experts.moe_layer(W, b, x, lambda e: exs[e], 2, 0.0, True, g["routed_scale"],
                                                  residual=r)
    assert routes[0].idx == [1, 0] and routes[0].n == 2
    assert routes[0].w32.tolist() == [1.25, 1.25]
    exp = [1.25 * a + 1.25 * c for a, c in zip(y1, y0)]
    assert np.allclose(delta[0], exp, rtol=1e-15, atol=1e-16)
    assert np.allclose(out[0], [rv + ev for rv, ev in zip(g["residual"], exp)], rtol=1e-15, atol=1e-15)
    assert group["entries"] == [1, 0]
    # top-p 0.4: prefix 0.5 >= 0.4 * 1.0 keeps one expert, renormalised to 1, times 2.5
    routes, _, delta, _ = experts.moe_layer(W, b, x, lambda e: exs[e], 2, 0.4, True, g["routed_scale"])
    assert routes[0].n == 1 and routes[0].w32.tolist() == [2.5, 0.0]
    assert np.allclose(delta[0], [2.5 * v for v in y1], rtol=1e-15, atol=1e-16)




# ---------------------------------------------------------------- the block around the experts

def _bf16_table():
    """Every finite bf16 value, ascending, with its bit pattern: brute force for the rounding."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    keep = np.isfinite(f)
    vals = np.where(keep, f, 0).astype(np.float64)
    vals, bits = vals[keep], bits[keep]
    order = np.lexsort((bits, vals))
    vals, bits = vals[order], bits[order]
    # -0 and +0 compare equal: keep +0 only
    first = np.concatenate([[True], vals[1:] != vals[:-1]])
    return vals[first], bits[first]


def pin_round_bf16_brute():
    """Nearest bf16, ties to the even pattern, by search over the whole bf16 table; exact ties,
    values just off a tie (where an intermediate float32 rounding would fall on the tie and go
    to even), subnormals, and the overflow edge."""
    vals, bits = _bf16_table()
    rng = np.random.default_rng(21)
    cases = list(rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000)))
    for i in rng.integers(1, len(vals) - 2, 400):
        lo, hi = vals[i], vals[i + 1]
        if np.isfinite(lo) and np.isfinite(hi):
            mid = (lo + hi) / 2
            cases += [mid, mid + abs(mid) * 2.0 ** -40, mid - abs(mid) * 2.0 ** -40]
    cases += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 1e-45, 2.0 ** 127 * 1.99, 3.3e38, 3.4e38, -3.39e38]
    for v in cases:
        v = float(v)
        got = oracle.block.round_bf16(v)
        j = np.searchsorted(vals, v)
        if j >= len(vals):
            assert math.isinf(got) and got > 0, v
            continue
        cand = [vals[j]] + ([vals[j - 1]] if j > 0 else [])
        d = [abs(c - v) for c in cand]
        if len(cand) == 2 and d[0] == d[1]:
            want = cand[0] if bits[j] % 2 == 0 else cand[1]
        else:
            want = cand[int(np.argmin(d))]
        # past the largest finite value: ties and beyond go to infinity
        if abs(v) >= 2.0 ** 128 - 2.0 ** 119:
            assert math.isinf(got), v
            continue
        assert got == want, (v, got, want)


def pin_round_bf16_vs_bits():
    """For float32 inputs the rounding equals the integer round-to-nearest-even on the bit
    pattern (the synthetic inputs' own conversion)."""
    from synth import round_f32_to_bf16_bits
    rng = np.random.default_rng(22)
    x = (rng.standard_normal(5000) * np.exp(rng.uniform(-30, 30, 5000))).astype(np.float32)
    # exact float32 ties of bf16: low half 0x8000
    t = (rng.integers(0, 1 << 16, 500).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, t[np.isfinite(t)]])
    got = oracle.block.round_activations(x.astype(np.float64), "bf16")
    assert np.array_equal(got, round_f32_to_bf16_bits(x))


def pin_rmsnorm_forms():
    rng = np.random.default_rng(23)
    D = 64
    g1 = np.ones(D, np.float32)
    # a constant row c: every output is c / sqrt(c^2 + eps)
    for c, eps in [(3.0, 1e-5), (-0.25, 1e-6), (1e-4, 1e-5)]:
        out = oracle.block.rmsnorm(np.full((1, D), c), g1, eps)
        e = float(np.float32(eps))
        assert np.allclose(out, c / math.sqrt(c * c + e), rtol=1e-15, atol=0)
    # eps = 0: the output's mean square is exactly 1 (to rounding), and scaling the row changes nothing
    x = rng.standard_normal((3, D))
    out = oracle.block.rmsnorm(x, g1, 0.0)
    assert np.allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-14)
    assert np.allclose(oracle.block.rmsnorm(7.5 * x, g1, 0.0), out, rtol=1e-14)
    # gamma multiplies column by column
    g = rng.normal(1.0, 0.2, D).astype(np.float32)
    assert np.allclose(oracle.block.rmsnorm(x, g, 1e-5), oracle.block.rmsnorm(x, g1, 1e-5) * g.astype(np.float64),
                       rtol=1e-15)
    # against a second formulation: the Euclidean norm
    e = float(np.float32(1e-5))
    ref = x / np.sqrt(np.linalg.norm(x, axis=1) ** 2 / D + e)[:, None]
    assert np.allclose(oracle.block.rmsnorm(x, g1, 1e-5), ref, rtol=1e-13)


def pin_block_identities():
    """The block is rmsnorm -> rounding -> the layer of the routed experts, plus the shared
    expert with weight 1, plus the residual."""
    rng = np.random.default_rng(24)
    D, I, E, K = 16, 8, 4, 2
    ex = [SimpleNamespace(gate=rand_tensor(rng, 2, 0, I, D), up=rand_tensor(rng, 2, 0, I, D),
                          down=rand_tensor(rng, 4, 4, D, I)) for _ in range(E)]
    sh = SimpleNamespace(gate=rand_tensor(rng, 4, 4, I, D), up=rand_tensor(rng, 2, 0, I, D),
                         down=rand_tensor(rng, 2, 0, D, I))
    W = rng.normal(0, 0.5, (E, D)).astype(np.float32)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    r = rng.standard_normal((2, D)).astype(np.float32)
    gam = rng.normal(1, 0.1, D).astype(np.float32)
    for dt in ("f32", "bf16"):
        a, routes, delta, out = oracle.block.moe_block(r, gam, 1e-5, dt, W, b, lambda e: ex[e], K, 0.0, True, 2.0,
                                                       shared=sh)
        n = oracle.block.rmsnorm(r, gam, 1e-5)
        a64 = router.widen_activations(a, dt)
        assert np.max(np.abs(a64 - n)) <= (2.0 ** -8 if dt == "bf16" else 2.0 ** -24) * np.max(np.abs(n))
        _, _, d_routed, _ = experts.moe_layer(W, b, a64, lambda e: ex[e], K, 0.0, True, 2.0)
        for t in range(2):
            ys = brute.expert(sh.gate, sh.up, sh.down, a64[t].tolist())
            assert np.allclose(delta[t], d_routed[t] + np.array(ys), rtol=1e-12, atol=1e-14)
            assert np.allclose(out[t], r[t].astype(np.float64) + delta[t], rtol=0, atol=0)
    # a shared expert of zero weights (all nibbles 8) adds nothing
    z = SimpleNamespace(gate=T(2, 0, I, D, np.full((I, D // 2), 0x88), np.ones(I)),
                        up=T(2, 0, I, D, np.full((I, D // 2), 0x88), np.ones(I)),
                        down=T(2, 0, D, I, np.full((D, I // 2), 0x88), np.ones(D)))
    _, _, d0, _ = oracle.block.moe_block(r, gam, 1e-5, "f32", W, b, lambda e: ex[e], K, 0.0, True, 2.0, shared=z)
    _, _, d1, _ = oracle.block.moe_block(r, gam, 1e-5, "f32", W, b, lambda e: ex[e], K, 0.0, True, 2.0)
    assert np.array_equal(d0, d1)


PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_") and callable(fn)}
