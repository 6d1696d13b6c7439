"""HIP path vs the f64 oracle through the C ABI, on seeded synthetic layers (MI355X only)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from harness import (TOL, digest, gpu_routes, layer_delta_threads, make_layer, near_tie, normwise_err, oracle_routes,
                     route_matches, upload_layer, x_to_device)
from synth import get_config

pytestmark = pytest.mark.gpu


def new_ctx():
    import torch
    from int4_grouped_expert_router_amd import Context
    assert torch.cuda.is_available()
    return Context(0, torch.cuda.current_stream())


def issue_with_taps(ctx, cfg, L, layer, x, K, topp, norm, scale):
    """route + issue, read the h and y taps before take; returns (route recs, h, y)."""
    from int4_grouped_expert_router_amd import binding as B
    rec = ctx.route(layer, x, K, topp, norm, scale, host_out=True)
    slot = ctx.issue(layer, x)
    h = ctx.tap(B.I4MOE_TAP_H)
    y = ctx.tap(B.I4MOE_TAP_Y, slot)
    return rec, h.reshape(-1, cfg.I), y.reshape(-1, cfg.D)


def check_group(ctx, layer, routes):
    g = ctx.tap_group(layer)
    og = oracle.build_group(routes)
    assert g["n_entries"] == len(og["entries"])
    assert g["entry_expert"][:g["n_entries"]].tolist() == og["entries"]
    assert g["n_rows"] == len(og["rows"])
    for row, (e, t, k) in enumerate(og["rows"]):
        assert g["row_expert"][row] == e and g["row_token"][row] == t
        assert g["row_weight"][row].view(np.uint32) == routes[t].w32[k].view(np.uint32)
    for t, rows in enumerate(og["token_rows"]):
        lo, hi = g["tok_row0"][t], g["tok_row0"][t + 1]
        assert g["red_rows"][lo:hi].tolist() == rows
    # the ends of both offset arrays, also when they sit at index 64
    assert g["entry_row0"][g["n_entries"]] == g["n_rows"]
    assert g["tok_row0"][len(og["token_rows"])] == g["n_rows"]
    return og


def full_layer_check(cfg, layer=0, mutate=None):
    """One layer against the oracle, element by element: the route (bit for bit away from
    near-ties), the group, every h row and every y row (the oracle's y from its own h, from x),
    and the layer delta.  A near-tie token's experts are checked on the GPU's own route, after the
    oracle's selection on the GPU's own logits has been shown to give that route.  Then the same
    layer in the launch configuration the benchmark times (no host copy of the route, no taps:
    the selection deferred into the dual projection where it can be, the down projection fused
    into the take where it can be) must give the same delta bits, and the residual join must add
    them exactly.  mutate(L), if given, edits the generated layer first (e.g. its x)."""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    L = make_layer(cfg, layer)
    if mutate is not None:
        mutate(L)
    ctx = new_ctx()
    upload_layer(ctx, L, layer)
    x = x_to_device(L.x, L.x_dtype)
    routes, x64 = oracle_routes(cfg, L)
    rec, h, y = issue_with_taps(ctx, cfg, L, layer, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    logits = ctx.tap(B.I4MOE_TAP_LOGITS, 0, np.float64).reshape(cfg.S, cfg.E)
    zero = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(zero)
    torch.cuda.synchronize()
    delta_gpu = zero.cpu().numpy()
    grec = gpu_routes(rec, cfg.S, cfg.K)
    use = []
    for t in range(cfg.S):
        if near_tie(routes[t], cfg.K, cfg.topp):
            r2 = oracle.route_token(logits[t], L.router_b, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
            assert route_matches(rec[t], r2, cfg.K), ("near-tie token: route differs on the GPU's logits", t)
            print(f"[parity] token {t}: near-tie, experts checked on the GPU's route", flush=True)
            use.append(grec[t])
        else:
            assert route_matches(rec[t], routes[t], cfg.K), (t, list(rec[t].idx[:cfg.K]), routes[t].idx)
            use.append(routes[t])
    og = check_group(ctx, layer, use)
    delta, inter = layer_delta_threads(use, L.expert, x64)
    for row, (e, t, k) in enumerate(og["rows"]):
        assert normwise_err(h[row], inter[(t, k)][2]) < TOL, ("h", row)
        assert normwise_err(y[row], inter[(t, k)][3]) < TOL, ("y", row)
    err = normwise_err(delta_gpu, delta)
    assert err < TOL, err
    # the benchmark's launch configuration: same bits
    ctx.route(layer, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(layer, x)
    fast = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(fast)
    torch.cuda.synchronize()
    assert fast.cpu().numpy().tobytes() == delta_gpu.tobytes()
    # residual join: out = residual + delta, bit for bit the f32 sum of the same delta
    ctx.route(layer, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(layer, x)
    r = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.take(r)
    torch.cuda.synchronize()
    out = r.cpu().numpy()
    assert np.array_equal(out, (L.residual + delta_gpu).astype(np.float32))
    ctx.close()
    print(f"[parity] {cfg.name}: normwise error {err:.2e} over {len(og['rows'])} rows", flush=True)
    return err


@pytest.mark.parametrize("name", ["tiny", "medium", "mix", "small_batch", "sustained"])
def test_full_layer(name):
    """Every workload at its full size, in both launch configurations, element by element."""
    print(f"[parity] full layer {name}", flush=True)
    full_layer_check(get_config(name))


RAGGED = [
    # D, I, E, K, S, formats, gs, x dtype
    (1000, 200, 16, 4, 1, "mix_even_odd", 64, "f32"),
    (2050, 650, 8, 2, 3, "mix_even_odd", 6, "bf16"),
    (4096, 1536, 32, 8, 2, "row", 0, "bf16"),
    (7168, 2048, 16, 8, 1, "mix_even_odd", 64, "f32"),
    (512, 256, 4, 2, 1, "group", 128, "f32"),
    (512, 96, 6, 3, 2, "group", 256, "bf16"),
    (256, 128, 8, 8, 8, "mix_even_odd", 2, "f32"),
    (130, 34, 5, 5, 1, "mix_even_odd", 32, "bf16"),
    (256, 128, 64, 1, 64, "row", 0, "f32"),         # 64 tokens: the group's offsets end at 64
    (512, 256, 128, 2, 32, "group", 64, "bf16"),    # up to 64 distinct experts in one group
    (1024, 512, 256, 8, 1, "group", 64, "bf16"),    # one token, 256 experts: the select kernel at S=1
    (256, 128, 130, 4, 2, "row", 0, "f32"),         # 130 experts: a lane's third column holds two
    (1024, 2304, 8, 2, 1, "group", 64, "f32"),      # down rows of 2304 columns: the long-row down kernel
    (512, 4096, 4, 2, 2, "row", 0, "bf16"),         # 4096-column down rows, per-row scales
    (8192, 8192, 4, 2, 1, "mix_even_odd", 64, "f32"),  # the column cap (I4MOE_MAX_COLS) on both sides
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: f"D{s[0]}_I{s[1]}_E{s[2]}_K{s[3]}_S{s[4]}_{s[5]}_gs{s[6]}_{s[7]}")
def test_ragged_shapes(shape):
    D, I, E, K, S, formats, gs, xd = shape
    print(f"[parity] ragged {shape}", flush=True)
    cfg = get_config("tiny", D=D, I=I, E=E, K=K, S=S, formats=formats, gs=gs, x_dtype=xd, topp=0.9,
                     routed_scale=2.5, seed=100 + D + I)
    full_layer_check(cfg)


DEGENERATE = {
    # one expert, top-1, one token: the fused selection over a single score (with norm on, the
    # layer is routed_scale * y, the oracle's closed-form pin)
    "one_expert": dict(D=256, I=128, E=1, K=1, S=1, formats="row", gs=0, x_dtype="f32", topp=0.0),
    # K = E: every expert for every token, entries of S rows
    "k_equals_e": dict(D=512, I=256, E=8, K=8, S=2, formats="group", gs=64, x_dtype="bf16", topp=0.0),
    # top-p near zero: one expert kept per token
    "topp_keeps_one": dict(D=512, I=256, E=16, K=4, S=3, formats="mix_even_odd", gs=64, x_dtype="f32", topp=1e-6),
}


@pytest.mark.parametrize("name", sorted(DEGENERATE))
def test_degenerate_layers(name):
    print(f"[parity] degenerate {name}", flush=True)
    cfg = get_config("tiny", routed_scale=2.5, seed=300, **DEGENERATE[name])
    full_layer_check(cfg)


def test_zero_activation_row():
    """One token's activations all zero: its row exponent takes the zero-row value, its expert
    rows are exactly zero (silu(0) * 0), and the router ranks it by the bias alone; the other
    tokens as usual."""
    print("[parity] zero activation row", flush=True)
    cfg = get_config("tiny", D=1024, I=512, E=8, K=2, S=3, formats="mix_even_odd", gs=64, x_dtype="f32", seed=301)

    def zero_row(L):
        L.x[1, :] = 0.0

    full_layer_check(cfg, mutate=zero_row)


def test_determinism_medium():
    import torch
    print("[parity] determinism medium x10", flush=True)
    cfg = get_config("medium")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    seen = set()
    for _ in range(10):
        r = torch.from_numpy(L.residual.copy()).to("cuda:0")
        rec = ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
        ctx.issue(0, x)
        ctx.take(r)
        torch.cuda.synchronize()
        seen.add(digest(r.cpu().numpy(), np.frombuffer(bytes(rec), dtype=np.uint8)))
    assert len(seen) == 1
    ctx.close()


def test_explicit_group_matches_device_route():
    import torch
    print("[parity] explicit group vs device route", flush=True)
    cfg = get_config("mix", E=16, layers=1)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    rec = ctx.route(0, x, cfg.K, 0.0, True, 1.0, host_out=True)
    ctx.issue(0, x)
    a = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(a)
    rows = [(rec[0].idx[k], 0, rec[0].w[k]) for k in range(rec[0].n)]
    ctx.issue(0, x, rows=rows)
    b = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(b)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())
    # two issues (slots) of the same experts split in halves: take sums slots in issue order
    h1, h2 = rows[: len(rows) // 2], rows[len(rows) // 2:]
    ctx.issue(0, x, rows=h1)
    ctx.issue(0, x, rows=h2)
    c = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(c)
    ctx.issue(0, x, rows=h1)
    p1 = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(p1)
    ctx.issue(0, x, rows=h2)
    p2 = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(p2)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy(), (p1.cpu().numpy() + p2.cpu().numpy()).astype(np.float32))
    routes, x64 = oracle_routes(cfg, L, topp=0.0, scale=1.0)
    delta, _ = oracle.experts.layer_delta(routes, L.expert, x64)
    assert normwise_err(c.cpu().numpy(), delta) < TOL
    ctx.close()


def test_g4_page_design_50x3():
    """50 trials x 3 experts in one launch: gs=64, a 200 % 64 tail group, and a per-row member."""
    import torch
    print("[parity] g4 50x3", flush=True)
    rng = np.random.default_rng(4242)
    D, I = 256, 200
    ctx = new_ctx()
    from harness import host_tensor
    for trial in range(50):
        ex = {}
        for e, (fmt, gs) in enumerate([(4, 64), (4, 64), (2, 0)]):
            def t(O, C_):
                ng = -(-C_ // gs) if gs else 1
                return host_tensor(fmt, gs, O, C_, rng.integers(0, 256, (O, C_ // 2), dtype=np.uint8),
                                   rng.lognormal(np.log(0.01), 0.5, O * ng).astype(np.float32))
            ex[e] = type("E", (), {})()
            ex[e].gate, ex[e].up, ex[e].down = t(I, D), t(I, D), t(D, I)
            hs = [ctx.upload_host_tensor(ex[e].gate), ctx.upload_host_tensor(ex[e].up), ctx.upload_host_tensor(ex[e].down)]
            ctx.set_expert(trial, e, *hs)
        S = int(rng.integers(1, 4))
        xs = rng.standard_normal((S, D)).astype(np.float32)
        rows = [(e, t_, float(rng.uniform(0.1, 1.0))) for t_ in range(S) for e in range(3)]
        x = torch.from_numpy(xs).to("cuda:0")
        ctx.issue(trial, x, rows=rows)
        out = torch.zeros((S, D), dtype=torch.float32, device="cuda:0")
        ctx.take(out)
        torch.cuda.synchronize()
        ref = np.zeros((S, D))
        for (e, t_, w) in rows:
            y = oracle.expert_forward(ex[e].gate, ex[e].up, ex[e].down, xs[t_].astype(np.float64))[3]
            ref[t_] += float(np.float32(w)) * y
        assert normwise_err(out.cpu().numpy(), ref) < TOL, trial
    ctx.close()


def test_router_page_design_200_trials():
    """200 random router trials mixing top-p, norm_topk and routed_scale; selections and weights
    must equal the oracle's bit for bit away from near-ties, and always equal the oracle's
    selection taken on the GPU's own logits."""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print("[parity] router 200 trials", flush=True)
    rng = np.random.default_rng(2024)
    ctx = new_ctx()
    mism = ties = 0
    for trial in range(200):
        E = int(rng.choice([8, 64, 256]))
        D = int(rng.choice([256, 512, 1536]))
        S = int(rng.integers(1, 5))
        K = int(rng.integers(1, min(E, 64 // S, 16) + 1))
        W = rng.normal(0, float(rng.choice([0.02, 0.1])), (E, D)).astype(np.float32)
        b = rng.normal(0, 0.1, E).astype(np.float32)
        xs = rng.standard_normal((S, D)).astype(np.float32)
        topp = float(rng.choice([0.0, 0.5, 0.8, 0.95, 1.0]))
        norm = bool(rng.integers(0, 2))
        scale = float(rng.choice([1.0, 2.5, 0.5]))
        bf = bool(rng.integers(0, 2))
        if bf:
            from synth import round_f32_to_bf16_bits
            xbits = round_f32_to_bf16_bits(xs)
            x = x_to_device(xbits, "bf16")
            x64 = oracle.widen_activations(xbits, "bf16")
        else:
            x = x_to_device(xs, "f32")
            x64 = xs.astype(np.float64)
        ctx.upload_router(0, W, b)
        rec = ctx.route(0, x, K, topp, norm, scale, host_out=True)
        logits = ctx.tap(B.I4MOE_TAP_LOGITS, 0, np.float64).reshape(S, E)
        routes = oracle.route(W, b, x64, K, topp, norm, scale)
        for t in range(S):
            # R2: oracle selection on the GPU's logits
            r2 = oracle.route_token(logits[t], b, K, topp, norm, scale)
            assert route_matches(rec[t], r2, K) or near_tie(r2, K, topp), (trial, t)
            if near_tie(routes[t], K, topp):
                ties += 1
                continue
            if not route_matches(rec[t], routes[t], K):
                mism += 1
    print(f"[parity] router trials: {mism} mismatches, {ties} near-tie tokens", flush=True)
    assert mism == 0
    ctx.close()


def test_router_exact_ties_take_lower_index():
    import torch
    ctx = new_ctx()
    E, D = 16, 256
    rng = np.random.default_rng(7)
    W = rng.normal(0, 0.05, (E, D)).astype(np.float32)
    W[9] = W[3]
    W[12] = W[3]
    b = np.zeros(E, np.float32)
    W[5] = W[3] * 0  # logit 0 exactly; sigma 0.5
    x = torch.from_numpy(rng.standard_normal((1, D)).astype(np.float32)).to("cuda:0")
    ctx.upload_router(0, W, b)
    rec = ctx.route(0, x, E, 0.0, False, 1.0, host_out=True)
    idx = list(rec[0].idx[:E])
    assert sorted(idx) == list(range(E))
    pos = {e: idx.index(e) for e in (3, 9, 12)}
    assert pos[3] < pos[9] < pos[12] and pos[12] - pos[3] == 2
    ctx.close()


@pytest.mark.parametrize("E,S", [(230, 1), (230, 3), (130, 2), (300, 2), (512, 4), (1000, 1)])
def test_router_exact_ties_many_experts(E, S):
    """E > 64 takes the K-rounds selection (2, 4, 8 or 16 experts per lane): exact ties between
    experts held by one lane in different columns (3, 67, 131, 259, 451, 963) and by different
    lanes (9, 200, 457, 999) still go to the lower index, for every token.  A bias lifts both
    groups to the top of the order so the ties are decided inside the selection."""
    import torch
    print(f"[parity] exact ties E={E} S={S}", flush=True)
    ctx = new_ctx()
    D = 256
    rng = np.random.default_rng(11 + E)
    W = rng.normal(0, 0.05, (E, D)).astype(np.float32)
    b = np.zeros(E, np.float32)
    groups = [[e for e in (3, 67, 131, 259, 451, 963) if e < E], [e for e in (9, 200, 457, 999) if e < E]]
    for lift, group in zip((1.0, 0.5), groups):
        for e in group:
            W[e] = W[group[0]]
            b[e] = lift
    xs = rng.standard_normal((S, D)).astype(np.float32)
    x = torch.from_numpy(xs).to("cuda:0")
    ctx.upload_router(0, W, b)
    K = 64 // S
    rec = ctx.route(0, x, K, 0.0, False, 1.0, host_out=True)
    routes = oracle.route(W, b, xs.astype(np.float64), K, 0.0, False, 1.0)
    for t in range(S):
        idx = list(rec[t].idx[:K])
        assert idx == list(routes[t].idx), (t, idx, list(routes[t].idx))
        for group in groups:
            at = [idx.index(e) for e in group if e in idx]
            assert len(at) == min(len(group), K) and at == sorted(at)
    ctx.close()


@pytest.mark.parametrize("E", [65, 127, 128, 129, 257, 640])
def test_router_column_edges(E):
    """Expert counts at the edges of the K-rounds variants (2, 4 and 8 experts per lane, with a
    lane's last column holding one real expert or none): every token's selection and weights
    equal the oracle's away from near-ties, and lanes past E are never chosen."""
    print(f"[parity] router column edges E={E}", flush=True)
    ctx = new_ctx()
    D, S, K = 256, 3, 8
    rng = np.random.default_rng(500 + E)
    W = rng.normal(0, 0.05, (E, D)).astype(np.float32)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    b[E - 1] = 2.0  # the last expert (alone in its column for E = 65, 129, 257) leads every token
    xs = rng.standard_normal((S, D)).astype(np.float32)
    x = x_to_device(xs, "f32")
    ctx.upload_router(0, W, b)
    rec = ctx.route(0, x, K, 0.9, True, 2.5, host_out=True)
    routes = oracle.route(W, b, xs.astype(np.float64), K, 0.9, True, 2.5)
    checked = 0
    for t in range(S):
        idx = list(rec[t].idx[:K])
        assert all(0 <= e < E for e in idx) and idx[0] == E - 1, (t, idx)
        if near_tie(routes[t], K, 0.9):
            continue
        assert route_matches(rec[t], routes[t], K), (t, idx, routes[t].idx)
        checked += 1
    assert checked >= 2
    ctx.close()


@pytest.mark.parametrize("S,K", [(1, 8), (4, 16), (16, 4), (64, 1)])
def test_router_max_experts(S, K):
    """The 1024-expert cap: 16 experts per lane in the K-rounds selection and the largest
    score staging (four tokens of 1024 experts per pass)."""
    print(f"[parity] router E=1024 S={S} K={K}", flush=True)
    ctx = new_ctx()
    E, D = 1024, 512
    rng = np.random.default_rng(31 + S)
    W = rng.normal(0, 0.05, (E, D)).astype(np.float32)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    xs = rng.standard_normal((S, D)).astype(np.float32)
    x = x_to_device(xs, "f32")
    ctx.upload_router(0, W, b)
    rec = ctx.route(0, x, K, 0.9, True, 2.5, host_out=True)
    routes = oracle.route(W, b, xs.astype(np.float64), K, 0.9, True, 2.5)
    checked = 0
    for t in range(S):
        if near_tie(routes[t], K, 0.9):
            continue
        assert route_matches(rec[t], routes[t], K), t
        checked += 1
    assert checked >= S // 2
    ctx.close()
