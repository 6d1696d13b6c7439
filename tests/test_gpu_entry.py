"""Several rows of one expert in one issue (S > 1): rows of an entry sharing weight passes in the
vector kernels, and entries of many rows on the matrix cores.  Explicit groups with
entries of 1 to 28 rows (listed out of order, so the library's expert-major row order is
exercised, and with repeated tokens inside an entry), checked row by row against the f64 oracle
(every h row and every y row, through the taps) and as a layer delta after the take, with pass
sharing forced on and the matrix cores on and off; every run repeated for bitwise determinism.
A device route at S = 64, K = 1 over 4 experts (about 16 rows each) is checked as a layer, and
entries at the column cap (D = I = 8192) and with all-zero activation rows, on the matrix cores
and on the vector kernels."""

from __future__ import annotations

import concurrent.futures as cf

import numpy as np
import pytest

import oracle
from harness import TOL, WORKERS, make_layer, normwise_err, upload_layer, x_to_device
from synth import get_config
from synth.gen import gen_expert

pytestmark = pytest.mark.gpu

# (base workload, overrides, tokens S, rows per entry); the dual spans 2 passes in every case,
# and the down projection runs short rows (16 lanes per row) or long rows
CASES = {
    # mixed g64 / per-row experts, f32 x, a 16-wide tail group in the down rows (I = 2000)
    "mix_short_down": ("mix", dict(D=2560, I=2000, E=16), 16, [1, 2, 3, 4, 5, 9, 16, 7]),
    # g64 experts, bf16 x
    "group_bf16": ("small_batch", dict(D=3072, I=1024, E=12), 8, [8, 1, 6, 4, 2, 3]),
    # down rows past 2048 columns (one wave per row), and an entry longer than S (repeated tokens)
    "mix_long_down": ("mix", dict(D=1024, I=2304, E=8), 4, [6, 4, 1, 3]),
    # every entry on the matrix cores (64 rows, 3 experts), bf16 x, g64
    "mfma_only": ("small_batch", dict(D=3072, I=1024, E=12), 64, [16, 20, 28]),
    # matrix-core entries beside vector entries in one issue; f32 x, g64 and per-row experts,
    # the down rows' 16-wide tail group
    "mfma_mixed": ("mix", dict(D=2560, I=2000, E=16), 48, [17, 5, 3, 1, 2, 16, 20]),
    # per-row experts only: the matrix cores keep each digit's sums in int32 over a slice; f32 x,
    # down rows of 2000 columns (not a multiple of 64), a vector entry beside them
    "mfma_row": ("medium", dict(D=2560, I=2000, E=12, x_dtype="f32"), 48, [17, 5, 16, 24]),
}


def make_rows(rng, S, sizes, E):
    experts = rng.permutation(E)[: len(sizes)]
    rows = []
    for e, n in zip(experts, sizes):
        toks = rng.permutation(S)[:n] if n <= S else rng.integers(0, S, n)
        rows += [(int(e), int(t), float(rng.uniform(0.05, 1.0))) for t in toks]
    order = rng.permutation(len(rows))
    return [rows[i] for i in order]


def expert_major(rows):
    """The library's row order: experts in first-appearance order, listed order inside each."""
    firsts = []
    for e, _, _ in rows:
        if e not in firsts:
            firsts.append(e)
    return [r for e in firsts for r in rows if r[0] == e]


@pytest.mark.parametrize("mfma", ["16", "0"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_entry_rows_match_oracle(case, mfma, monkeypatch):
    import torch
    from int4_grouped_expert_router_amd import Context
    from int4_grouped_expert_router_amd import binding as B
    base, over, S, sizes = CASES[case]
    if mfma == "16" and max(sizes) < 16:
        pytest.skip("no entry reaches the matrix-core row count")
    print(f"[entry] {case}: S={S} entries={sizes} mfma_min={mfma}", flush=True)
    cfg = get_config(base, S=S, layers=1, **over)
    L = make_layer(cfg, 0)
    rng = np.random.default_rng(sum(sizes) * 1000 + S)
    rows = make_rows(rng, S, sizes, cfg.E)
    assert len(rows) <= 64
    monkeypatch.setenv("I4MOE_MFMA_MIN_ROWS", mfma)
    monkeypatch.setenv("I4MOE_ENTRY_ROWS", "4")  # pass sharing for every entry the vector kernels run
    ctx = Context(0, torch.cuda.current_stream())
    monkeypatch.delenv("I4MOE_MFMA_MIN_ROWS")
    monkeypatch.delenv("I4MOE_ENTRY_ROWS")
    upload_layer(ctx, L, 0, experts=sorted({r[0] for r in rows}))
    x = x_to_device(L.x, L.x_dtype)
    outs, hs, ys = [], [], []
    for _ in range(2):
        slot = ctx.issue(0, x, rows=rows)
        hs.append(ctx.tap(B.I4MOE_TAP_H).reshape(-1, cfg.I)[: len(rows)].copy())
        ys.append(ctx.tap(B.I4MOE_TAP_Y, slot).reshape(-1, cfg.D)[: len(rows)].copy())
        out = torch.zeros((S, cfg.D), dtype=torch.float32, device="cuda:0")
        ctx.take(out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    ctx.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(hs[0], hs[1]) and np.array_equal(ys[0], ys[1])

    x64 = oracle.widen_activations(L.x, L.x_dtype)
    ordered = expert_major(rows)
    ws = {e: gen_expert(cfg, 0, e) for e in {r[0] for r in rows}}
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        fw = list(ex.map(lambda r: oracle.expert_forward(ws[r[0]].gate, ws[r[0]].up, ws[r[0]].down, x64[r[1]]),
                         ordered))
    for i, (r, (_, _, h, y)) in enumerate(zip(ordered, fw)):
        assert normwise_err(hs[0][i], h) < TOL, (case, i, r, "h")
        # y from the oracle's own h (x -> h -> y), so a wrong h row cannot hide in y
        assert normwise_err(ys[0][i], y) < TOL, (case, i, r, "y")
    ref = np.zeros((S, cfg.D))
    for r, (_, _, _, y) in zip(ordered, fw):
        ref[r[1]] += float(np.float32(r[2])) * y
    for t in range(S):
        if np.any(ref[t]):
            assert normwise_err(outs[0][t], ref[t]) < TOL, (case, t)
        else:
            assert not np.any(outs[0][t])
    print(f"[entry] {case}: {len(rows)} rows ok", flush=True)


def test_device_route_many_rows_per_expert():
    """S = 64 tokens, K = 1 of E = 4 experts: the device route gives every expert about 16 rows,
    so the issue mixes matrix-core and vector entries; the layer matches the oracle (the experts
    checked on the GPU's own route, after the route itself is checked away from near-ties)."""
    import torch
    from harness import gpu_routes, layer_delta_threads, near_tie, oracle_routes, route_matches, run_layer
    from int4_grouped_expert_router_amd import Context
    print("[entry] device route S=64 K=1 E=4", flush=True)
    cfg = get_config("mix", D=2048, I=1024, E=4, K=1, S=64, layers=1)
    L = make_layer(cfg, 0)
    ctx = Context(0, torch.cuda.current_stream())
    upload_layer(ctx, L, 0)
    rec, out, _ = run_layer(ctx, cfg, L, 0)
    rec2, out2, _ = run_layer(ctx, cfg, L, 0)
    ctx.close()
    assert np.array_equal(out, out2)
    routes, x64 = oracle_routes(cfg, L)
    counts = np.bincount([int(r.idx[0]) for r in routes], minlength=cfg.E)
    print(f"[entry] rows per expert {counts.tolist()}", flush=True)
    assert counts.max() >= 16
    for t in range(cfg.S):
        assert route_matches(rec[t], routes[t], cfg.K) or near_tie(routes[t], cfg.K, cfg.topp), t
    delta, _ = layer_delta_threads(gpu_routes(rec, cfg.S, cfg.K), L.expert, x64)
    for t in range(cfg.S):
        assert normwise_err(out[t], delta[t]) < TOL, t


def check_entries_batched(cfg, L, S, sizes, mfma, monkeypatch, seed):
    """Explicit entries of the given sizes, the matrix cores from `mfma` rows (0: off): every h
    and y row and the layer delta against the oracle run one expert at a time (its rows as the
    columns of one matrix), twice for bitwise determinism."""
    import torch
    from int4_grouped_expert_router_amd import Context
    from int4_grouped_expert_router_amd import binding as B
    rng = np.random.default_rng(seed)
    rows = make_rows(rng, S, sizes, cfg.E)
    monkeypatch.setenv("I4MOE_MFMA_MIN_ROWS", mfma)
    ctx = Context(0, torch.cuda.current_stream())
    monkeypatch.delenv("I4MOE_MFMA_MIN_ROWS")
    upload_layer(ctx, L, 0, experts=sorted({r[0] for r in rows}))
    x = x_to_device(L.x, L.x_dtype)
    outs, hs, ys = [], [], []
    for _ in range(2):
        slot = ctx.issue(0, x, rows=rows)
        hs.append(ctx.tap(B.I4MOE_TAP_H).reshape(-1, cfg.I)[: len(rows)].copy())
        ys.append(ctx.tap(B.I4MOE_TAP_Y, slot).reshape(-1, cfg.D)[: len(rows)].copy())
        out = torch.zeros((S, cfg.D), dtype=torch.float32, device="cuda:0")
        ctx.take(out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    ctx.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(hs[0], hs[1]) and np.array_equal(ys[0], ys[1])
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    ordered = expert_major(rows)
    ref_h, ref_y = {}, {}
    for e in sorted({r[0] for r in rows}):
        ew = gen_expert(cfg, 0, e)
        idx = [i for i, r in enumerate(ordered) if r[0] == e]
        _, _, h, y = oracle.expert_forward(ew.gate, ew.up, ew.down, x64[[ordered[i][1] for i in idx]].T)
        for j, i in enumerate(idx):
            ref_h[i], ref_y[i] = h[:, j], y[:, j]
    for i, r in enumerate(ordered):
        assert normwise_err(hs[0][i], ref_h[i]) < TOL, (i, r, "h")
        assert normwise_err(ys[0][i], ref_y[i]) < TOL, (i, r, "y")
    ref = np.zeros((S, cfg.D))
    for i, r in enumerate(ordered):
        ref[r[1]] += float(np.float32(r[2])) * ref_y[i]
    for t in range(S):
        if np.any(ref[t]):
            assert normwise_err(outs[0][t], ref[t]) < TOL, t
        else:
            assert not np.any(outs[0][t]), t
    return rows, hs[0], ys[0], ordered


@pytest.mark.parametrize("mfma", ["8", "0"])
def test_entries_at_column_cap(mfma, monkeypatch):
    """D = I = 8192 (the column cap on both projections), group-wise g64 experts with f32 x: two
    entries of 12 and 9 rows on the matrix cores (or on the vector kernels), every h and y row
    and the layer delta against the oracle, run twice for bitwise determinism."""
    S, sizes = 16, [12, 9]
    print(f"[entry] column cap D=I=8192 S={S} entries={sizes} mfma_min={mfma}", flush=True)
    cfg = get_config("small_batch", D=8192, I=8192, E=4, S=S, layers=1, x_dtype="f32")
    L = make_layer(cfg, 0)
    rows, _, _, _ = check_entries_batched(cfg, L, S, sizes, mfma, monkeypatch, 8192)
    print(f"[entry] column cap: {len(rows)} rows ok", flush=True)


@pytest.mark.parametrize("mfma", ["8", "0"])
def test_entries_with_zero_activation_rows(mfma, monkeypatch):
    """Two tokens' activations all zero inside matrix-core entries (bf16 x and f32 x): their
    digit rows and exponents take the zero-row values and their h and y rows are exactly zero;
    the other rows against the oracle."""
    S, sizes = 16, [10, 14]
    for xd in ("bf16", "f32"):
        print(f"[entry] zero activation rows x={xd} mfma_min={mfma}", flush=True)
        cfg = get_config("small_batch", D=2048, I=1024, E=6, S=S, layers=1, x_dtype=xd)
        L = make_layer(cfg, 0)
        L.x[[2, 9], :] = 0
        rows, h, y, ordered = check_entries_batched(cfg, L, S, sizes, mfma, monkeypatch, 16)
        zero = [i for i, r in enumerate(ordered) if r[1] in (2, 9)]
        assert zero and not np.any(h[zero]) and not np.any(y[zero])
