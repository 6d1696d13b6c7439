"""The CPU tier through the C ABI: experts kept on the host run on the CPU while the device
group runs on the GPU, and the take joins both.  Checked against the f64 oracle on the GPU's own
route (mixed tiers, all on the host, bf16 and f32 activations, per-row / group-wise / tail
groups, device entries on the matrix cores), bitwise against the plain explicit issue when every
expert is on the device, bitwise run to run, and on its error path."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from harness import TOL, gpu_routes, layer_delta_threads, make_layer, normwise_err, x_to_device
from synth import get_config
from synth.gen import gen_expert

pytestmark = pytest.mark.gpu

CASES = {
    # f32 x, even experts g64 and odd per-row, a 16-wide tail group in the down rows
    "mix_f32": ("mix", dict(D=2048, I=2000, E=16, K=6, S=3)),
    # bf16 x, g64 experts
    "group_bf16": ("small_batch", dict(D=3072, I=1024, E=16, K=8, S=4)),
    # 16 tokens over 4 experts (about 8 rows each): device entries on the matrix cores beside the
    # host rows
    "many_rows": ("mix", dict(D=2048, I=1024, E=4, K=2, S=16)),
}


def new_ctx():
    import torch
    from int4_grouped_expert_router_amd import Context
    return Context(0, torch.cuda.current_stream())


def bind(ctx, cfg, L, on_host):
    ctx.upload_router(0, L.router_W, L.router_b)
    for e in range(cfg.E):
        ew = gen_expert(cfg, 0, e)
        if e in on_host:
            ctx.set_host_expert(0, e, ew.gate, ew.up, ew.down)
        else:
            ctx.set_expert(0, e, ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up),
                           ctx.upload_host_tensor(ew.down))


def run_tiered(ctx, cfg, L, x):
    import torch
    rec = ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    n, times = ctx.tiered_issue(0, x, list(rec))
    out = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(out)
    torch.cuda.synchronize()
    return rec, n, times, out.cpu().numpy()


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("split", ["odd_on_host", "all_on_host"])
def test_tiered_matches_oracle(case, split, monkeypatch):
    base, over = CASES[case]
    cfg = get_config(base, layers=1, **over)
    print(f"[tier] {case} {split}", flush=True)
    L = make_layer(cfg, 0)
    on_host = set(range(cfg.E)) if split == "all_on_host" else set(range(1, cfg.E, 2))
    if case == "many_rows":
        monkeypatch.setenv("I4MOE_MFMA_MIN_ROWS", "4")  # every device entry of 4+ rows on the matrix cores
    ctx = new_ctx()
    monkeypatch.delenv("I4MOE_MFMA_MIN_ROWS", raising=False)
    bind(ctx, cfg, L, on_host)
    x = x_to_device(L.x, L.x_dtype)
    rec, n, times, out = run_tiered(ctx, cfg, L, x)
    from int4_grouped_expert_router_amd import binding as B
    ctx.set_profiling(True)
    _, n2, _, out2 = run_tiered(ctx, cfg, L, x)
    mfma_launches = ctx.profile(B.I4MOE_K_MFMA)[1]
    ctx.set_profiling(False)
    ctx.close()
    if case == "many_rows" and split == "odd_on_host":
        assert mfma_launches > 0  # the device entries ran on the matrix cores
    assert np.array_equal(out, out2)  # bitwise run to run
    routes = gpu_routes(rec, cfg.S, cfg.K)
    pairs = [(t, routes[t].idx[k]) for t in range(cfg.S) for k in range(routes[t].n)]
    n_host = sum(1 for _, e in pairs if e in on_host)
    assert times.host_rows == n_host and times.device_rows == len(pairs) - n_host
    assert n == n2 == (1 if n_host else 0) + (1 if n_host < len(pairs) else 0)
    assert times.cpu_ms > 0.0 if n_host else times.cpu_ms == 0.0
    print(f"[tier] {case} {split}: device rows {times.device_rows}, host rows {times.host_rows}, "
          f"issue {times.issue_ms:.2f} ms, x wait {times.x_wait_ms:.2f} ms, cpu {times.cpu_ms:.2f} ms", flush=True)
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    delta, _ = layer_delta_threads(routes, lambda e: gen_expert(cfg, 0, e), x64)
    for t in range(cfg.S):
        assert normwise_err(out[t], delta[t]) < TOL, (case, split, t)


def test_tiered_all_device_equals_explicit_issue():
    """With every expert on the device the tiered issue is one explicit group in route order:
    the same bits as i4moe_expert_group_issue with those rows."""
    import torch
    cfg = get_config("mix", D=2048, I=2000, E=16, K=6, S=3, layers=1)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    bind(ctx, cfg, L, set())
    x = x_to_device(L.x, L.x_dtype)
    rec, n, times, out = run_tiered(ctx, cfg, L, x)
    assert n == 1 and times.host_rows == 0
    rows = [(rec[t].idx[k], t, rec[t].w[k]) for t in range(cfg.S) for k in range(rec[t].n)]
    ctx.issue(0, x, rows=rows)
    ref = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(ref)
    torch.cuda.synchronize()
    ctx.close()
    assert np.array_equal(out, ref.cpu().numpy())


def test_tiered_errors_leave_nothing_pending():
    """An expert that is neither on the device nor on the host, or a bad argument, is refused
    with EINVAL; the take that follows is a no-op and the context stays usable."""
    import torch
    from int4_grouped_expert_router_amd import I4moeError
    from int4_grouped_expert_router_amd import binding as B
    cfg = get_config("mix", D=512, I=256, E=8, K=2, S=2, layers=1)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    ctx.upload_router(0, L.router_W, L.router_b)
    for e in range(cfg.E - 1):  # the last expert is bound nowhere
        ew = gen_expert(cfg, 0, e)
        if e % 2:
            ctx.set_host_expert(0, e, ew.gate, ew.up, ew.down)
        else:
            ctx.set_expert(0, e, ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up),
                           ctx.upload_host_tensor(ew.down))
    x = x_to_device(L.x, L.x_dtype)
    routes = [B.i4moe_route_host() for _ in range(cfg.S)]
    for t in range(cfg.S):
        routes[t].n = 2
        routes[t].idx[0], routes[t].idx[1] = 0, cfg.E - 1
        routes[t].w[0], routes[t].w[1] = 0.5, 0.5
    with pytest.raises(I4moeError) as ei:
        ctx.tiered_issue(0, x, routes)
    assert ei.value.code == B.I4MOE_EINVAL
    routes[0].n = B.I4MOE_MAX_K + 1
    with pytest.raises(I4moeError):
        ctx.tiered_issue(0, x, routes)
    resid = torch.ones((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(resid)  # nothing pending: a no-op
    torch.cuda.synchronize()
    assert np.array_equal(resid.cpu().numpy(), np.ones((cfg.S, cfg.D), np.float32))
    # still usable: a valid split runs
    for t in range(cfg.S):
        routes[t].n = 2
        routes[t].idx[0], routes[t].idx[1] = 0, 1
    n, times = ctx.tiered_issue(0, x, routes)
    assert n == 2 and times.host_rows == cfg.S and times.device_rows == cfg.S
    out = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(out)
    torch.cuda.synchronize()
    ctx.close()
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    from types import SimpleNamespace
    rs = [SimpleNamespace(n=2, idx=[0, 1], w32=np.array([0.5, 0.5], np.float32)) for _ in range(cfg.S)]
    delta, _ = layer_delta_threads(rs, lambda e: gen_expert(cfg, 0, e), x64)
    for t in range(cfg.S):
        assert normwise_err(out.cpu().numpy()[t], delta[t]) < TOL


def test_tiered_host_paths(monkeypatch):
    """The CPU rows of a tiered issue on each host path: the integer path at 512 and at 256 bits
    give the same bits, and the float32 path (I4MOE_HOST_INT=0) is within the bar of the oracle."""
    from int4_grouped_expert_router_amd import binding as B
    base, over = CASES["mix_f32"]
    cfg = get_config(base, layers=1, **over)
    L = make_layer(cfg, 0)
    on_host = set(range(1, cfg.E, 2))
    ctx = new_ctx()
    bind(ctx, cfg, L, on_host)
    x = x_to_device(L.x, L.x_dtype)
    outs = {}
    for path in ("default", "256", "0"):
        print(f"[tier] host path {path}", flush=True)
        if path == "default":
            monkeypatch.delenv("I4MOE_HOST_INT", raising=False)
        else:
            monkeypatch.setenv("I4MOE_HOST_INT", path)
        rec, n, times, outs[path] = run_tiered(ctx, cfg, L, x)
        assert times.host_rows > 0
    monkeypatch.delenv("I4MOE_HOST_INT", raising=False)
    ctx.close()
    if B.i4moe_host_int_path():
        assert np.array_equal(outs["default"], outs["256"])
    routes = gpu_routes(rec, cfg.S, cfg.K)
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    delta, _ = layer_delta_threads(routes, lambda e: gen_expert(cfg, 0, e), x64)
    for path, out in outs.items():
        for t in range(cfg.S):
            assert normwise_err(out[t], delta[t]) < TOL, (path, t)
