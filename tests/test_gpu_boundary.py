"""The C ABI's contracts on the GPU: argument errors are rejected on the host with nothing
enqueued and leave the context healthy, host buffers are free after an upload returns, tensor
handles recycle, the fail-after hook gates compute calls only, a failed take poisons the
context, and up to the slot limit of issues reduce in issue order.  Every failure here is
forced from the host; no kernel is ever launched on bad input."""

from __future__ import annotations

import ctypes as C
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from harness import TOL, make_layer, normwise_err, oracle_routes, upload_layer, x_to_device
from synth import get_config

pytestmark = pytest.mark.gpu


def new_ctx():
    import torch
    from int4_grouped_expert_router_amd import Context
    assert torch.cuda.is_available()
    return Context(0, torch.cuda.current_stream())


def tiny_delta(ctx, cfg, L, x, layer=0):
    """route + issue + take into zeros; returns the f32 delta on the host."""
    import torch
    ctx.route(layer, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(layer, x)
    z = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(z)
    torch.cuda.synchronize()
    return z.cpu().numpy()


def oracle_delta(cfg, L):
    routes, x64 = oracle_routes(cfg, L)
    delta, _ = oracle.experts.layer_delta(routes, L.expert, x64)
    return delta


def raw_upload(ctx, fmt, gs, O, C_, packed, scales):
    from int4_grouped_expert_router_amd import binding as B
    return B.i4moe_upload_expert_tensor(ctx.p, fmt, gs, O, C_, packed.ctypes.data_as(C.c_void_p),
                                        scales.ctypes.data_as(C.c_void_p))


def test_bad_uploads_rejected_then_healthy():
    print("[boundary] bad uploads", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    q = np.full((8, 32), 0x88, np.uint8)
    s = np.ones(8 * 64, np.float32)
    cases = [
        (3, 0, 8, 64, "unsupported"),      # no other format codes
        (1, 0, 8, 64, "unsupported"),
        (4, 3, 8, 64, "even"),            # odd group size
        (4, -2, 8, 64, "even"),
        (2, 64, 8, 64, "per-row"),        # per-row tensors take gs = 0
        (2, 0, 8, 63, "even"),            # odd C
        (2, 0, 0, 64, "shape"),
        (2, 0, 8, 8194, "exceeds"),
    ]
    for fmt, gs, O, C_, word in cases:
        assert raw_upload(ctx, fmt, gs, O, C_, q, s) == 0, (fmt, gs, O, C_)
        assert word in ctx.last_error(), (fmt, gs, O, C_, ctx.last_error())
    # a NaN router is refused; the layer stays unrouted until a finite one arrives
    bad = L.router_W.copy()
    bad[1, 2] = np.nan
    with pytest.raises(Exception):
        ctx.upload_router(0, bad, L.router_b)
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    assert normwise_err(tiny_delta(ctx, cfg, L, x), oracle_delta(cfg, L)) < TOL
    ctx.close()


def test_bad_compute_arguments_enqueue_nothing():
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print("[boundary] bad compute arguments", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    xp = C.c_void_p(x.data_ptr())
    p = ctx.p
    f = C.c_float
    assert B.i4moe_route(p, 0, xp, 0, 1, cfg.E + 1, f(0), 1, f(1), None) == B.I4MOE_EINVAL      # K > E
    assert B.i4moe_route(p, 0, xp, 0, 1, 0, f(0), 1, f(1), None) == B.I4MOE_EINVAL             # K = 0
    assert B.i4moe_route(p, 0, xp, 7, 1, 2, f(0), 1, f(1), None) == B.I4MOE_EINVAL             # dtype
    assert B.i4moe_route(p, 0, xp, 0, 65, 1, f(0), 1, f(1), None) == B.I4MOE_EINVAL            # S > 64
    assert B.i4moe_route(p, 0, xp, 0, 1, 2, f(float("nan")), 1, f(1), None) == B.I4MOE_EINVAL  # topp
    assert B.i4moe_route(p, 5, xp, 0, 1, 2, f(0), 1, f(1), None) == B.I4MOE_EINVAL             # no router
    assert B.i4moe_route(p, 0, None, 0, 1, 2, f(0), 1, f(1), None) == B.I4MOE_EINVAL           # NULL x
    # issue before any route of the layer, and explicit groups with bad rows
    assert B.i4moe_expert_group_issue(p, 0, xp, 0, 1, None) == B.I4MOE_EINVAL
    for ex, tk, wt in [(cfg.E, 0, 1.0), (0, 1, 1.0), (0, 0, float("nan")), (-1, 0, 1.0)]:
        g = B.i4moe_group(1, (C.c_int32 * 1)(ex), (C.c_int32 * 1)(tk), (C.c_float * 1)(wt))
        assert B.i4moe_expert_group_issue(p, 0, xp, 0, 1, C.byref(g)) == B.I4MOE_EINVAL, (ex, tk, wt)
    g = B.i4moe_group(0, (C.c_int32 * 1)(0), (C.c_int32 * 1)(0), (C.c_float * 1)(1.0))
    assert B.i4moe_expert_group_issue(p, 0, xp, 0, 1, C.byref(g)) == B.I4MOE_EINVAL
    # misaligned activations
    xb = torch.zeros(2 * cfg.D + 1, dtype=torch.float32, device="cuda:0")
    assert B.i4moe_expert_group_issue(p, 0, C.c_void_p(xb.data_ptr() + 4), 0, 1, None) == B.I4MOE_EINVAL
    # nothing was enqueued: a take now is a no-op and the context is healthy
    z = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(z)
    torch.cuda.synchronize()
    assert not z.cpu().numpy().any()
    assert normwise_err(tiny_delta(ctx, cfg, L, x), oracle_delta(cfg, L)) < TOL
    ctx.close()


def test_host_buffers_free_after_upload():
    print("[boundary] host buffers scribbled after upload", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    rng = np.random.default_rng(123)
    W, b = L.router_W.copy(), L.router_b.copy()
    ctx.upload_router(0, W, b)
    W[:] = rng.standard_normal(W.shape)
    b[:] = 1e3
    for e in range(cfg.E):
        ew = L.expert(e)
        hs = []
        for t in (ew.gate, ew.up, ew.down):
            q, s = t.packed.copy(), t.scales.copy()
            hs.append(ctx.upload_tensor(t.fmt, t.gs, t.O, t.C, q, s))
            q[:] = rng.integers(0, 256, q.shape, dtype=np.uint8)
            s[:] = -7.0
            del q, s
        ctx.set_expert(0, e, *hs)
    x = x_to_device(L.x, L.x_dtype)
    assert normwise_err(tiny_delta(ctx, cfg, L, x), oracle_delta(cfg, L)) < TOL
    ctx.close()


def test_tensor_handles_recycle():
    print("[boundary] 64 upload/free cycles", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    handles = upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    ref = tiny_delta(ctx, cfg, L, x)
    for i in range(64):
        e = i % cfg.E
        old = handles[e]
        ew = L.expert(e)
        new = tuple(ctx.upload_host_tensor(t) for t in (ew.gate, ew.up, ew.down))
        ctx.set_expert(0, e, *new)
        for h in old:
            ctx.free_tensor(h)
        handles[e] = new
    with pytest.raises(Exception):
        ctx.free_tensor(old[0])           # already freed
    got = tiny_delta(ctx, cfg, L, x)
    assert np.array_equal(got, ref)
    # freeing an expert's tensor unbinds the expert: the device route path refuses the layer
    ctx.free_tensor(handles[0][0])
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    with pytest.raises(Exception):
        ctx.issue(0, x)
    ctx.close()


def test_fail_after_gates_compute_only():
    import torch
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd.runtime import I4moeError
    print("[boundary] fail-after hook", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    ctx.set_fail_after(0)
    upload_layer(ctx, L, 0)                 # uploads are never gated
    x = x_to_device(L.x, L.x_dtype)
    with pytest.raises(I4moeError) as ei:
        ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    assert ei.value.code == B.I4MOE_EINJECTED
    ctx.set_fail_after(-1)                  # a refused route or issue does not poison
    ref = tiny_delta(ctx, cfg, L, x)
    assert normwise_err(ref, oracle_delta(cfg, L)) < TOL
    # route (call 0) and issue (call 1) pass, the take (call 2) is refused: the context is poisoned
    ctx.set_fail_after(2)
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(0, x)
    z = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    with pytest.raises(I4moeError) as ei:
        ctx.take(z)
    assert ei.value.code == B.I4MOE_EINJECTED
    ctx.set_fail_after(-1)
    for call in (lambda: ctx.route(0, x, cfg.K), lambda: ctx.issue(0, x), lambda: ctx.take(z)):
        with pytest.raises(I4moeError) as ei:
            call()
        assert ei.value.code == B.I4MOE_EPOISONED
    torch.cuda.synchronize()
    assert not z.cpu().numpy().any()        # the refused take wrote nothing
    ctx.close()
    # a fresh context on the same device is healthy
    ctx2 = new_ctx()
    upload_layer(ctx2, L, 0)
    assert np.array_equal(tiny_delta(ctx2, cfg, L, x), ref)
    ctx2.close()


def test_sixteen_slots_reduce_in_issue_order():
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print("[boundary] 16 pending issues", flush=True)
    cfg = get_config("mix", D=512, I=256, E=16, K=4, layers=1)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    rng = np.random.default_rng(7)
    groups = []
    for s in range(B.I4MOE_MAX_SLOTS):
        n = int(rng.integers(1, 5))
        ex = rng.choice(cfg.E, n, replace=False)
        groups.append([(int(e), 0, float(np.float32(rng.uniform(0.1, 2.0)))) for e in ex])
    for s, g in enumerate(groups):
        assert ctx.issue(0, x, rows=g) == s
    with pytest.raises(Exception):
        ctx.issue(0, x, rows=groups[0])   # the 17th pending issue is refused
    r0 = np.random.default_rng(8).standard_normal((1, cfg.D)).astype(np.float32)
    r = torch.from_numpy(r0.copy()).to("cuda:0")
    ctx.take(r)
    # each slot alone, then the same f32 sum in issue order on the host
    parts = []
    for g in groups:
        ctx.issue(0, x, rows=g)
        z = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
        ctx.take(z)
        parts.append(z)
    torch.cuda.synchronize()
    total = np.zeros((1, cfg.D), np.float32)
    for z in parts:
        total = (total + z.cpu().numpy()).astype(np.float32)
    assert np.array_equal(r.cpu().numpy(), (r0 + total).astype(np.float32))
    # against the oracle: the sum over all rows of all issues
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    ref = np.zeros(cfg.D)
    for g in groups:
        for e, _, w in g:
            ew = L.expert(e)
            ref += w * oracle.expert_forward(ew.gate, ew.up, ew.down, x64[0])[3]
    assert normwise_err(total, ref[None, :]) < TOL
    ctx.close()


def test_rebinding_an_expert_requires_a_new_route():
    """A device route copies the expert records when it runs, so after set_expert or tensor_free
    the layer's route is stale: the issue is refused (nothing enqueued) until the layer is routed
    again, and the new route runs the new tensors."""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd.runtime import I4moeError
    print("[boundary] stale route after a re-bind", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    handles = upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    rec = ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    e0 = int(rec[0].idx[0])
    # bind expert e0 to a copy of itself with every down scale doubled: its y doubles
    ew = L.expert(e0)
    down2 = SimpleNamespace(fmt=ew.down.fmt, gs=ew.down.gs, O=ew.down.O, C=ew.down.C, packed=ew.down.packed,
                            scales=(2 * ew.down.scales).astype(np.float32))
    new = (ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up), ctx.upload_host_tensor(down2))
    ctx.set_expert(0, e0, *new)
    with pytest.raises(I4moeError) as ei:
        ctx.issue(0, x)
    assert ei.value.code == B.I4MOE_EINVAL and "route" in str(ei.value)
    got = tiny_delta(ctx, cfg, L, x)   # routes again first
    routes, x64 = oracle_routes(cfg, L)
    ref = np.zeros((1, cfg.D))
    for k in range(routes[0].n):
        e = routes[0].idx[k]
        ex = L.expert(e)
        y = oracle.expert_forward(ex.gate, ex.up, down2 if e == e0 else ex.down, x64[0])[3]
        ref[0] += float(routes[0].w32[k]) * y
    assert normwise_err(got, ref) < TOL
    # freeing a bound tensor also leaves the route stale (and the expert unbound)
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.free_tensor(handles[e0][0])      # the old gate: no longer bound, route stays valid
    ctx.issue(0, x)
    z = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(z)
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.free_tensor(new[2])              # bound to e0: the expert is unset, the route is stale
    with pytest.raises(I4moeError) as ei:
        ctx.issue(0, x)
    assert ei.value.code == B.I4MOE_EINVAL
    torch.cuda.synchronize()
    assert np.array_equal(z.cpu().numpy(), got)
    ctx.close()


def test_fail_after_from_environment(monkeypatch):
    """I4MOE_FAIL_AFTER=N set when the context is created: N compute calls pass, the next is
    refused with I4MOE_EINJECTED; a value that is not a non-negative integer is ignored."""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd.runtime import I4moeError
    print("[boundary] fail-after from the environment", flush=True)
    cfg = get_config("tiny")
    L = make_layer(cfg, 0)
    x = x_to_device(L.x, L.x_dtype)
    monkeypatch.setenv("I4MOE_FAIL_AFTER", "2")
    ctx = new_ctx()
    monkeypatch.delenv("I4MOE_FAIL_AFTER")
    upload_layer(ctx, L, 0)             # uploads are never gated
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(0, x)
    z = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
    with pytest.raises(I4moeError) as ei:
        ctx.take(z)
    assert ei.value.code == B.I4MOE_EINJECTED
    ctx.close()
    for bad in ("-1", "two", "3x", ""):
        monkeypatch.setenv("I4MOE_FAIL_AFTER", bad)
        c2 = new_ctx()
        monkeypatch.delenv("I4MOE_FAIL_AFTER")
        upload_layer(c2, L, 0)
        for _ in range(3):
            assert normwise_err(tiny_delta(c2, cfg, L, x), oracle_delta(cfg, L)) < TOL
        c2.close()


@pytest.mark.parametrize("name", ["medium", "mix"])
def test_wave_factor_changes_tiling_not_bits(name, monkeypatch):
    """I4MOE_WAVE_FACTOR retiles the projections (rows per wave) but every row is still reduced by
    one wave in a fixed order: contexts created with different factors give the same bits."""
    import torch
    print(f"[boundary] wave factor {name}", flush=True)
    cfg = get_config(name)
    L = make_layer(cfg, 0)
    x = x_to_device(L.x, L.x_dtype)
    outs = []
    for f in ("0.1", "1", "8"):
        monkeypatch.setenv("I4MOE_WAVE_FACTOR", f)
        ctx = new_ctx()
        monkeypatch.delenv("I4MOE_WAVE_FACTOR")
        upload_layer(ctx, L, 0)
        pair = []
        for host in (True, False):      # the separate kernels, and the fused ones the bench times
            ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=host)
            ctx.issue(0, x)
            r = torch.from_numpy(L.residual.copy()).to("cuda:0")
            ctx.take(r)
            torch.cuda.synchronize()
            pair.append(r.cpu().numpy().tobytes())
        assert pair[0] == pair[1]
        outs.append(pair[0])
        ctx.close()
    assert outs[0] == outs[1] == outs[2]


def test_read_probe_reads_and_rejects_bad_arguments():
    """The read probe (a measuring aid) launches once per call, is timed as I4MOE_K_PROBE, leaves
    the layer's results untouched, and refuses a bad layer, mask, list or unbound expert with
    EINVAL and nothing launched."""
    from int4_grouped_expert_router_amd import I4moeError
    from int4_grouped_expert_router_amd import binding as B
    cfg = get_config("mix", D=1024, I=200, E=6, K=2, S=1, layers=1)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    before = tiny_delta(ctx, cfg, L, x)
    ctx.set_profiling(True)
    for mask in (1, 2, 3, 4, 7):
        ctx.read_probe(0, mask, list(range(cfg.E)))
    ms, n = ctx.profile(B.I4MOE_K_PROBE)
    assert n == 5 and ms > 0.0
    for layer, mask, ex in [(1, 3, [0]), (0, 0, [0]), (0, 8, [0]), (0, 3, []), (0, 3, [cfg.E]), (0, 3, [-1]),
                            (0, 3, list(range(65)))]:
        with pytest.raises(I4moeError) as ei:
            ctx.read_probe(layer, mask, ex)
        assert ei.value.code == B.I4MOE_EINVAL
    assert ctx.profile(B.I4MOE_K_PROBE)[1] == 5  # nothing launched by the refused calls
    ctx.set_profiling(False)
    assert np.array_equal(tiny_delta(ctx, cfg, L, x), before)
    ctx.close()
