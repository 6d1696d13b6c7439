"""One-token device routes without a host copy: the route call enqueues only the logits GEMV and
the issue that consumes the route runs the selection inside its dual projection.  These tests
hold that path to the oracle and, bit for bit, to the separate selection kernel (which runs when
a host copy is requested), and walk the host-side cases in which the deferred selection must
run on its own first (MI355X only)."""

from __future__ import annotations

import ctypes as C

import numpy as np
import pytest

from harness import TOL, digest, make_layer, near_tie, normwise_err, oracle_routes, route_matches, upload_layer, x_to_device
from synth import get_config

pytestmark = pytest.mark.gpu


def new_ctx():
    import torch
    from int4_grouped_expert_router_amd import Context
    assert torch.cuda.is_available()
    return Context(0, torch.cuda.current_stream())


def layer_pass(ctx, cfg, L, x, host_out, layer=0):
    """route + issue with every tap, then take into the layer's residual."""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    ctx.route(layer, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=host_out)
    slot = ctx.issue(layer, x)
    got = {
        "h": ctx.tap(B.I4MOE_TAP_H),
        "y": ctx.tap(B.I4MOE_TAP_Y, slot),
        "route": ctx.tap(B.I4MOE_TAP_ROUTE, layer, np.uint8),
        "group": ctx.tap(B.I4MOE_TAP_GROUP, layer, np.int32),
        "logits": ctx.tap(B.I4MOE_TAP_LOGITS, 0, np.float64),
    }
    r = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.take(r)
    torch.cuda.synchronize()
    got["out"] = r.cpu().numpy()
    return got


def route_records(raw: np.ndarray, S: int):
    from int4_grouped_expert_router_amd import binding as B
    return (B.i4moe_route_host * S).from_buffer_copy(raw.tobytes())


CASES = {
    "tiny": {},
    "tiny_k_eq_e": {"K": 8},
    "tiny_topp_cut": {"topp": 0.3, "routed_scale": 2.5},
    "tiny_no_norm": {"norm_topk": False, "topp": 0.0},
    "ragged_16e": {"D": 1000, "I": 200, "E": 16, "K": 4, "formats": "mix_even_odd", "gs": 64, "topp": 0.9},
    "ragged_wide": {"D": 7168, "I": 2048, "E": 16, "K": 8, "formats": "mix_even_odd", "gs": 64},
    "generic_spans": {"D": 130, "I": 34, "E": 5, "K": 5, "formats": "mix_even_odd", "gs": 32, "x_dtype": "bf16"},
}


@pytest.mark.parametrize("name", ["medium", "mix", *CASES])
def test_fused_matches_separate_and_oracle(name):
    print(f"[fused] {name}", flush=True)
    cfg = get_config(name) if name in ("medium", "mix") else get_config("tiny", seed=7, **CASES[name])
    assert cfg.S == 1
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    sep = layer_pass(ctx, cfg, L, x, host_out=True)
    fus = layer_pass(ctx, cfg, L, x, host_out=False)
    for k in sep:
        assert sep[k].tobytes() == fus[k].tobytes(), k
    routes, x64 = oracle_routes(cfg, L)
    if near_tie(routes[0], cfg.K, cfg.topp):
        pytest.skip("near-tie route; selection not comparable bit for bit")
    rec = route_records(fus["route"], 1)
    assert route_matches(rec[0], routes[0], cfg.K)
    import oracle
    delta, _ = oracle.experts.layer_delta(routes, L.expert, x64)
    assert normwise_err(fus["out"] - L.residual, delta) < TOL
    ctx.close()


def test_fused_determinism_medium():
    import torch
    print("[fused] determinism medium x10", flush=True)
    cfg = get_config("medium")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    seen = set()
    for _ in range(10):
        r = torch.from_numpy(L.residual.copy()).to("cuda:0")
        ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
        ctx.issue(0, x)
        ctx.take(r)
        torch.cuda.synchronize()
        seen.add(digest(r.cpu().numpy()))
    assert len(seen) == 1
    ctx.close()


def two_layers():
    cfg = get_config("tiny", D=512, I=256, E=16, K=4, topp=0.9, routed_scale=2.5, seed=11)
    L0, L1 = make_layer(cfg, 0), make_layer(cfg, 1)
    ctx = new_ctx()
    upload_layer(ctx, L0, 0)
    upload_layer(ctx, L1, 1)
    return cfg, L0, L1, ctx


def reference_two(ctx, cfg, L0, L1, x0, x1):
    """Both layers routed with host copies (separate selection kernels), one take."""
    import torch
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    ctx.route(1, x1, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    ctx.issue(0, x0)
    ctx.issue(1, x1)
    r = torch.from_numpy(L0.residual.copy()).to("cuda:0")
    ctx.take(r)
    torch.cuda.synchronize()
    return r.cpu().numpy()


def test_pending_selection_runs_before_next_route():
    """A second route overwrites the router scratch: the first route's selection runs before it,
    and the first layer's issue then reads that materialised group."""
    import torch
    print("[fused] route, route, issue, issue", flush=True)
    cfg, L0, L1, ctx = two_layers()
    x0, x1 = x_to_device(L0.x, L0.x_dtype), x_to_device(L1.x, L1.x_dtype)
    ref = reference_two(ctx, cfg, L0, L1, x0, x1)
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.route(1, x1, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(0, x0)   # layer 0's selection already ran as its own kernel
    ctx.issue(1, x1)   # layer 1's selection runs inside this dual projection
    r = torch.from_numpy(L0.residual.copy()).to("cuda:0")
    ctx.take(r)
    torch.cuda.synchronize()
    assert r.cpu().numpy().tobytes() == ref.tobytes()
    ctx.close()


def test_pending_selection_with_tap_stream_switch_and_explicit_group():
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print("[fused] tap / explicit group / stream switch / injected failure", flush=True)
    cfg, L0, L1, ctx = two_layers()
    x0, x1 = x_to_device(L0.x, L0.x_dtype), x_to_device(L1.x, L1.x_dtype)
    ref = reference_two(ctx, cfg, L0, L1, x0, x1)
    rec1 = ctx.route(1, x1, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    rows1 = [(int(rec1[0].idx[k]), 0, float(rec1[0].w[k])) for k in range(rec1[0].n)]

    def finish():
        r = torch.from_numpy(L0.residual.copy()).to("cuda:0")
        ctx.take(r)
        torch.cuda.synchronize()
        return r.cpu().numpy()

    # a tap of the pending route runs its selection first; the issue then reads that group
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    tapped = route_records(ctx.tap(B.I4MOE_TAP_ROUTE, 0, np.uint8), 1)
    ctx.issue(0, x0)
    ctx.issue(1, x1, rows=rows1)
    assert finish().tobytes() == ref.tobytes()
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    assert bytes(tapped) == bytes(route_records(ctx.tap(B.I4MOE_TAP_ROUTE, 0, np.uint8), 1))

    # an explicit-group issue of another layer leaves the pending selection to the next issue
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(1, x1, rows=rows1)
    ctx.issue(0, x0)
    out = finish()
    # same sums, slots taken in issue order: layer 1 first this time
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    ctx.issue(1, x1, rows=rows1)
    ctx.issue(0, x0)
    assert out.tobytes() == finish().tobytes()

    # a stream switch runs the pending selection on the old stream
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.set_stream(s1)
    s1.wait_stream(s0)
    with torch.cuda.stream(s1):
        ctx.issue(0, x0)
        ctx.issue(1, x1, rows=rows1)
        r = torch.from_numpy(L0.residual.copy()).to("cuda:0")
        ctx.take(r)
    s1.synchronize()
    ctx.set_stream(s0)
    assert r.cpu().numpy().tobytes() == ref.tobytes()

    # an injected issue failure enqueues nothing; the selection still runs with the next issue
    ctx.route(0, x0, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.set_fail_after(0)
    from int4_grouped_expert_router_amd import I4moeError
    with pytest.raises(I4moeError):
        ctx.issue(0, x0)
    ctx.set_fail_after(-1)
    ctx.issue(0, x0)
    ctx.issue(1, x1, rows=rows1)
    assert finish().tobytes() == ref.tobytes()
    ctx.close()


DOWN_TAKE_CASES = {
    "tiny": {},
    "topp_dead_rows": {"topp": 0.3, "routed_scale": 2.5},
    "ragged_d": {"D": 1000, "I": 200, "E": 16, "K": 4, "formats": "mix_even_odd", "gs": 64, "topp": 0.9},
    "group_tail": {"D": 520, "I": 2000, "E": 8, "K": 8, "formats": "group", "gs": 64, "x_dtype": "bf16"},
    "one_expert": {"K": 1},
    # several tokens: the down projection runs on its own before the take either way
    "tokens4_topp": {"D": 1024, "I": 512, "E": 32, "K": 4, "S": 4, "formats": "group", "gs": 64, "x_dtype": "bf16",
                     "topp": 0.6},
    "tokens64_k1": {"D": 256, "I": 128, "E": 8, "K": 1, "S": 64},
    "tokens8_all_experts": {"D": 256, "I": 256, "E": 8, "K": 8, "S": 8, "formats": "mix_even_odd", "gs": 32},
}


@pytest.mark.parametrize("name", ["medium", "mix", "small_batch", *DOWN_TAKE_CASES])
def test_down_take_fused_matches_separate(name):
    """A lone one-token issue of a device route runs its down projection inside the take; a y
    tap before the take makes the down projection run on its own first. Both must give the
    same residual bits, and the residual must match the oracle. Several tokens take the
    separate down projection and take both times. (The full small-batch layer is compared
    bit for bit only; its oracle check is the sampled full-size test.)"""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print(f"[fused] down+take {name}", flush=True)
    full = name in ("medium", "mix", "small_batch")
    cfg = get_config(name) if full else get_config("tiny", seed=5, **DOWN_TAKE_CASES[name])
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    outs = []
    for tap_first in (True, False):
        ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
        slot = ctx.issue(0, x)
        if tap_first:
            ctx.tap(B.I4MOE_TAP_Y, slot)
        r = torch.from_numpy(L.residual.copy()).to("cuda:0")
        ctx.take(r)
        torch.cuda.synchronize()
        outs.append(r.cpu().numpy())
    assert outs[0].tobytes() == outs[1].tobytes()
    if name == "small_batch":
        ctx.close()
        return
    routes, x64 = oracle_routes(cfg, L)
    if any(near_tie(routes[t], cfg.K, cfg.topp) for t in range(cfg.S)):
        pytest.skip("near-tie route; selection not comparable bit for bit")
    import oracle
    delta, _ = oracle.experts.layer_delta(routes, L.expert, x64)
    assert normwise_err(outs[1] - L.residual, delta) < TOL
    ctx.close()


def test_same_route_issued_twice():
    """Two issues of one deferred route: the first runs the selection inside its dual
    projection and leaves its down projection waiting; the second issue runs that down
    projection first and then reads the group the first one published. The take then adds
    two identical slots: exactly twice one slot's sum."""
    import torch
    print("[fused] one route, two issues", flush=True)
    cfg = get_config("medium")
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    outs = []
    for issues in (1, 2):
        ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
        for _ in range(issues):
            ctx.issue(0, x)
        r = torch.zeros((1, cfg.D), dtype=torch.float32, device="cuda:0")
        ctx.take(r)
        torch.cuda.synchronize()
        outs.append(r.cpu().numpy())
    assert outs[1].tobytes() == (2 * outs[0]).astype(np.float32).tobytes()
    ctx.close()


def test_tensor_free_runs_the_waiting_down_projection_first():
    """Freeing a tensor while a down projection waits for the take: the library runs that
    down projection (and waits for it) before it frees anything, so the take still adds the
    same bits."""
    import torch
    print("[fused] free while the down projection waits", flush=True)
    cfg = get_config("tiny", K=2, seed=3)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    handles = upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    rec = ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    ctx.issue(0, x)
    ref = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.take(ref)
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(0, x)
    ctx.free_tensor(handles[int(rec[0].idx[0])][2])  # the first selected expert's down tensor
    r = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.take(r)
    torch.cuda.synchronize()
    assert r.cpu().numpy().tobytes() == ref.cpu().numpy().tobytes()
    ctx.close()
