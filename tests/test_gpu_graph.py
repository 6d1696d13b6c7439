"""One captured HIP graph per MoE layer (route -> issue -> take, no host work between the
kernels): every replay, with eager work of the program between replays, gives the eager
result bit for bit, and a replay into a zero residual gives the oracle's two-layer delta
(MI355X only).  One case has about 16 rows per expert, so the matrix-core launches are in the
graph."""

from __future__ import annotations

import numpy as np
import pytest

from harness import (TOL, gpu_routes, layer_delta_threads, make_layer, near_tie, normwise_err, oracle_routes,
                     route_matches, upload_layer, x_to_device)
from synth import get_config

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["medium", "mix", "small_batch_like", "prefill_like"])
def test_graph_replays_match_eager(name):
    import torch
    from int4_grouped_expert_router_amd import Context
    print(f"[graph] {name}", flush=True)
    if name == "small_batch_like":
        cfg = get_config("tiny", D=1024, I=512, E=32, K=4, S=4, formats="group", gs=64, x_dtype="bf16", seed=21)
    elif name == "prefill_like":
        # 32 tokens over 4 experts, about 16 rows each: the matrix-core launches inside the graph
        cfg = get_config("tiny", D=1024, I=512, E=4, K=2, S=32, formats="mix_even_odd", gs=64, x_dtype="bf16",
                         seed=22)
    else:
        cfg = get_config(name)
    s = torch.cuda.Stream()
    ctx = Context(0, s)
    layers = [make_layer(cfg, l) for l in range(2)]
    for l, L in enumerate(layers):
        upload_layer(ctx, L, l)
    xs = [x_to_device(L.x, L.x_dtype) for L in layers]
    r0 = torch.from_numpy(layers[0].residual.copy()).to("cuda:0")
    resid = torch.empty_like(r0)

    def two_layers():
        for l in range(2):
            ctx.route(l, xs[l], cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
            ctx.issue(l, xs[l])
            ctx.take(resid)

    with torch.cuda.stream(s):
        resid.copy_(r0)
        two_layers()
    s.synchronize()
    eager = resid.cpu().numpy()
    if name == "prefill_like":
        # the same layers eager with profiling on: the matrix-core launches are part of the step
        from int4_grouped_expert_router_amd import binding as B
        ctx.set_profiling(True)
        with torch.cuda.stream(s):
            resid.copy_(r0)
            two_layers()
        s.synchronize()
        assert ctx.profile(B.I4MOE_K_MFMA)[1] > 0
        ctx.set_profiling(False)
        assert resid.cpu().numpy().tobytes() == eager.tobytes()
    # the routes each layer takes (deterministic, so the graph's routes are these too)
    recs = [ctx.route(l, xs[l], cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True) for l in range(2)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        two_layers()
    s.synchronize()
    other = torch.zeros_like(r0)
    for rep in range(5):
        with torch.cuda.stream(s):
            resid.copy_(r0)
        g.replay()
        s.synchronize()
        assert resid.cpu().numpy().tobytes() == eager.tobytes(), f"replay {rep}"
        # eager work between replays: the library's own path on another buffer, and torch ops
        with torch.cuda.stream(s):
            other.copy_(r0)
            ctx.route(1, xs[1], cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
            ctx.issue(1, xs[1])
            ctx.take(other)
            other.mul_(0.5).add_(1.0)
        s.synchronize()
    # one more replay into a zero residual: the sum of both layers' deltas, against the oracle
    with torch.cuda.stream(s):
        resid.zero_()
    g.replay()
    s.synchronize()
    got = resid.cpu().numpy()
    ref = np.zeros((cfg.S, cfg.D))
    for l, L in enumerate(layers):
        routes, x64 = oracle_routes(cfg, L)
        use = []
        for t in range(cfg.S):
            if near_tie(routes[t], cfg.K, cfg.topp):
                use.append(gpu_routes(recs[l], cfg.S, cfg.K)[t])
            else:
                assert route_matches(recs[l][t], routes[t], cfg.K), (l, t)
                use.append(routes[t])
        ref += layer_delta_threads(use, L.expert, x64)[0]
    err = normwise_err(got, ref)
    print(f"[graph] {name}: replay vs oracle normwise error {err:.2e}", flush=True)
    assert err < TOL, err
    ctx.close()
