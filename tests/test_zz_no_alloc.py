"""The allocation-free route entry point through the C ABI (MI355X only): i4moe_route_noalloc
gives the records of i4moe_route bit for bit, on two calls in a row (the second smaller, on the
scratch the first left behind), refuses sizes beyond its static scratch with nothing written,
and leaves the layer's own device route (the one an issue consumes) untouched."""

from __future__ import annotations

import ctypes as C

import numpy as np
import pytest

from harness import make_layer, upload_layer, x_to_device
from synth import get_config

pytestmark = pytest.mark.gpu

REC = 4 + 64 * 4 + 64 * 4   # bytes of one i4moe_route_host record


def new_ctx():
    import torch
    from int4_grouped_expert_router_amd import Context
    assert torch.cuda.is_available()
    return Context(0, torch.cuda.current_stream())


def test_route_noalloc_matches_route():
    import torch
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd.runtime import I4moeError
    print("[no-alloc] route_noalloc vs route", flush=True)
    ctx = new_ctx()
    rng = np.random.default_rng(97)
    # (layer, E, D, S, K, topp, norm, scale, x dtype): the second call is smaller in every size
    cases = [(0, 256, 1536, 4, 8, 0.9, True, 2.5, "bf16"), (1, 64, 512, 1, 4, 0.0, False, 1.0, "f32")]
    for layer, E, D, S, K, topp, norm, scale, xd in cases:
        W = rng.normal(0, 0.02, (E, D)).astype(np.float32)
        b = rng.normal(0, 0.1, E).astype(np.float32)
        ctx.upload_router(layer, W, b)
    from synth import round_f32_to_bf16_bits
    for layer, E, D, S, K, topp, norm, scale, xd in cases:
        xs = rng.standard_normal((S, D)).astype(np.float32)
        x = x_to_device(round_f32_to_bf16_bits(xs) if xd == "bf16" else xs, xd)
        out = torch.full((S * REC,), 0xAB, dtype=torch.uint8, device="cuda:0")
        ctx.route_noalloc(layer, x, K, topp, norm, scale, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().tobytes()
        ref = ctx.route(layer, x, K, topp, norm, scale, host_out=True)
        assert got == bytes(ref), (layer, S, K)
        print(f"[no-alloc] layer {layer} S={S} K={K}: {S} records equal", flush=True)
    # beyond the scratch: refused, nothing written
    x = x_to_device(rng.standard_normal((65, 512)).astype(np.float32), "f32")
    out = torch.full((65 * REC,), 0xCD, dtype=torch.uint8, device="cuda:0")
    for S, K in ((65, 1), (8, 9)):
        with pytest.raises(I4moeError) as ei:
            ctx.route_noalloc(1, x[:S], K, 0.0, True, 1.0, out)
        assert ei.value.code == B.I4MOE_EUNSUPPORTED, (S, K)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 0xCD).all()
    ctx.close()


def test_route_noalloc_leaves_the_device_route():
    """route (device route kept for the issue) -> route_noalloc of another x -> issue -> take
    gives the layer output of the first route, bit for bit."""
    import torch
    print("[no-alloc] the layer's device route is untouched", flush=True)
    cfg = get_config("tiny", E=16, K=4)
    L = make_layer(cfg, 0)
    ctx = new_ctx()
    upload_layer(ctx, L, 0)
    x = x_to_device(L.x, L.x_dtype)
    other = x_to_device(np.random.default_rng(5).standard_normal((1, cfg.D)).astype(np.float32), "f32")
    ref = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.issue(0, x)
    ctx.take(ref)
    out = torch.empty((REC,), dtype=torch.uint8, device="cuda:0")
    r = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    ctx.route_noalloc(0, other, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, out)
    ctx.issue(0, x)
    ctx.take(r)
    torch.cuda.synchronize()
    assert r.cpu().numpy().tobytes() == ref.cpu().numpy().tobytes()
    ctx.close()
