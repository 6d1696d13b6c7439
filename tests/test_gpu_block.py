"""The steps around the routed experts through the C ABI (MI355X only): rmsnorm against the
oracle (bit for bit, away from rounding ties), the shared expert, and the whole MoE block in one
call against the oracle's block, equal bit for bit to the same steps called one by one (the
block's shared expert riding in the routed group, or in its own issue when the group is full),
and replayed from a captured graph."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from harness import (TOL, gpu_routes, layer_delta_threads, make_layer, near_tie, normwise_err, route_matches,
                     upload_layer, x_to_device)
from synth import gen_norm, gen_shared_expert, get_config

pytestmark = pytest.mark.gpu
EPS = 1e-5


def new_ctx():
    import torch
    from int4_grouped_expert_router_amd import Context
    assert torch.cuda.is_available()
    return Context(0, torch.cuda.current_stream())


def rounding_tie(v: float, dtype: str) -> bool:
    """The f64 value sits within 1e-12 (relative) of a boundary between two representable values."""
    if dtype == "f32":
        f = np.float32(v)
        nb = [float(np.nextafter(f, np.float32(-np.inf))), float(np.nextafter(f, np.float32(np.inf)))]
        mids = [(float(f) + x) / 2 for x in nb]
    else:
        r = oracle.block.round_bf16(v)
        b = oracle.block.bf16_bits(r)
        nb = [float(np.array([((b + d) & 0xFFFF) << 16], np.uint32).view(np.float32)[0]) for d in (-1, 1)]
        mids = [(r + x) / 2 for x in nb]
    return any(abs(v - m) <= 1e-12 * abs(v) for m in mids)


def check_norm_codes(got, n64, dtype):
    """Bit-equal rounded outputs, except at f64 values within 1e-12 of a rounding tie (then one
    step apart at most)."""
    want = oracle.block.round_activations(n64, dtype)
    g = np.asarray(got).view(np.uint32 if dtype == "f32" else np.uint16)
    w = want.view(np.uint32 if dtype == "f32" else np.uint16)
    bad = np.argwhere(g != w)
    for idx in bad:
        v = float(n64[tuple(idx)])
        assert rounding_tie(v, dtype), (tuple(idx), v, g[tuple(idx)], w[tuple(idx)])
        assert abs(int(g[tuple(idx)]) - int(w[tuple(idx)])) == 1
    return len(bad)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rmsnorm_matches_oracle(dtype):
    import torch
    print(f"[block] rmsnorm {dtype}", flush=True)
    rng = np.random.default_rng(61)
    D, S, ld = 7168, 5, 7168 + 96
    ctx = new_ctx()
    gamma = rng.normal(1.0, 0.1, D).astype(np.float32)
    ctx.upload_norm(0, gamma, EPS)
    x = np.zeros((S, ld), np.float32)
    x[:, :D] = rng.standard_normal((S, D)).astype(np.float32) * np.array([[1.0], [3e-3], [250.0], [1.0], [1e-20]])
    x[3, :D] = 0.0                                       # a zero row: eps keeps it finite (all zeros out)
    x[:, D:] = np.nan                                     # past the row: never read
    xd = torch.from_numpy(x).to("cuda:0")
    out = torch.full((S, D + 32), 7.0, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda:0")
    ctx.rmsnorm(0, xd, out, ld_x=ld, ld_out=D + 32)
    torch.cuda.synchronize()
    o = out.cpu()
    got = (o.numpy() if dtype == "f32" else o.view(torch.int16).numpy().view(np.uint16))[:, :D]
    n64 = oracle.block.rmsnorm(x[:, :D], gamma, EPS)
    ties = check_norm_codes(got, n64, dtype)
    print(f"[block] rmsnorm {dtype}: {ties} tie(s) of {S * D}", flush=True)
    tail = (o.numpy() if dtype == "f32" else o.float().numpy())[:, D:]
    assert (tail == 7.0).all()                            # past the row: never written
    ctx.close()


def block_layer(name, **over):
    cfg = get_config(name, **over)
    L = make_layer(cfg, 0)
    return cfg, L


def setup_block(ctx, cfg, L, shared=True):
    upload_layer(ctx, L, 0)
    ctx.upload_norm(0, gen_norm(cfg, 0), EPS)
    sh = gen_shared_expert(cfg, 0)
    if shared:
        ctx.set_shared_expert(0, ctx.upload_host_tensor(sh.gate), ctx.upload_host_tensor(sh.up),
                              ctx.upload_host_tensor(sh.down))
    return sh


CASES = {
    "medium_like": ("medium", {"E": 16}),
    "small_batch_like": ("small_batch", {"D": 2048, "I": 768, "E": 32, "K": 4}),
    "sustained_like": ("sustained", {"E": 16, "K": 8}),
    # 16 tokens: the shared expert's entry (16 rows) and the routed entries of 8 rows or more run on
    # the matrix cores, the others on the vector kernels, in one block
    "prefill_like": ("small_batch", {"D": 2048, "I": 768, "E": 8, "K": 2, "S": 16}),
    # S * K = 64 routed rows: no room for the shared rows in the routed group, so the shared
    # expert takes its own issue and slot
    "full_group": ("small_batch", {"D": 1024, "I": 512, "E": 16, "K": 8, "S": 8}),
    # one token over 128 experts: the select kernel (not the dual) builds the group with the
    # shared row
    "wide_router": ("small_batch", {"D": 1024, "I": 512, "E": 128, "K": 8, "S": 1}),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_moe_block_matches_oracle(case):
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print(f"[block] moe block {case}", flush=True)
    name, over = CASES[case]
    cfg, L = block_layer(name, **over)
    ctx = new_ctx()
    sh = setup_block(ctx, cfg, L)
    gamma = gen_norm(cfg, 0)
    dt = B.I4MOE_DTYPE_BF16 if cfg.x_dtype == "bf16" else B.I4MOE_DTYPE_F32
    r0 = L.residual.copy()
    # the block in one call
    r = torch.from_numpy(r0.copy()).to("cuda:0")
    ctx.moe_block(0, r, dt, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    torch.cuda.synchronize()
    out_block = r.cpu().numpy()
    # the same steps one call at a time, with host copies for the checks
    tdt = torch.float32 if dt == B.I4MOE_DTYPE_F32 else torch.bfloat16
    r2 = torch.from_numpy(r0.copy()).to("cuda:0")
    a = torch.empty((cfg.S, cfg.D), dtype=tdt, device="cuda:0")
    ctx.rmsnorm(0, r2, a)
    rec = ctx.route(0, a, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
    ctx.issue(0, a)
    ctx.shared_issue(0, a)
    ctx.take(r2)
    torch.cuda.synchronize()
    assert r2.cpu().numpy().tobytes() == out_block.tobytes()
    # against the oracle
    a_gpu = a.cpu().numpy() if dt == B.I4MOE_DTYPE_F32 else a.cpu().view(torch.int16).numpy().view(np.uint16)
    n64 = oracle.block.rmsnorm(r0, gamma, EPS)
    check_norm_codes(a_gpu, n64, cfg.x_dtype)
    a64 = oracle.widen_activations(a_gpu, cfg.x_dtype)      # equal to the oracle's own, ties aside
    routes = oracle.route(L.router_W, L.router_b, a64, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
    use = []
    for t in range(cfg.S):
        if near_tie(routes[t], cfg.K, cfg.topp):
            use.append(gpu_routes(rec, cfg.S, cfg.K)[t])
        else:
            assert route_matches(rec[t], routes[t], cfg.K), t
            use.append(routes[t])
    delta, _ = layer_delta_threads(use, L.expert, a64)
    for t in range(cfg.S):
        delta[t] += oracle.expert_forward(sh.gate, sh.up, sh.down, a64[t])[3]
    err = normwise_err(out_block.astype(np.float64) - r0.astype(np.float64), delta)
    print(f"[block] {case}: normwise error {err:.2e}", flush=True)
    assert err < TOL, err
    ctx.close()


def test_shared_expert_alone():
    """The shared expert's issue, alone, over three tokens: weight 1 per token."""
    import torch
    print("[block] shared expert alone", flush=True)
    cfg, L = block_layer("mix", D=1024, I=512, E=8, K=2, S=3)
    ctx = new_ctx()
    sh = setup_block(ctx, cfg, L)
    x = x_to_device(L.x, L.x_dtype)
    ctx.shared_issue(0, x)
    z = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    ctx.take(z)
    torch.cuda.synchronize()
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    ref = np.stack([oracle.expert_forward(sh.gate, sh.up, sh.down, x64[t])[3] for t in range(cfg.S)])
    assert normwise_err(z.cpu().numpy(), ref) < TOL
    ctx.close()


def test_moe_block_in_a_graph():
    """Two blocks captured in one graph: every replay equals the eager result bit for bit."""
    import torch
    from int4_grouped_expert_router_amd import binding as B
    print("[block] graph", flush=True)
    cfg, L = block_layer("medium", E=16)
    s = torch.cuda.Stream()
    from int4_grouped_expert_router_amd import Context
    ctx = Context(0, s)
    setup_block(ctx, cfg, L)
    r0 = torch.from_numpy(L.residual.copy()).to("cuda:0")
    r = torch.empty_like(r0)
    dt = B.I4MOE_DTYPE_BF16

    def two_blocks():
        for _ in range(2):
            ctx.moe_block(0, r, dt, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)

    with torch.cuda.stream(s):
        r.copy_(r0)
        two_blocks()                                     # the first call allocates the block scratch
        r.copy_(r0)
        two_blocks()
    s.synchronize()
    eager = r.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        two_blocks()
    for rep in range(3):
        with torch.cuda.stream(s):
            r.copy_(r0)
        g.replay()
        s.synchronize()
        assert r.cpu().numpy().tobytes() == eager.tobytes(), rep
    ctx.close()


def test_moe_block_refused_when_gated():
    import torch
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd.runtime import I4moeError
    cfg, L = block_layer("tiny")
    ctx = new_ctx()
    setup_block(ctx, cfg, L)
    r = torch.from_numpy(L.residual.copy()).to("cuda:0")
    ctx.set_fail_after(0)
    with pytest.raises(I4moeError) as ei:
        ctx.moe_block(0, r, B.I4MOE_DTYPE_F32, cfg.K)
    assert ei.value.code == B.I4MOE_EINJECTED
    ctx.set_fail_after(1)                                # the whole block is one call
    ctx.moe_block(0, r, B.I4MOE_DTYPE_F32, cfg.K)
    with pytest.raises(I4moeError):
        ctx.moe_block(0, r, B.I4MOE_DTYPE_F32, cfg.K)
    torch.cuda.synchronize()
    ctx.close()
