"""Shared helpers for the GPU parity tests: upload synthetic layers through the C ABI, run
route/issue/take, and compare with the f64 oracle."""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import math
import os
from types import SimpleNamespace

import numpy as np

import oracle
from oracle import router as orouter
from synth import gen_layer
from synth.gen import gen_expert

TOL = 1e-4          # normwise relative error bar for expert outputs (f32 accumulation vs f64)
NEAR_TIE = 1e-9     # score / top-p distance below which a selection counts as a near-tie


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def x_to_device(x: np.ndarray, dtype: str):
    torch, dev = torch_dev()
    if dtype == "bf16":
        t = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dev)


WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def upload_layer(ctx, L, layer: int, experts=None):
    """Upload the router and experts of L to `layer`.  Experts are drawn in a thread pool and
    not kept on the host (the oracle draws the ones it needs again, with the same bytes)."""
    cfg = L.cfg
    ctx.upload_router(layer, L.router_W, L.router_b)
    experts = list(range(cfg.E) if experts is None else experts)
    handles = {}
    draw = lambda e: L._experts.get(e) or gen_expert(cfg, L.layer, e)
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        for e, ew in zip(experts, ex.map(draw, experts)):
            h = (ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up), ctx.upload_host_tensor(ew.down))
            ctx.set_expert(layer, e, *h)
            handles[e] = h
    return handles


def layer_delta_threads(routes, expert_of, x64):
    """oracle.experts.layer_delta with each (token, k) row's expert forward evaluated in a thread
    pool (numpy releases the interpreter lock inside them); the weighted sums are then taken in
    the oracle's own (token, k) order, so delta and the intermediates are the oracle's bit for
    bit."""
    x64 = np.atleast_2d(x64)
    pairs = [(t, k) for t, r in enumerate(routes) for k in range(r.n)]
    distinct = sorted({int(routes[t].idx[k]) for t, k in pairs})
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        ws = dict(zip(distinct, ex.map(expert_of, distinct)))
        outs = list(ex.map(lambda tk: oracle.expert_forward(ws[int(routes[tk[0]].idx[tk[1]])].gate,
                                                            ws[int(routes[tk[0]].idx[tk[1]])].up,
                                                            ws[int(routes[tk[0]].idx[tk[1]])].down, x64[tk[0]]),
                           pairs))
    delta = np.zeros(x64.shape, dtype=np.float64)
    inter = {}
    for (t, k), o in zip(pairs, outs):
        inter[(t, k)] = o
        delta[t] += float(routes[t].w32[k]) * o[3]
    return delta, inter


def gpu_routes(rec, S: int, K: int):
    """The GPU's route records in the form the oracle's expert functions take (n, idx, w32): used to
    check the experts on the GPU's own route when a selection is a near-tie."""
    return [SimpleNamespace(n=int(rec[t].n), idx=[int(v) for v in rec[t].idx[:K]],
                            w32=np.array(rec[t].w[:K], dtype=np.float32)) for t in range(S)]


def near_tie(r: orouter.RouteResult, K: int, topp: float, tau: float = NEAR_TIE) -> bool:
    c = np.sort(r.scores)[::-1][:K + 1]
    if np.any(c[:-1] - c[1:] < tau):
        return True
    p = float(np.float32(topp))
    if 0.0 < p < 1.0:
        w = [float(r.sigma[e]) for e in r.idx]
        total = math.fsum(w)
        run = 0.0
        for v in w:
            run += v
            if abs(run - p * total) < tau * total:
                return True
    for v in r.w64[:r.n]:
        f = np.float32(v)
        lo = float(np.nextafter(f, np.float32(-np.inf)))
        hi = float(np.nextafter(f, np.float32(np.inf)))
        for mid in ((float(f) + lo) / 2, (float(f) + hi) / 2):
            if abs(v - mid) < 1e-12 * abs(v):
                return True
    return False


def route_matches(gpu_rec, r: orouter.RouteResult, K: int) -> bool:
    if gpu_rec.n != r.n:
        return False
    if list(gpu_rec.idx[:K]) != list(r.idx):
        return False
    gw = np.array(gpu_rec.w[:K], dtype=np.float32)
    return np.array_equal(gw.view(np.uint32), r.w32.view(np.uint32))


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.atleast_2d(got).astype(np.float64)
    ref = np.atleast_2d(ref)
    errs = []
    for g, r in zip(got, ref):
        den = np.max(np.abs(r))
        errs.append(np.max(np.abs(g - r)) / den if den > 0 else np.max(np.abs(g)))
    return float(max(errs))


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def run_layer(ctx, cfg, L, layer: int, K=None, topp=None, norm=None, scale=None, residual=None):
    """route + issue + take on the device; returns (route records, out numpy, x device tensor)."""
    torch, dev = torch_dev()
    K = cfg.K if K is None else K
    topp = cfg.topp if topp is None else topp
    norm = cfg.norm_topk if norm is None else norm
    scale = cfg.routed_scale if scale is None else scale
    x = x_to_device(L.x, L.x_dtype)
    res = np.zeros((cfg.S, cfg.D), np.float32) if residual is None else residual
    r_dev = torch.from_numpy(res.copy()).to(dev)
    rec = ctx.route(layer, x, K, topp, norm, scale, host_out=True)
    ctx.issue(layer, x)
    ctx.take(r_dev)
    torch.cuda.synchronize()
    return rec, r_dev.cpu().numpy(), x


def oracle_routes(cfg, L, K=None, topp=None, norm=None, scale=None):
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    return oracle.route(L.router_W, L.router_b, x64, cfg.K if K is None else K,
                        cfg.topp if topp is None else topp, cfg.norm_topk if norm is None else norm,
                        cfg.routed_scale if scale is None else scale), x64


def make_layer(cfg, layer=0):
    return gen_layer(cfg, layer)


def host_tensor(fmt, gs, O, C, packed, scales):
    return SimpleNamespace(fmt=fmt, gs=gs, O=O, C=C, packed=packed, scales=scales)
