"""Benchmark: microseconds per decode MoE layer (route + grouped int4 experts + take) on one
MI355X, with the int4 expert-weight bandwidth of the dominant kernel against HBM peak.

A step is one MoE layer at S=1 on the medium decode workload (D=4096, I=1536, E=64, top-8,
per-row int4 experts, bf16 activations, top-p 0.95, norm_topk, routed_scale 2.5).  Steps
cycle through 8 distinct layers (~606 MB of selected expert weights per cycle, more than the
256 MB Infinity Cache), so weights stream from HBM.  Inputs are resident in HBM before timing.

Prints one JSON line.  --gpus must be 1: this path runs on one GPU.
"""

from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE layer at S=1 + expert int4 weight GB/s (% of HBM peak)"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def tensor_bytes(t) -> int:
    return t.packed.nbytes + t.scales.nbytes


def setup(cfg, layers, ctx, torch):
    from synth import gen_layer
    Ls = []
    for l in range(layers):
        L = gen_layer(cfg, l)
        ctx.upload_router(l, L.router_W, L.router_b)
        for e in range(cfg.E):
            ew = L.expert(e)
            ctx.set_expert(l, e, ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up),
                           ctx.upload_host_tensor(ew.down))
        L.bytes_gate_up = {e: tensor_bytes(L.expert(e).gate) + tensor_bytes(L.expert(e).up) for e in range(cfg.E)}
        L.bytes_down = {e: tensor_bytes(L.expert(e).down) for e in range(cfg.E)}
        L.drop_experts()
        if L.x_dtype == "bf16":
            L.x_dev = torch.from_numpy(L.x.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")
        else:
            L.x_dev = torch.from_numpy(L.x).to("cuda:0")
        L.r_dev = torch.from_numpy(L.residual.copy()).to("cuda:0")
        Ls.append(L)
        log(f"layer {l} uploaded")
    return Ls


def cpu_baseline(cfg, budget_s: float):
    """The f64 oracle, as it stands, on the host: whole layers of the same workload."""
    import oracle
    from synth import gen_layer
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    times = []
    t_start = time.perf_counter()
    l = 0
    while True:
        L = gen_layer(cfg, 100 + l)
        x64 = oracle.widen_activations(L.x, L.x_dtype)
        t0 = time.perf_counter()
        oracle.moe_layer(L.router_W, L.router_b, x64, L.expert, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale,
                         residual=L.residual)
        times.append(time.perf_counter() - t0)
        l += 1
        if time.perf_counter() - t_start > budget_s or l >= 8:
            break
    us = float(np.median(times)) * 1e6
    return {"value": round(us, 1), "unit": "us/layer", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{len(times)} whole layers of the same workload (fresh seeds), median; numpy f64 "
                      f"dequantise + BLAS matvec, correctly rounded router sums; host "
                      f"os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}, "
                      f"BLAS threads={blas_threads}"}


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    path = os.path.join(PROFILES, f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for name in rec.get("sources", []):
        with open(os.path.join(ROOT, "int4_grouped_expert_router_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if not rec.get("sources") or h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_sleep(torch, stream, host_us_per_step: float = 150.0, burst: int = 40) -> int:
    """GPU sleep cycles that outlast the host's enqueue of one burst of steps (with margin)."""
    probe = 1_000_000
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record()
        torch.cuda._sleep(probe)
        b.record()
    b.synchronize()
    us = max(a.elapsed_time(b) * 1e3, 1.0)
    return int(probe * host_us_per_step * burst / us)


def copy_calibration(torch, nbytes: int = 256 << 20, reps: int = 5):
    """Plain device-to-device copies of known size: what FETCH_SIZE and WRITE_SIZE report per
    dispatch here, against nbytes, is the scale applied to the same counters on the kernels."""
    torch.cuda.set_device(0)
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def sustained_stream(torch, B, layers: int = 2, steps: int = 60, reps: int = 3):
    """The steady-state expert stream: the sustained workload (D=7168, I=2048, all 64 experts
    of a layer taken, S=1, half g64 / half per-row), `layers` distinct layers (1.5 GB of int4
    each, far more than the 256 MB Infinity Cache) cycled from one captured graph."""
    from int4_grouped_expert_router_amd import Context
    from synth import get_config
    cfg = get_config("sustained")
    stream = torch.cuda.current_stream()
    ctx = Context(0, stream)
    Ls = setup(cfg, layers, ctx, torch)
    per_layer = [sum(L.bytes_gate_up[e] + L.bytes_down[e] for e in range(cfg.E)) for L in Ls]

    def step(i):
        L = Ls[i % layers]
        ctx.route(i % layers, L.x_dev, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)
        ctx.issue(i % layers, L.x_dev)
        ctx.take(L.r_dev)

    for i in range(2 * layers):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    elapsed = float(np.median(times))
    ctx.set_profiling(True)
    sleep_cycles = calibrate_sleep(torch, stream, burst=8)
    for b0 in range(0, steps, 8):
        torch.cuda._sleep(sleep_cycles)
        for i in range(b0, min(steps, b0 + 8)):
            step(i)
    torch.cuda.synchronize()
    kt = {name: ctx.profile(k) for name, k in
          [("route", B.I4MOE_K_ROUTE), ("dual", B.I4MOE_K_DUAL), ("down", B.I4MOE_K_DOWN), ("take", B.I4MOE_K_TAKE)]}
    ctx.close()
    nbytes = sum(per_layer[i % layers] for i in range(steps))
    gbps = nbytes / elapsed / 1e9
    dual_gu = sum(sum(Ls[i % layers].bytes_gate_up[e] for e in range(cfg.E)) for i in range(steps))
    dual_gbps = dual_gu / (kt["dual"][0] * 1e-3) / 1e9
    return {"workload": f"sustained stream: D={cfg.D} I={cfg.I}, all {cfg.K} of E={cfg.E} experts per layer, S=1, "
                        f"{cfg.formats} int4 (gs={cfg.gs}), {cfg.x_dtype} activations; {layers} distinct layers "
                        f"({per_layer[0] / 1e9:.2f} GB each) cycled from one graph",
            "steps": steps, "replays": f"median of {reps}", "us_per_layer": round(elapsed / steps * 1e6, 2),
            "expert_weight_GBps_layer": round(gbps, 1), "pct_hbm_peak_layer": round(100 * gbps / HBM_PEAK_GBPS, 2),
            "dual_GBps": round(dual_gbps, 1), "dual_pct_hbm_peak": round(100 * dual_gbps / HBM_PEAK_GBPS, 2),
            "kernel_us": {k: round(v[0] * 1e3 / max(v[1], 1), 3) for k, v in kt.items()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="medium")
    ap.add_argument("--layers", type=int, default=0, help="distinct layers to cycle (0 = workload default)")
    ap.add_argument("--eager", action="store_true", help="launch the timed steps one call at a time (no graph)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sustained", action="store_true", help="skip the sustained-stream measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain 256 MiB device copies (scale for the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this decode MoE expert path runs on one GPU; --gpus must be 1 "
                                   "(expert-parallel sharding across GPUs is a design, not run here)"}))
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from int4_grouped_expert_router_amd import Context
    from int4_grouped_expert_router_amd import binding as B
    from synth import get_config

    cfg = get_config(args.workload)
    layers = args.layers or cfg.layers
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()   # default priority; a non-legacy stream so it can be captured
    torch.cuda.set_stream(stream)
    ctx = Context(0, stream)
    Ls = setup(cfg, layers, ctx, torch)

    # routes are deterministic per layer: read the kept experts once for the byte count
    kept = []
    for l, L in enumerate(Ls):
        rec = ctx.route(l, L.x_dev, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
        kept.append([[rec[t].idx[k] for k in range(rec[t].n)] for t in range(cfg.S)])
    lib = B.load()
    p = ctx.p
    xargs = [(C.c_void_p(L.x_dev.data_ptr()), B.I4MOE_DTYPE_BF16 if L.x_dtype == "bf16" else B.I4MOE_DTYPE_F32,
              C.c_void_p(L.r_dev.data_ptr())) for L in Ls]
    topp, norm, scale, K, S = C.c_float(cfg.topp), 1 if cfg.norm_topk else 0, C.c_float(cfg.routed_scale), cfg.K, cfg.S

    def step(i):
        l = i % layers
        x, dt, r = xargs[l]
        rc = lib.i4moe_route(p, l, x, dt, S, K, topp, norm, scale, None)
        rc2 = lib.i4moe_expert_group_issue(p, l, x, dt, S, None)
        rc3 = lib.i4moe_expert_group_take(p, r, S)
        if rc or rc2 < 0 or rc3:
            raise RuntimeError(f"step failed: {ctx.last_error()}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed steps replay from one captured graph (the host enqueues a whole sequence of
    # layers at once, as a decode loop would); --eager launches them one call at a time.
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        log("graph captured")

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us_per_layer = elapsed / args.steps * 1e6

    # The same steps again, eager, with HIP events around every launch on the library's stream.
    # They go in bursts queued behind a GPU sleep, so the GPU runs each burst back to back and
    # an event pair spans its kernel only, not host launch gaps.
    ctx.set_profiling(True)
    sleep_cycles = calibrate_sleep(torch, stream)
    burst = 40
    for b0 in range(0, args.steps, burst):
        torch.cuda._sleep(sleep_cycles)
        for i in range(b0, min(args.steps, b0 + burst)):
            step(i)
    torch.cuda.synchronize()
    kt = {name: ctx.profile(k) for name, k in
          [("route", B.I4MOE_K_ROUTE), ("dual", B.I4MOE_K_DUAL), ("down", B.I4MOE_K_DOWN), ("take", B.I4MOE_K_TAKE)]}
    ctx.set_profiling(False)

    gu_bytes = sum(sum(Ls[i % layers].bytes_gate_up[e] for t in kept[i % layers] for e in t) for i in range(args.steps))
    dn_bytes = sum(sum(Ls[i % layers].bytes_down[e] for t in kept[i % layers] for e in t) for i in range(args.steps))
    x_bytes = cfg.S * cfg.D * (2 if cfg.x_dtype == "bf16" else 4)
    dual_alg = gu_bytes + args.steps * x_bytes
    dual_ms, dual_n = kt["dual"]
    achieved = dual_alg / (dual_ms * 1e-3) / 1e9
    down_ms, _ = kt["down"]
    take_ms, _ = kt["take"]
    # the expert weights stream through the dual kernel and the down projection, which runs
    # inside the take kernel for a lone one-token issue
    expert_gbps_kernels = (gu_bytes + dn_bytes) / ((dual_ms + down_ms + take_ms) * 1e-3) / 1e9
    expert_gbps_layer = (gu_bytes + dn_bytes) / elapsed / 1e9
    traffic = load_traffic("dual", args.workload)

    line = {
        "metric": METRIC,
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} decode MoE layer: D={cfg.D} I={cfg.I} E={cfg.E} top-{cfg.K} S={cfg.S}, "
                               f"{cfg.formats} int4 (gs={cfg.gs}), {cfg.x_dtype} activations, top-p {cfg.topp}, "
                               f"routed_scale {cfg.routed_scale}",
                   "layers_cycled": layers, "launch": "graph" if graph is not None else "eager stream",
                   "weights": "random int4, seeded"},
        "expert_weight_GBps_layer": round(expert_gbps_layer, 1),
        "expert_weight_GBps_kernels": round(expert_gbps_kernels, 1),
        "expert_weight_pct_hbm_peak_kernels": round(100 * expert_gbps_kernels / HBM_PEAK_GBPS, 2),
        "kernel_us": {k: round(v[0] * 1e3 / max(v[1], 1), 3) for k, v in kt.items()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "k_proj dual gate/up+SiLU with the one-token expert selection", "bytes_per_launch": round(dual_alg / args.steps),
                     "avg_launch_us": round(dual_ms * 1e3 / max(dual_n, 1), 3)},
    }
    ctx.close()
    if not args.no_sustained and args.workload == "medium":
        log("sustained stream")
        line["sustained_stream"] = sustained_stream(torch, B)
    if not args.no_cpu:
        log("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
