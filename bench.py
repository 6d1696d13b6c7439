"""Benchmark: microseconds per decode MoE layer (route + grouped int4 experts + take) on one
MI355X, with the int4 expert-weight bandwidth of the dominant kernel against HBM peak.

The headline workload is the sustained stream: D=7168, I=2048, S=1, all 64 experts of a layer
taken per launch (the 64-expert cap), experts 0-31 group-wise int4 (gs=64) and 32-63 per-row,
f32 activations, issued over 16 layers with distinct weights back to back (24 GB of int4, far
more than the 256 MB Infinity Cache, so every weight streams from HBM).  A step is one MoE layer;
the timed steps replay from one captured graph, inputs resident in HBM.  The medium decode layer
(D=4096, I=1536, top-8 of 64, bf16) and the small batch (S=4, top-8 of 256, g64, bf16) are
measured after it as secondary records.

Prints one JSON line.  --gpus must be 1: this path runs on one GPU.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
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
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))
# secondary workloads: (name, distinct layers, timed steps)
SECONDARY = {"medium": (8, 400), "small_batch": (2, 100)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def tensor_bytes(t) -> int:
    return t.packed.nbytes + t.scales.nbytes


def setup(cfg, layers, ctx, torch):
    """Upload `layers` distinct layers of the workload; experts are drawn in a thread pool and
    uploaded in order (the context is single-threaded)."""
    from synth import gen_layer
    from synth.gen import gen_expert
    Ls = []
    with cf.ThreadPoolExecutor(WORKERS) as pool:
        for l in range(layers):
            L = gen_layer(cfg, l)
            ctx.upload_router(l, L.router_W, L.router_b)
            L.bytes_gate_up, L.bytes_down = {}, {}
            for e, ew in enumerate(pool.map(lambda e: gen_expert(cfg, l, e), range(cfg.E))):
                ctx.set_expert(l, e, ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up),
                               ctx.upload_host_tensor(ew.down))
                L.bytes_gate_up[e] = tensor_bytes(ew.gate) + tensor_bytes(ew.up)
                L.bytes_down[e] = tensor_bytes(ew.down)
            if L.x_dtype == "bf16":
                L.x_dev = torch.from_numpy(L.x.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")
            else:
                L.x_dev = torch.from_numpy(L.x).to("cuda:0")
            L.r_dev = torch.from_numpy(L.residual.copy()).to("cuda:0")
            Ls.append(L)
    log(f"{cfg.name}: {layers} layers uploaded")
    return Ls


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


def torch_read(torch, gib: float = 1.5, reps: int = 10):
    """Context for the plain-read figure: what PyTorch's own kernels reach on the same GPU, a
    float32 sum (reads the tensor once) and a device copy (reads and writes it), on a resident
    tensor of `gib` GiB; one JSON line of GB/s."""
    torch.cuda.set_device(0)
    n = int(gib * (1 << 30)) // 4
    t = torch.ones(n, dtype=torch.float32, device="cuda:0")
    u = torch.empty_like(t)
    res = {"tensor_bytes": 4 * n}
    for name, fn, nbytes in (("sum_f32", lambda: t.sum(), 4 * n), ("copy", lambda: u.copy_(t), 8 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[name + "_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(res), flush=True)


def workload_text(cfg, layers):
    extra = f", top-p {cfg.topp}" if cfg.topp else ""
    return (f"{cfg.name}: D={cfg.D} I={cfg.I} E={cfg.E} top-{cfg.K} S={cfg.S}, {cfg.formats} int4 (gs={cfg.gs}), "
            f"{cfg.x_dtype} activations{extra}, routed_scale {cfg.routed_scale}; {layers} distinct layers issued "
            f"back to back")


WARM_STEPS = 48  # untimed graph-replayed steps before the timed ones (at least)


def measure(name, layers, steps, warmup, torch, B, eager=False):
    """Time `steps` MoE layers of the workload (cycling `layers` distinct layers), then the same
    steps again with HIP events around every launch; returns the measurements."""
    from int4_grouped_expert_router_amd import Context
    from synth import get_config
    cfg = get_config(name)
    stream = torch.cuda.Stream()   # default priority; a non-legacy stream so it can be captured
    torch.cuda.set_stream(stream)
    ctx = Context(0, stream)
    Ls = setup(cfg, layers, ctx, torch)

    # routes are deterministic per layer: the distinct experts each layer takes (an expert picked by
    # several tokens is one weight stream), for the byte counts
    taken = []
    for l, L in enumerate(Ls):
        rec = ctx.route(l, L.x_dev, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
        pairs = [int(rec[t].idx[k]) for t in range(cfg.S) for k in range(rec[t].n)]
        taken.append((sorted(set(pairs)), len(pairs)))
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

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed steps replay from one captured graph (the host enqueues a whole sequence of
    # layers at once, as a decode loop would); --eager launches them one call at a time.
    # The captured graph is replayed untimed until at least WARM_STEPS steps have run: sustained
    # load first lowers the clocks for some 30 layers and then settles (the per-dispatch trace
    # in profiles/kernel_trace_stats_sustained.md), and the timed steps should see the settled
    # state a long decode runs in, not that transient.
    graph = None
    warm_replays = 0
    if not eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                step(i)
        warm_replays = max(1, -(-WARM_STEPS // steps))
        for _ in range(warm_replays):
            graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # The same steps again, eager, with HIP events around every launch on the library's stream.
    # They go in bursts queued behind a GPU sleep, so the GPU runs each burst back to back and
    # an event pair spans its kernel only, not host launch gaps.
    ctx.set_profiling(True)
    burst = 40
    sleep_cycles = calibrate_sleep(torch, stream, burst=burst)
    for b0 in range(0, steps, burst):
        torch.cuda._sleep(sleep_cycles)
        for i in range(b0, min(steps, b0 + burst)):
            step(i)
    torch.cuda.synchronize()
    kt = {k: ctx.profile(v) for k, v in
          [("route", B.I4MOE_K_ROUTE), ("dual", B.I4MOE_K_DUAL), ("down", B.I4MOE_K_DOWN), ("take", B.I4MOE_K_TAKE),
           ("mfma", B.I4MOE_K_MFMA)]}
    if kt["mfma"][1] == 0:
        del kt["mfma"]

    # The plain-read rate of the same experts' weights on this GPU: the read probe over each
    # step's distinct experts (gate + up, then down), in the same bursts behind a GPU sleep.
    probe = {}
    for key, mask in (("gate_up", 3), ("down", 4)):
        ctx.set_profiling(True)
        for b0 in range(0, steps, burst):
            torch.cuda._sleep(sleep_cycles)
            for i in range(b0, min(steps, b0 + burst)):
                ctx.read_probe(i % layers, mask, taken[i % layers][0])
        torch.cuda.synchronize()
        probe[key] = ctx.profile(B.I4MOE_K_PROBE)
    ctx.set_profiling(False)
    launch = "graph" if graph is not None else "eager stream"
    del graph
    torch.cuda.synchronize()
    ctx.close()
    torch.cuda.empty_cache()

    gu = [sum(Ls[l].bytes_gate_up[e] for e in taken[l][0]) for l in range(layers)]
    dn = [sum(Ls[l].bytes_down[e] for e in taken[l][0]) for l in range(layers)]
    x_bytes = cfg.S * cfg.D * (2 if cfg.x_dtype == "bf16" else 4)
    gu_bytes = sum(gu[i % layers] for i in range(steps))
    dn_bytes = sum(dn[i % layers] for i in range(steps))
    dual_alg = gu_bytes + steps * x_bytes
    dual_ms, dual_n = kt["dual"]
    down_ms, down_n = kt["down"]
    take_ms, _ = kt["take"]
    achieved = dual_alg / (dual_ms * 1e-3) / 1e9
    us = elapsed / steps * 1e6
    res = {
        "workload": workload_text(cfg, layers),
        "steps": steps,
        "launch": launch,
        "us_per_layer": round(us, 3),
        "untimed_steps_before": warmup + warm_replays * steps,
        "ms_per_step": round(elapsed / steps * 1e3, 6),
        "experts_per_layer": round(sum(len(taken[i % layers][0]) for i in range(steps)) / steps, 2),
        "rows_per_layer": round(sum(taken[i % layers][1] for i in range(steps)) / steps, 2),
        "expert_weight_bytes_per_layer": round((gu_bytes + dn_bytes) / steps),
        "expert_weight_GBps_layer": round((gu_bytes + dn_bytes) / elapsed / 1e9, 1),
        "expert_weight_pct_hbm_peak_layer": round(100 * (gu_bytes + dn_bytes) / elapsed / 1e9 / HBM_PEAK_GBPS, 2),
        "expert_weight_GBps_kernels": round((gu_bytes + dn_bytes) / ((dual_ms + down_ms + take_ms) * 1e-3) / 1e9, 1),
        "kernel_us": {k: round(v[0] * 1e3 / max(v[1], 1), 3) for k, v in kt.items()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic("dual", name),
                     "kernel": "k_proj dual gate/up + SiLU (with the one-token selection when S=1, E<=64)",
                     "bytes_per_launch": round(dual_alg / steps), "avg_launch_us": round(dual_ms * 1e3 / max(dual_n, 1), 3)},
    }
    pr_gu = gu_bytes / (probe["gate_up"][0] * 1e-3) / 1e9
    pr_dn = dn_bytes / (probe["down"][0] * 1e-3) / 1e9
    res["plain_read"] = {
        "kernel": "k_read_probe: the same experts' nibbles and scales as contiguous ~16 KB row blocks, "
                  "no arithmetic (HIP events, as the kernels above)",
        "gate_up_GBps": round(pr_gu, 1), "gate_up_pct_hbm_peak": round(100 * pr_gu / HBM_PEAK_GBPS, 2),
        "down_GBps": round(pr_dn, 1), "down_pct_hbm_peak": round(100 * pr_dn / HBM_PEAK_GBPS, 2),
        "dual_frac_of_plain_read": round((gu_bytes / (dual_ms * 1e-3) / 1e9) / pr_gu, 4),
        "avg_launch_us": {"gate_up": round(probe["gate_up"][0] * 1e3 / max(probe["gate_up"][1], 1), 3),
                          "down": round(probe["down"][0] * 1e3 / max(probe["down"][1], 1), 3)},
    }
    if down_n:   # a down projection launched on its own (otherwise it ran inside the take kernel)
        res["plain_read"]["down_frac_of_plain_read"] = round((dn_bytes / (down_ms * 1e-3) / 1e9) / pr_dn, 4)
        res["down_GBps"] = round(dn_bytes / (down_ms * 1e-3) / 1e9, 1)
        res["down_pct_hbm_peak"] = round(100 * dn_bytes / (down_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)
    return res, cfg


# Rows per expert in one issue: the vector kernels one row at a time, the vector kernels with
# rows sharing weight passes, the matrix cores (every entry of 2 rows or more), and the library's
# own choice.
CROSS_ROWS = (1, 2, 3, 4, 8, 12, 16, 24, 32, 48, 64)
CROSS_MODES = {"per_row": {"I4MOE_ENTRY_ROWS": "0", "I4MOE_MFMA_MIN_ROWS": "0"},
               "shared_passes": {"I4MOE_ENTRY_ROWS": "4", "I4MOE_MFMA_MIN_ROWS": "0"},
               "matrix_cores": {"I4MOE_ENTRY_ROWS": "0", "I4MOE_MFMA_MIN_ROWS": "2"},
               "automatic": {}}


def crossover(torch, B, reps: int = 24, n_experts: int = 32, rows=CROSS_ROWS, modes=tuple(CROSS_MODES),
              formats: str = "group"):
    """Device time of one issue + take for explicit groups of R rows per expert (S = 64 tokens,
    min(8, 64 // R) experts per issue, rotating over 32 experts of the small-batch shape so the
    weights stream from HBM; group-wise g64 experts, or per-row with formats="row"), under each
    launch mode; prints one JSON line per R."""
    from int4_grouped_expert_router_amd import Context
    from synth import gen_layer, get_config
    from synth.gen import gen_expert
    cfg = get_config("small_batch", S=64, E=n_experts, formats=formats, gs=64 if formats == "group" else 0)
    L = gen_layer(cfg, 0)
    with cf.ThreadPoolExecutor(WORKERS) as pool:
        ews = list(pool.map(lambda e: gen_expert(cfg, 0, e), range(n_experts)))
    per_expert = tensor_bytes(ews[0].gate) + tensor_bytes(ews[0].up) + tensor_bytes(ews[0].down)
    x = torch.from_numpy(L.x.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")
    out = torch.zeros((cfg.S, cfg.D), dtype=torch.float32, device="cuda:0")
    table = {R: {"rows_per_expert": R, "experts_per_issue": max(1, min(8, cfg.S // R)), "formats": formats}
             for R in rows}
    for mode in modes:
        env = CROSS_MODES[mode]
        saved = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        ctx = Context(0, torch.cuda.current_stream())
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k)
            else:
                os.environ[k] = v
        for e, ew in enumerate(ews):
            ctx.set_expert(0, e, ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up),
                           ctx.upload_host_tensor(ew.down))
        for R in rows:
            n = table[R]["experts_per_issue"]

            def group(it):
                ex = [(it * n + k) % n_experts for k in range(n)]
                return [(e, (k * R + j) % cfg.S, 0.5) for k, e in enumerate(ex) for j in range(R)]

            for it in range(3):
                ctx.issue(0, x, rows=group(it))
                ctx.take(out)
            torch.cuda.synchronize()
            ctx.set_profiling(True)
            for it in range(reps):
                ctx.issue(0, x, rows=group(it))
                ctx.take(out)
            torch.cuda.synchronize()
            kt = {k: ctx.profile(v) for k, v in [("dual", B.I4MOE_K_DUAL), ("down", B.I4MOE_K_DOWN),
                                                 ("mfma", B.I4MOE_K_MFMA), ("take", B.I4MOE_K_TAKE)]}
            ctx.set_profiling(False)
            dev_us = sum(v[0] for v in kt.values()) * 1e3 / reps
            table[R][mode] = {"device_us_per_issue": round(dev_us, 2),
                              "device_us_per_expert": round(dev_us / n, 3),
                              "weight_GBps": round(per_expert * n / (dev_us * 1e-6) / 1e9, 1),
                              "kernel_us": {k: round(v[0] * 1e3 / reps, 2) for k, v in kt.items() if v[1]}}
            log(f"crossover {mode} R={R}: {dev_us:.1f} us per issue")
        ctx.close()
        torch.cuda.empty_cache()
    for R in rows:
        best = min(modes, key=lambda m: table[R][m]["device_us_per_issue"])
        table[R]["fastest"] = best
        print(json.dumps(table[R]), flush=True)


def block(torch, B, name: str = "medium", layers: int = 8, steps: int = 400, warmup: int = 16):
    """The MoE block around the routed experts at decode: per layer one i4moe_moe_block call
    (rmsnorm of the residual row, route, routed experts, the layer's shared expert, the join
    into the residual), over `layers` distinct layers each with its norm weights and shared
    expert, replayed from one captured graph; then the same calls eager with HIP events around
    every launch.  Each layer's residual row carries on from block to block (the rmsnorm keeps
    the activations at scale).  Prints one JSON line."""
    from int4_grouped_expert_router_amd import Context
    from synth import gen_norm, gen_shared_expert, get_config
    cfg = get_config(name)
    stream = torch.cuda.Stream()   # default priority
    torch.cuda.set_stream(stream)
    ctx = Context(0, stream)
    Ls = setup(cfg, layers, ctx, torch)
    shared_bytes = 0
    for l in range(layers):
        ctx.upload_norm(l, gen_norm(cfg, l), 1e-5)
        sh = gen_shared_expert(cfg, l)
        ctx.set_shared_expert(l, ctx.upload_host_tensor(sh.gate), ctx.upload_host_tensor(sh.up),
                              ctx.upload_host_tensor(sh.down))
        shared_bytes = tensor_bytes(sh.gate) + tensor_bytes(sh.up) + tensor_bytes(sh.down)
    dt = B.I4MOE_DTYPE_BF16 if cfg.x_dtype == "bf16" else B.I4MOE_DTYPE_F32

    def step(i):
        L = Ls[i % layers]
        ctx.moe_block(i % layers, L.r_dev, dt, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graph
    ctx.set_profiling(True)
    burst = 40
    sleep_cycles = calibrate_sleep(torch, stream, burst=burst)
    for b0 in range(0, steps, burst):
        torch.cuda._sleep(sleep_cycles)
        for i in range(b0, min(steps, b0 + burst)):
            step(i)
    torch.cuda.synchronize()
    kt = {k: ctx.profile(v) for k, v in [("route", B.I4MOE_K_ROUTE), ("dual", B.I4MOE_K_DUAL),
                                         ("down", B.I4MOE_K_DOWN), ("take", B.I4MOE_K_TAKE)]}
    ctx.set_profiling(False)
    finite = all(bool(torch.isfinite(L.r_dev).all()) for L in Ls)
    ctx.close()
    torch.cuda.empty_cache()
    us = elapsed / steps * 1e6
    print(json.dumps({
        "block": workload_text(cfg, layers) + ", S=1 decode, rmsnorm + route + routed experts + shared expert + join",
        "steps": steps, "launch": "graph", "us_per_block": round(us, 3),
        "kernel_us_per_block": {k: round(v[0] * 1e3 / steps, 3) for k, v in kt.items()},
        "launches_per_block": {k: round(v[1] / steps, 2) for k, v in kt.items()},
        "shared_expert_bytes": shared_bytes,
        "residual_finite": finite}), flush=True)


def tiered(torch, B, reps: int = 30):
    """The CPU tier's overlap: experts of the small-batch shape (D=6144, I=2048, g64, bf16; 64
    experts, even ones on the device, odd ones kept on the host), top-8 routes at S = 1, 4 and 8.
    Per S: wall time of the device rows alone, the host rows alone (with the host's integer dot
    products when it has them, those at 256 bits, and the float32 ones), and both in one tiered issue (route
    copy to the host excluded: the routes are computed once); prints one JSON line per S."""
    from int4_grouped_expert_router_amd import Context
    from synth import gen_layer, get_config
    from synth.gen import gen_expert
    for S in (1, 4, 8):
        cfg = get_config("small_batch", S=S, E=64)
        L = gen_layer(cfg, 0)
        ctx = Context(0, torch.cuda.current_stream())
        ctx.upload_router(0, L.router_W, L.router_b)
        with cf.ThreadPoolExecutor(WORKERS) as pool:
            for e, ew in enumerate(pool.map(lambda e: gen_expert(cfg, 0, e), range(cfg.E))):
                if e % 2:
                    ctx.set_host_expert(0, e, ew.gate, ew.up, ew.down)
                else:
                    ctx.set_expert(0, e, ctx.upload_host_tensor(ew.gate), ctx.upload_host_tensor(ew.up),
                                   ctx.upload_host_tensor(ew.down))
        x = torch.from_numpy(L.x.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")
        out = torch.zeros((S, cfg.D), dtype=torch.float32, device="cuda:0")
        rec = list(ctx.route(0, x, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True))

        def only(keep):
            rs = [B.i4moe_route_host() for _ in range(S)]
            for t in range(S):
                ks = [k for k in range(rec[t].n) if keep(rec[t].idx[k])]
                rs[t].n = len(ks)
                for j, k in enumerate(ks):
                    rs[t].idx[j], rs[t].w[j] = rec[t].idx[k], rec[t].w[k]
            return rs

        host = only(lambda e: e % 2 == 1)
        # the same host rows with the integer dot products kept at 256 bits (I4MOE_HOST_INT=256)
        # and with the float32 ones (I4MOE_HOST_INT=0)
        arms = {"device_only": only(lambda e: e % 2 == 0), "host_only": host, "host_only_256": host,
                "host_only_float": host, "tiered": rec}
        forced = {"host_only_256": "256", "host_only_float": "0"}
        res = {"S": S, "threads": None, "host_int_path": int(B.i4moe_host_int_path())}
        walls = {k: [] for k in arms}
        cpus = []
        prev = os.environ.get("I4MOE_HOST_INT")
        for rep in range(reps + 3):  # the arms interleaved, so they see the same machine state
            for name, routes in arms.items():
                if name in forced:
                    os.environ["I4MOE_HOST_INT"] = forced[name]
                elif prev is None:
                    os.environ.pop("I4MOE_HOST_INT", None)
                else:
                    os.environ["I4MOE_HOST_INT"] = prev
                t0 = time.perf_counter()
                _, tt = ctx.tiered_issue(0, x, routes)
                ctx.take(out)
                torch.cuda.synchronize()
                if rep >= 3:
                    walls[name].append(time.perf_counter() - t0)
                    if name == "tiered":
                        cpus.append(tt.cpu_ms)
                        res["device_rows"], res["host_rows"] = tt.device_rows, tt.host_rows
        for name in arms:
            res[name + "_ms"] = round(float(np.median(walls[name])) * 1e3, 3)
        res["tiered_cpu_ms"] = round(float(np.median(cpus)), 3)
        if prev is None:
            os.environ.pop("I4MOE_HOST_INT", None)
        else:
            os.environ["I4MOE_HOST_INT"] = prev
        # int4 weight bytes the host rows read (nibbles and scales of gate, up and down)
        ex1 = gen_expert(cfg, 0, 1)
        per_row = sum(t.packed.nbytes + t.scales.nbytes for t in (ex1.gate, ex1.up, ex1.down))
        res["host_weight_gbps"] = round(res["host_rows"] * per_row / (res["host_only_ms"] * 1e-3) / 1e9, 1)
        res["serial_ms"] = round(res["device_only_ms"] + res["host_only_ms"], 3)
        res["hidden_ms"] = round(res["serial_ms"] - res["tiered_ms"], 3)
        hw = len(os.sched_getaffinity(0))
        res["threads"] = int(os.environ.get("I4MOE_HOST_THREADS", "0")) or (1 if hw <= 2 else min(16, hw - 1))
        log(f"tiered S={S}: {res}")
        print(json.dumps(res), flush=True)
        ctx.close()
        torch.cuda.empty_cache()


def reread(torch, B, name: str = "medium", layers: int = 8, reps: int = 40):
    """Whether weights read a moment ago read faster: the read probe over each layer's taken
    experts, in bursts behind a GPU sleep, as down alone, gate + up then down, and gate + up,
    down, down again (the second down read right after the first).  Median µs per launch from
    HIP events on the library's stream; one JSON line."""
    from int4_grouped_expert_router_amd import Context
    from synth import get_config
    cfg = get_config(name)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    ctx = Context(0, stream)
    Ls = setup(cfg, layers, ctx, torch)
    taken = []
    for l, L in enumerate(Ls):
        rec = ctx.route(l, L.x_dev, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale, host_out=True)
        taken.append(sorted(set(int(rec[t].idx[k]) for t in range(cfg.S) for k in range(rec[t].n))))
    sleep_cycles = calibrate_sleep(torch, stream, burst=reps)

    def run(seq):
        times = {}
        for rep in range(3):  # the first burst warms up and is dropped
            torch.cuda._sleep(sleep_cycles)
            evs = []
            for i in range(reps):
                for label, mask in seq:
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    ctx.read_probe(i % layers, mask, taken[i % layers])
                    b.record()
                    evs.append((label, a, b))
            torch.cuda.synchronize()
            if rep:
                for label, a, b in evs:
                    times.setdefault(label, []).append(a.elapsed_time(b) * 1e3)
        return {k: round(float(np.median(v)), 2) for k, v in times.items()}

    res = {"workload": workload_text(cfg, layers),
           "gate_up_MB": round(sum(Ls[0].bytes_gate_up[e] for e in taken[0]) / 1e6, 2),
           "down_MB": round(sum(Ls[0].bytes_down[e] for e in taken[0]) / 1e6, 2),
           "down_alone_us": run([("down", 4)]),
           "gate_up_then_down_us": run([("gate_up", 3), ("down", 4)]),
           "down_read_twice_us": run([("gate_up", 3), ("down_first", 4), ("down_again", 4)])}
    log(f"reread {name}: {res}")
    print(json.dumps(res), flush=True)
    ctx.close()


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(cfg, layers: int):
    """The f64 oracle, as it stands, on the host: one whole layer of the same workload (a fresh
    seed), at the BLAS thread count the host gives and again at one thread; plus the pure-Python
    brute force on the tiny workload."""
    import oracle
    from oracle import brute
    from synth import gen_layer, get_config
    from threadpoolctl import threadpool_limits
    L = gen_layer(cfg, 100)
    x64 = oracle.widen_activations(L.x, L.x_dtype)
    for e in range(cfg.E):     # drawn before the clock starts
        L.expert(e)

    def one_layer():
        t0 = time.perf_counter()
        oracle.moe_layer(L.router_W, L.router_b, x64, L.expert, cfg.K, cfg.topp, cfg.norm_topk, cfg.routed_scale,
                         residual=L.residual)
        return time.perf_counter() - t0

    nthreads = blas_threads()
    t_all = one_layer()
    log(f"oracle, {nthreads} BLAS threads: {t_all:.2f} s per layer")
    with threadpool_limits(limits=1):
        t_one = one_layer()
    log(f"oracle, one thread: {t_one:.2f} s per layer")
    tiny = get_config("tiny")
    T = gen_layer(tiny, 0)
    xt = oracle.widen_activations(T.x, T.x_dtype)[0].tolist()
    t0 = time.perf_counter()
    n, idx, w = brute.route(T.router_W, T.router_b, xt, tiny.K, tiny.topp, tiny.norm_topk, tiny.routed_scale)
    for k in range(n):
        ew = T.expert(idx[k])
        brute.expert(ew.gate, ew.up, ew.down, xt)
    t_brute = time.perf_counter() - t0
    return {"value": round(t_all * 1e6, 1), "unit": "us/layer", "cores": int(nthreads), "kind": "oracle",
            "sample": f"1 whole layer of the same workload (fresh seed, {cfg.K} experts), route + experts + "
                      f"weighted reduce + residual; numpy f64 dequantise + BLAS matvec, correctly rounded router "
                      f"sums; {nthreads} BLAS threads (the dequantisation is single-threaded numpy); host "
                      f"os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}",
            "one_thread_us_per_layer": round(t_one * 1e6, 1),
            "stream_s": {"layers": layers, "all_threads": round(layers * t_all, 2), "one_thread": round(layers * t_one, 2),
                         "how": f"one layer x {layers}"},
            "tiny_brute_force_us_per_layer": round(t_brute * 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="sustained")
    ap.add_argument("--layers", type=int, default=0, help="distinct layers to cycle (0 = workload default)")
    ap.add_argument("--eager", action="store_true", help="launch the timed steps one call at a time (no graph)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="measure the headline workload only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain 256 MiB device copies (scale for the HBM byte counters)")
    ap.add_argument("--torch-read", action="store_true",
                    help="only time PyTorch's own sum and copy of a resident 1.5 GiB tensor (read-rate context)")
    ap.add_argument("--crossover", action="store_true",
                    help="only time explicit groups of 1..64 rows per expert under each launch mode")
    ap.add_argument("--crossover-rows", default="", help="comma-separated rows per expert (default: all)")
    ap.add_argument("--block", action="store_true",
                    help="only time the MoE block (rmsnorm, route, routed and shared experts, join) on medium")
    ap.add_argument("--tiered", action="store_true",
                    help="only time the CPU tier: device rows, host rows, and both overlapped")
    ap.add_argument("--reread", action="store_true",
                    help="only time the read probe on medium weights read once and read again at once")
    ap.add_argument("--crossover-modes", default="", help="comma-separated launch modes (default: all)")
    ap.add_argument("--crossover-formats", default="group", choices=("group", "row"),
                    help="crossover experts: group-wise g64 (default) or per-row int4")
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
    if args.torch_read:
        torch_read(torch)
        return
    from int4_grouped_expert_router_amd import binding as B
    from synth import get_config

    torch.cuda.set_device(0)
    if args.tiered:
        tiered(torch, B)
        return
    if args.block:
        block(torch, B)
        return
    if args.reread:
        reread(torch, B)
        return
    if args.crossover:
        rows = tuple(int(v) for v in args.crossover_rows.split(",")) if args.crossover_rows else CROSS_ROWS
        modes = tuple(args.crossover_modes.split(",")) if args.crossover_modes else tuple(CROSS_MODES)
        crossover(torch, B, rows=rows, modes=modes, formats=args.crossover_formats)
        return
    layers = args.layers or get_config(args.workload).layers
    head, cfg = measure(args.workload, layers, args.steps, args.warmup, torch, B, eager=args.eager)
    log(f"{args.workload}: {head['us_per_layer']} us/layer")
    line = {
        "metric": METRIC,
        "value": head["us_per_layer"],
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.x_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "layers_cycled": layers, "launch": head["launch"],
                   "weights": "random int4, seeded", "untimed_steps_before": head["untimed_steps_before"]},
    }
    for k in ("expert_weight_bytes_per_layer", "expert_weight_GBps_layer", "expert_weight_pct_hbm_peak_layer",
              "expert_weight_GBps_kernels", "kernel_us", "down_GBps", "down_pct_hbm_peak", "plain_read"):
        if k in head:
            line[k] = head[k]
    line["roofline"] = head["roofline"]
    if not args.no_secondary:
        line["secondary"] = {}
        for name, (nl, st) in SECONDARY.items():
            if name == args.workload:
                continue
            res, _ = measure(name, nl, st, max(2 * nl, 8), torch, B)
            log(f"{name}: {res['us_per_layer']} us/layer")
            line["secondary"][name] = res
    if not args.no_cpu:
        log("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(cfg, layers)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
