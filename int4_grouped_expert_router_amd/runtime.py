"""Thin Python wrapper over the C ABI: owns a context, turns status codes into exceptions,
passes numpy host arrays and torch device tensors through.  No computation happens here."""

from __future__ import annotations

import ctypes as C

import numpy as np

from . import binding as B


class I4moeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"i4moe error {code}: {msg}")
        self.code = code


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return B.I4MOE_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return B.I4MOE_DTYPE_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def host_rows(S: int, D: int, I: int, rows, x: np.ndarray, threads: int = 1) -> np.ndarray:
    """The CPU tier's arithmetic alone (i4moe_host_rows; host only): rows is a list of
    (token, weight, gate, up, down) with host tensors; x is S x D float32.  Returns P (S x D)."""
    n = len(rows)
    x = np.ascontiguousarray(x, dtype=np.float32)
    P = np.zeros((S, D), dtype=np.float32)
    keep = []

    def desc(t):
        packed = np.ascontiguousarray(t.packed, dtype=np.uint8)
        scales = np.ascontiguousarray(t.scales, dtype=np.float32)
        keep.append((packed, scales))
        return B.i4moe_host_tensor(t.fmt, t.gs, t.O, t.C, _ptr(packed), _ptr(scales))

    tok = np.array([r[0] for r in rows] or [0], dtype=np.int32)
    wt = np.array([r[1] for r in rows] or [0.0], dtype=np.float32)
    g = (B.i4moe_host_tensor * max(n, 1))(*[desc(r[2]) for r in rows])
    u = (B.i4moe_host_tensor * max(n, 1))(*[desc(r[3]) for r in rows])
    d = (B.i4moe_host_tensor * max(n, 1))(*[desc(r[4]) for r in rows])
    rc = B.i4moe_host_rows(S, D, I, n, _ptr(tok), _ptr(wt), g, u, d, _ptr(x), _ptr(P), threads)
    if rc < 0:
        raise I4moeError(rc, "i4moe_host_rows refused its arguments")
    return P


class Context:
    def __init__(self, device: int = 0, stream=None):
        B.load()
        p = C.c_void_p()
        rc = B.i4moe_ctx_create(device, C.byref(p))
        if rc != 0:
            raise I4moeError(rc, "i4moe_ctx_create failed")
        self.p = p
        self.device = device
        if stream is not None:
            self.set_stream(stream)

    # -- plumbing
    def check(self, rc: int) -> int:
        if rc < 0:
            raise I4moeError(rc, B.i4moe_last_error(self.p).decode())
        return rc

    def last_error(self) -> str:
        return B.i4moe_last_error(self.p).decode()

    def close(self):
        if self.p:
            B.i4moe_ctx_destroy(self.p)
            self.p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_stream(self, stream):
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream or 0)
        self.check(B.i4moe_set_stream(self.p, C.c_void_p(handle)))

    # -- weights
    def upload_tensor(self, fmt: int, gs: int, O: int, C_: int, packed: np.ndarray, scales: np.ndarray) -> int:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        h = B.i4moe_upload_expert_tensor(self.p, fmt, gs, O, C_, _ptr(packed), _ptr(scales))
        if h == 0:
            raise I4moeError(-1, self.last_error())
        return h

    def upload_host_tensor(self, t) -> int:
        return self.upload_tensor(t.fmt, t.gs, t.O, t.C, t.packed, t.scales)

    def free_tensor(self, h: int):
        self.check(B.i4moe_tensor_free(self.p, h))

    def set_expert(self, layer: int, e: int, gate: int, up: int, down: int):
        self.check(B.i4moe_set_expert(self.p, layer, e, gate, up, down))

    def upload_router(self, layer: int, W: np.ndarray, bias=None):
        W = np.ascontiguousarray(W, dtype=np.float32)
        E, D = W.shape
        bp = None
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            bp = _ptr(bias)
        self.check(B.i4moe_upload_router(self.p, layer, E, D, _ptr(W), bp))

    # -- compute
    def route(self, layer: int, x, K: int, topp: float = 0.0, norm_topk: bool = True, routed_scale: float = 1.0,
              host_out: bool = False):
        S = x.shape[0]
        out = (B.i4moe_route_host * S)() if host_out else None
        self.check(B.i4moe_route(self.p, layer, C.c_void_p(x.data_ptr()), _dtype_code(x), S, K, topp,
                                 1 if norm_topk else 0, routed_scale,
                                 C.cast(out, C.POINTER(B.i4moe_route_host)) if out is not None else None))
        return out

    def route_noalloc(self, layer: int, x, K: int, topp: float, norm_topk: bool, routed_scale: float, out):
        """The route into `out`, a device tensor of S * sizeof(i4moe_route_host) bytes, with the
        library's static scratch (no allocation)."""
        S = x.shape[0]
        if out.numel() * out.element_size() < S * C.sizeof(B.i4moe_route_host):
            raise ValueError("out too small for S route records")
        self.check(B.i4moe_route_noalloc(self.p, layer, C.c_void_p(x.data_ptr()), _dtype_code(x), S, K, topp,
                                         1 if norm_topk else 0, routed_scale, C.c_void_p(out.data_ptr())))

    def issue(self, layer: int, x, rows=None) -> int:
        """rows: None (device route of the layer) or a list of (expert, token, weight)."""
        S = x.shape[0]
        g = None
        if rows is not None:
            n = len(rows)
            ex = (C.c_int32 * max(n, 1))(*[int(r[0]) for r in rows])
            tk = (C.c_int32 * max(n, 1))(*[int(r[1]) for r in rows])
            wt = (C.c_float * max(n, 1))(*[float(r[2]) for r in rows])
            g = B.i4moe_group(n, ex, tk, wt)
            self._keep = (ex, tk, wt)
        return self.check(B.i4moe_expert_group_issue(self.p, layer, C.c_void_p(x.data_ptr()), _dtype_code(x), S,
                                                     C.byref(g) if g is not None else None))

    def take(self, residual):
        import torch
        if residual.dtype != torch.float32 or not residual.is_contiguous():
            raise TypeError("residual must be a contiguous float32 device tensor")
        self.check(B.i4moe_expert_group_take(self.p, C.c_void_p(residual.data_ptr()), residual.shape[0]))

    def set_shared_expert(self, layer: int, gate: int, up: int, down: int):
        self.check(B.i4moe_set_shared_expert(self.p, layer, gate, up, down))

    def upload_norm(self, layer: int, gamma: np.ndarray, eps: float):
        gamma = np.ascontiguousarray(gamma, dtype=np.float32)
        self.check(B.i4moe_upload_norm(self.p, layer, gamma.shape[0], _ptr(gamma), eps))

    def rmsnorm(self, layer: int, x, out, ld_x: int = 0, ld_out: int = 0):
        """x: float32 device rows [S][>= D]; out: float32 or bfloat16 device rows [S][>= D]."""
        S = x.shape[0]
        self.check(B.i4moe_rmsnorm(self.p, layer, C.c_void_p(x.data_ptr()), ld_x or x.shape[1], S,
                                   C.c_void_p(out.data_ptr()), ld_out or out.shape[1], _dtype_code(out)))

    def shared_issue(self, layer: int, x) -> int:
        return self.check(B.i4moe_shared_expert_issue(self.p, layer, C.c_void_p(x.data_ptr()), _dtype_code(x),
                                                      x.shape[0]))

    def moe_block(self, layer: int, residual, act_dtype: int, K: int, topp: float = 0.0, norm_topk: bool = True,
                  routed_scale: float = 1.0):
        import torch
        if residual.dtype != torch.float32 or not residual.is_contiguous():
            raise TypeError("residual must be a contiguous float32 device tensor")
        self.check(B.i4moe_moe_block(self.p, layer, C.c_void_p(residual.data_ptr()), residual.shape[0], act_dtype, K,
                                     topp, 1 if norm_topk else 0, routed_scale))

    def set_host_expert(self, layer: int, e: int, gate, up, down):
        """Keep expert e of `layer` on the host: gate/up/down are host tensors (fmt, gs, O, C,
        packed uint8 [O][C/2], scales float32), copied by the library."""
        keep = []

        def desc(t):
            packed = np.ascontiguousarray(t.packed, dtype=np.uint8)
            scales = np.ascontiguousarray(t.scales, dtype=np.float32)
            keep.append((packed, scales))
            return B.i4moe_host_tensor(t.fmt, t.gs, t.O, t.C, _ptr(packed), _ptr(scales))

        g, u, d = desc(gate), desc(up), desc(down)
        self.check(B.i4moe_set_host_expert(self.p, layer, e, C.byref(g), C.byref(u), C.byref(d)))

    def tiered_issue(self, layer: int, x, routes):
        """Device rows as a device group, host rows on the CPU meanwhile (see i4moe_tiered_issue);
        routes: S route records (i4moe_route_host).  Returns (slots issued, timings)."""
        S = x.shape[0]
        if len(routes) < S:
            raise ValueError("need S route records")
        arr = (B.i4moe_route_host * S)(*routes[:S])
        times = B.i4moe_tier_times()
        n = self.check(B.i4moe_tiered_issue(self.p, layer, C.c_void_p(x.data_ptr()), _dtype_code(x), S, arr,
                                            C.byref(times)))
        return n, times

    def set_fail_after(self, n: int):
        self.check(B.i4moe_set_fail_after(self.p, n))

    # -- taps and profiling
    def tap(self, what: int, index: int = 0, dtype=np.float32) -> np.ndarray:
        n = B.i4moe_debug_size(self.p, what, index)
        if n == 0:
            raise I4moeError(-1, f"tap {what}/{index} unavailable")
        buf = np.empty(n // np.dtype(dtype).itemsize, dtype=dtype)
        self.check(B.i4moe_debug_read(self.p, what, index, _ptr(buf), n))
        return buf

    def tap_group(self, layer: int) -> dict:
        w = self.tap(B.I4MOE_TAP_GROUP, layer, np.int32)
        o = 4
        rec = {"n_entries": int(w[0]), "n_rows": int(w[1]), "S": int(w[2])}
        for name, n in [("entry_expert", 64), ("entry_row0", 65), ("row_token", 64), ("row_expert", 64),
                        ("row_weight", 64), ("tok_row0", 65), ("red_rows", 64)]:
            rec[name] = w[o:o + n].copy()
            o += n
        rec["row_weight"] = rec["row_weight"].view(np.float32)
        return rec

    def set_profiling(self, on: bool):
        self.check(B.i4moe_set_profiling(self.p, 1 if on else 0))

    def profile(self, kernel: int):
        ms = C.c_double()
        n = C.c_longlong()
        self.check(B.i4moe_profile_query(self.p, kernel, C.byref(ms), C.byref(n)))
        return ms.value, n.value

    def read_probe(self, layer: int, tensor_mask: int, experts):
        """Enqueue the plain read of the listed experts' tensors (see i4moe_read_probe)."""
        arr = (C.c_int32 * len(experts))(*[int(e) for e in experts])
        self.check(B.i4moe_read_probe(self.p, layer, tensor_mask, len(experts), arr))
