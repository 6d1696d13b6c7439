"""The C ABI without a GPU: every function include/i4moe.h declares is exported by
libi4moe.so and bound by the Python binding under the same name, and the constants agree.
No compute call is made."""

from __future__ import annotations

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i4moe.h")


def _strip_comments(text: str) -> str:
    return re.sub(r"/\*.*?\*/", " ", text, flags=re.S)


def header_functions() -> list[str]:
    body = _strip_comments(open(HEADER).read())
    return sorted(set(re.findall(r"\b(i4moe_[a-z_]+)\s*\(", body)))


def header_constants() -> dict[str, int]:
    body = _strip_comments(open(HEADER).read())
    out = {}
    for name, expr in re.findall(r"#define\s+(I4MOE_[A-Z0-9_]+)\s+([^\n]+)", body):
        if name != "I4MOE_H":
            out[name] = eval(expr, {"__builtins__": {}})  # integer literals and + only
    for block in re.findall(r"enum\s*\{([^}]*)\}", body):
        for name, val in re.findall(r"(I4MOE_[A-Z0-9_]+)\s*=\s*(-?\d+)", block):
            out[name] = int(val)
    return out


@pytest.fixture(scope="module")
def lib_path():
    from int4_grouped_expert_router_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from int4_grouped_expert_router_amd.build import build_library
        build_library()
    return binding.LIB_PATH


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("i4moe_upload_expert_tensor", "i4moe_route", "i4moe_expert_group_issue",
                     "i4moe_expert_group_take"):
        assert required in names


def test_library_exports_every_declared_function(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], check=True, capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in header_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    # the C ABI is unmangled: nothing declared is exported only under a C++ name
    assert not [n for n in exported if n.startswith("_Z") and "i4moe_" in n and "i4moe_ctx" not in n]


def test_library_loads_and_binding_matches_header(lib_path):
    from int4_grouped_expert_router_amd import binding
    lib = binding.load(lib_path)
    assert sorted(binding.SIGNATURES) == header_functions()
    for name in header_functions():
        assert callable(getattr(lib, name))
        assert callable(getattr(binding, name))


def test_constants_match_header():
    from int4_grouped_expert_router_amd import binding
    consts = header_constants()
    assert consts, "no constants parsed"
    for name, val in consts.items():
        assert getattr(binding, name) == val, name


def test_null_context_rejected_before_any_device_call(lib_path):
    """Every entry point refuses a NULL context (or output pointer) with its documented error
    value before it touches the HIP runtime, so these calls are safe without a GPU."""
    import ctypes as C

    from int4_grouped_expert_router_amd import binding as B
    B.load(lib_path)
    EINVAL, OK = B.I4MOE_EINVAL, B.I4MOE_OK
    assert B.i4moe_ctx_create(0, None) == EINVAL
    assert B.i4moe_ctx_destroy(None) == OK
    assert B.i4moe_set_stream(None, None) == EINVAL
    assert B.i4moe_last_error(None)  # static text, never NULL
    assert B.i4moe_upload_expert_tensor(None, 2, 0, 16, 16, None, None) == 0  # handle 0: not uploaded
    assert B.i4moe_tensor_free(None, 1) == EINVAL
    assert B.i4moe_set_expert(None, 0, 0, 1, 2, 3) == EINVAL
    assert B.i4moe_upload_router(None, 0, 8, 16, None, None) == EINVAL
    assert B.i4moe_route(None, 0, None, 0, 1, 1, 0.0, 1, 1.0, None) == EINVAL
    assert B.i4moe_route_noalloc(None, 0, None, 0, 1, 1, 0.0, 1, 1.0, None) == EINVAL
    assert B.i4moe_expert_group_issue(None, 0, None, 0, 1, None) == EINVAL
    assert B.i4moe_expert_group_take(None, None, 1) == EINVAL
    assert B.i4moe_set_shared_expert(None, 0, 1, 2, 3) == EINVAL
    assert B.i4moe_upload_norm(None, 0, 8, None, 1e-5) == EINVAL
    assert B.i4moe_rmsnorm(None, 0, None, 8, 1, None, 8, 0) == EINVAL
    assert B.i4moe_shared_expert_issue(None, 0, None, 0, 1) == EINVAL
    assert B.i4moe_moe_block(None, 0, None, 1, 0, 1, 0.0, 1, 1.0) == EINVAL
    assert B.i4moe_set_host_expert(None, 0, 0, None, None, None) == EINVAL
    assert B.i4moe_tiered_issue(None, 0, None, 0, 1, None, None) == EINVAL
    assert B.i4moe_set_fail_after(None, 0) == EINVAL
    buf = (C.c_char * 8)()
    assert B.i4moe_debug_read(None, 0, 0, C.cast(buf, C.c_void_p), 8) == EINVAL
    assert B.i4moe_debug_size(None, 0, 0) == 0
    assert B.i4moe_set_profiling(None, 1) == EINVAL
    ms, n = C.c_double(), C.c_longlong()
    assert B.i4moe_profile_query(None, 0, C.byref(ms), C.byref(n)) == EINVAL
    ex = (C.c_int32 * 1)(0)
    assert B.i4moe_read_probe(None, 0, 3, 1, ex) == EINVAL
