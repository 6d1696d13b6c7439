"""The CPU tier's arithmetic through the C ABI, on the host only (i4moe_host_rows: no device is
touched): against the f64 oracle on per-row and group-wise experts with a tail group, bitwise the
same at every worker count, and its argument checks."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from harness import normwise_err
from synth import get_config
from synth.gen import gen_expert


@pytest.fixture(scope="module")
def lib():
    from int4_grouped_expert_router_amd import binding as B
    return B.load()


def case(S=3):
    # D=256 and I=200: the down rows' last group (gs=64) is 8 columns wide; even experts g64, odd per-row
    cfg = get_config("mix", D=256, I=200, E=4, layers=1)
    ex = {e: gen_expert(cfg, 0, e) for e in range(cfg.E)}
    rng = np.random.default_rng(77)
    x = rng.standard_normal((S, cfg.D)).astype(np.float32)
    plan = [(0, 0, 0.75), (1, 0, 0.25), (2, 1, 1.0), (3, 2, 0.5), (0, 2, 0.125), (2, 2, 2.0)]
    rows = [(t, w, ex[e].gate, ex[e].up, ex[e].down) for e, t, w in plan]
    return cfg, ex, x, plan, rows


def test_host_rows_match_oracle(lib):
    from int4_grouped_expert_router_amd import host_rows
    cfg, ex, x, plan, rows = case()
    P = host_rows(3, cfg.D, cfg.I, rows, x, threads=4)
    ref = np.zeros((3, cfg.D))
    for e, t, w in plan:
        ref[t] += float(np.float32(w)) * oracle.expert_forward(ex[e].gate, ex[e].up, ex[e].down, x[t].astype(np.float64))[3]
    for t in range(3):
        # float32 sums over at most 256 columns: far inside the 1e-4 bar
        assert normwise_err(P[t], ref[t]) < 1e-5, t


def test_host_rows_same_bits_at_every_thread_count(lib):
    from int4_grouped_expert_router_amd import host_rows
    cfg, ex, x, plan, rows = case()
    base = host_rows(3, cfg.D, cfg.I, rows, x, threads=1)
    for n in (2, 3, 7, 16):
        assert np.array_equal(host_rows(3, cfg.D, cfg.I, rows, x, threads=n), base), n
    # no rows: P stays zero
    assert not np.any(host_rows(3, cfg.D, cfg.I, [], x, threads=2))


def test_host_rows_refuses_bad_arguments(lib):
    from types import SimpleNamespace

    from int4_grouped_expert_router_amd import I4moeError, host_rows
    from int4_grouped_expert_router_amd import binding as B
    cfg, ex, x, plan, rows = case()
    with pytest.raises(I4moeError) as e1:
        host_rows(3, cfg.D, cfg.I, [(3, 1.0) + rows[0][2:]], x)  # token 3 of S = 3
    assert e1.value.code == B.I4MOE_EINVAL
    with pytest.raises(I4moeError) as e2:
        host_rows(3, cfg.D, cfg.I, [(0, float("nan")) + rows[0][2:]], x)
    assert e2.value.code == B.I4MOE_EINVAL
    g = rows[0][2]
    bad_fmt = SimpleNamespace(fmt=3, gs=0, O=g.O, C=g.C, packed=g.packed, scales=g.scales)
    with pytest.raises(I4moeError) as e3:
        host_rows(3, cfg.D, cfg.I, [(0, 1.0, bad_fmt) + rows[0][3:]], x)
    assert e3.value.code == B.I4MOE_EUNSUPPORTED
    with pytest.raises(I4moeError) as e4:  # gate given where down belongs: shape mismatch
        host_rows(3, cfg.D, cfg.I, [(0, 1.0, g, g, g)], x)
    assert e4.value.code == B.I4MOE_EINVAL
    assert B.i4moe_host_rows(0, 8, 8, 0, None, None, None, None, None, None, None, 1) == B.I4MOE_EINVAL


# (D, I, formats, gs), each reaching one form of the integer path's dot product: one 64-column
# block per group, groups of two blocks (digit sums joined in int32), of five blocks and whole
# rows (joined in double); D = 1000 and I = 392 end in a partial block (40 and 8 columns).  g32
# takes the float32 path on every host.
SHAPES = [(1000, 392, "group", 64), (1000, 392, "group", 128), (1000, 392, "group", 320),
          (1000, 392, "row", 0), (256, 200, "group", 32)]


def shaped_case(D, I, formats, gs):
    cfg = get_config("mix", D=D, I=I, E=3, formats=formats, gs=gs, layers=1)
    ex = {e: gen_expert(cfg, 0, e) for e in range(cfg.E)}
    rng = np.random.default_rng(D + I + gs)
    x = rng.standard_normal((4, D)).astype(np.float32)
    x[1] *= np.float32(1e-6)        # the fixed point follows each row's own magnitude
    x[2, 17] = np.float32(3e4)      # one large column: the rest keep fewer bits
    x[3] = 0.0                      # an all-zero row
    plan = [(0, 0, 0.75), (1, 0, 1.5), (2, 1, 0.5), (0, 2, 0.25), (2, 3, 1.0), (1, 1, 2.0)]
    rows = [(t, w, ex[e].gate, ex[e].up, ex[e].down) for e, t, w in plan]
    ref = np.zeros((4, D))
    for e, t, w in plan:
        ref[t] += float(np.float32(w)) * oracle.expert_forward(ex[e].gate, ex[e].up, ex[e].down,
                                                               x[t].astype(np.float64))[3]
    return cfg, x, rows, ref


@pytest.mark.parametrize("path", ["int", "float"])
@pytest.mark.parametrize("D,I,formats,gs", SHAPES)
def test_host_rows_paths_match_oracle(lib, monkeypatch, D, I, formats, gs, path):
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd import host_rows
    monkeypatch.setenv("I4MOE_HOST_INT", "1" if path == "int" else "0")
    if path == "int" and not B.i4moe_host_int_path():
        pytest.skip("no AVX-512 VNNI on this host")
    cfg, x, rows, ref = shaped_case(D, I, formats, gs)
    P = host_rows(4, D, I, rows, x, threads=3)
    for t in range(3):
        # 24-bit activations and float32 SiLU: about 1e-7 of the output's norm
        assert normwise_err(P[t], ref[t]) < 1e-5, (t, path)
    assert not np.any(P[3])  # no row routes token 3
    assert np.array_equal(host_rows(4, D, I, rows, x, threads=1), P)


def test_host_int_path_query(lib, monkeypatch):
    from int4_grouped_expert_router_amd import binding as B
    with open("/proc/cpuinfo") as f:
        flags = next((ln.split(":", 1)[1].split() for ln in f if ln.startswith("flags")), [])
    has = all(fl in flags for fl in ("avx512f", "avx512bw", "avx512vl", "avx512_vnni"))
    monkeypatch.setenv("I4MOE_HOST_INT", "1")
    assert B.i4moe_host_int_path() == int(has)
    monkeypatch.setenv("I4MOE_HOST_INT", "0")
    assert B.i4moe_host_int_path() == 0


@pytest.mark.parametrize("D,I,formats,gs", SHAPES[:4])
def test_host_rows_shared_expert_same_bits_as_alone(lib, D, I, formats, gs):
    """Rows naming the same tensors are one expert, computed together (on the integer path, four
    activation rows per pass over a weight row): each row's result is the same bits as when it
    is computed alone.  One row per token with weight 1, so P[t] is that row's output exactly."""
    from int4_grouped_expert_router_amd import host_rows
    cfg = get_config("mix", D=D, I=I, E=2, formats=formats, gs=gs, layers=1)
    ex = [gen_expert(cfg, 0, e) for e in range(2)]
    x = np.random.default_rng(5).standard_normal((7, D)).astype(np.float32)
    plan = [0, 0, 0, 0, 0, 0, 1]  # token t -> expert: six rows of expert 0 (4 + 2), one of expert 1
    rows = [(t, 1.0, ex[e].gate, ex[e].up, ex[e].down) for t, e in enumerate(plan)]
    P = host_rows(7, D, I, rows, x, threads=4)
    for t, e in enumerate(plan):
        alone = host_rows(1, D, I, [(0, 1.0, ex[e].gate, ex[e].up, ex[e].down)], x[t:t + 1], threads=2)
        assert np.array_equal(P[t], alone[0]), t
        ref = oracle.expert_forward(ex[e].gate, ex[e].up, ex[e].down, x[t].astype(np.float64))[3]
        assert normwise_err(P[t], ref) < 1e-5, t


@pytest.mark.parametrize("D,I,formats,gs", SHAPES[:4])
def test_host_int_widths_same_bits(lib, monkeypatch, D, I, formats, gs):
    """The integer path's 512-bit form (per-row, g64 and multiples of 128) and its 256-bit form
    (I4MOE_HOST_INT=256) do the same integer sums and the same double operations in the same
    order: the same bits, shared experts included."""
    from int4_grouped_expert_router_amd import binding as B
    from int4_grouped_expert_router_amd import host_rows
    monkeypatch.delenv("I4MOE_HOST_INT", raising=False)
    if not B.i4moe_host_int_path():
        pytest.skip("no AVX-512 VNNI on this host")
    cfg, x, rows, ref = shaped_case(D, I, formats, gs)
    wide = host_rows(4, D, I, rows, x, threads=3)
    monkeypatch.setenv("I4MOE_HOST_INT", "256")
    assert np.array_equal(host_rows(4, D, I, rows, x, threads=2), wide)


@pytest.mark.parametrize("path", ["int", "float"])
def test_host_rows_nonfinite_x_is_not_an_error(lib, monkeypatch, path):
    """Non-finite activations give unspecified values (the header says so), never an error or
    a fault, on either path; the other tokens' rows are unaffected."""
    from int4_grouped_expert_router_amd import host_rows
    monkeypatch.setenv("I4MOE_HOST_INT", "1" if path == "int" else "0")
    cfg, x, rows, ref = shaped_case(1000, 392, "group", 64)
    clean = host_rows(4, 1000, 392, rows, x, threads=2)
    xb = x.copy()
    xb[1, 3], xb[1, 700] = np.nan, np.inf
    P = host_rows(4, 1000, 392, rows, xb, threads=2)
    for t in (0, 2, 3):  # token 1 alone has the bad values
        assert np.array_equal(P[t], clean[t]), t
