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
