"""The GPU tests' helpers on the CPU: the threaded evaluation of the oracle's layer delta is the
oracle's own result bit for bit, and GPU route records convert to the oracle's route form."""

from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import pytest

import oracle
from harness import gpu_routes, layer_delta_threads, make_layer, oracle_routes
from synth import get_config


@pytest.mark.parametrize("name,over", [("tiny", {}), ("mix", {"D": 512, "I": 200, "E": 16, "K": 4, "S": 3})])
def test_threaded_layer_delta_is_the_oracle(name, over):
    cfg = get_config(name, **over)
    L = make_layer(cfg, 0)
    routes, x64 = oracle_routes(cfg, L)
    d0, i0 = oracle.experts.layer_delta(routes, L.expert, x64)
    d1, i1 = layer_delta_threads(routes, L.expert, x64)
    assert d0.tobytes() == d1.tobytes()
    assert i0.keys() == i1.keys()
    for key in i0:
        for a, b in zip(i0[key], i1[key]):
            assert a.tobytes() == b.tobytes()


def test_gpu_route_records_convert():
    rec = [SimpleNamespace(n=2, idx=[5, 1, 3] + [0] * 61, w=[0.5, 0.25, 0.0] + [0.0] * 61)]
    r = gpu_routes(rec, 1, 3)[0]
    assert r.n == 2 and r.idx == [5, 1, 3]
    assert r.w32.dtype == np.float32 and r.w32.tolist() == [0.5, 0.25, 0.0]
    g = oracle.build_group([r])
    assert g["entries"] == [5, 1] and g["token_rows"] == [[0, 1]]
