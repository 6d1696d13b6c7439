"""Seeded generators.

Every random stream is keyed by (config seed, layer, role[, expert]) through
``numpy.random.SeedSequence`` spawn keys, so any one expert of any layer can be
drawn on its own, in any order, with the same bytes every time.

Host formats produced here (the library's upload format and the oracle's input
format are the same thing):

* int4 tensor, O rows x C columns: ``packed`` uint8 [O, C // 2]; the byte at
  [o, c // 2] holds column c in its low nibble when c is even, in its high
  nibble when c is odd.  Bytes are drawn i.i.d. uniform over 0..255, which is
  the same as drawing every nibble i.i.d. uniform over 0..15.
* scales: float32, O of them (per-row) or O * ceil(C / gs) row-major
  (group-wise), lognormal.
* activations: float32 [S, D], or for bf16 workloads the uint16 bit patterns
  of the float32 draws rounded to bf16 (round to nearest, ties to even).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

from .configs import FMT_GROUP, FMT_ROW, Config

ROLE_ROUTER = 0
ROLE_EXPERT = 1
ROLE_ACT = 2
ROLE_RESID = 3
ROLE_SHARED = 4
ROLE_NORM = 5


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def round_f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bit patterns.

    Input preparation only: finite inputs are assumed (the draws are normal)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


@dataclass
class TensorHost:
    fmt: int
    gs: int
    O: int
    C: int
    packed: np.ndarray   # uint8 [O, C//2]
    scales: np.ndarray   # float32 [O] or [O * ceil(C/gs)]

    @property
    def nbytes_algorithmic(self) -> int:
        return self.packed.nbytes + self.scales.nbytes


@dataclass
class ExpertWeights:
    gate: TensorHost
    up: TensorHost
    down: TensorHost

    @property
    def nbytes_algorithmic(self) -> int:
        return self.gate.nbytes_algorithmic + self.up.nbytes_algorithmic + self.down.nbytes_algorithmic


def expert_format(cfg: Config, e: int):
    """(fmt, gs) of expert e under the workload's format mix."""
    if cfg.formats == "row":
        return FMT_ROW, 0
    if cfg.formats == "group":
        return FMT_GROUP, cfg.gs
    if cfg.formats == "mix_even_odd":
        return (FMT_GROUP, cfg.gs) if e % 2 == 0 else (FMT_ROW, 0)
    if cfg.formats == "mix_halves":
        return (FMT_GROUP, cfg.gs) if e < cfg.E // 2 else (FMT_ROW, 0)
    raise ValueError(f"unknown format mix {cfg.formats!r}")


def _n_scales(fmt: int, gs: int, O: int, C: int) -> int:
    if fmt == FMT_GROUP and gs > 0:
        return O * (-(-C // gs))
    return O


def _tensor(rng: np.random.Generator, cfg: Config, fmt: int, gs: int, O: int, C: int) -> TensorHost:
    packed = np.frombuffer(rng.bytes(O * (C // 2)), dtype=np.uint8).reshape(O, C // 2).copy()
    scales = rng.lognormal(cfg.scale_mu, cfg.scale_sigma, _n_scales(fmt, gs, O, C)).astype(np.float32)
    return TensorHost(fmt=fmt, gs=gs, O=O, C=C, packed=packed, scales=scales)


def gen_expert(cfg: Config, layer: int, e: int) -> ExpertWeights:
    fmt, gs = expert_format(cfg, e)
    rng = _rng(cfg.seed, layer, ROLE_EXPERT, e)
    gate = _tensor(rng, cfg, fmt, gs, cfg.I, cfg.D)
    up = _tensor(rng, cfg, fmt, gs, cfg.I, cfg.D)
    down = _tensor(rng, cfg, fmt, gs, cfg.D, cfg.I)
    return ExpertWeights(gate, up, down)


def gen_shared_expert(cfg: Config, layer: int) -> ExpertWeights:
    """The layer's shared expert: the same shapes as a routed expert; group-wise when the workload
    has group-wise experts at all, else per-row."""
    fmt, gs = (FMT_ROW, 0) if cfg.formats == "row" else (FMT_GROUP, cfg.gs)
    rng = _rng(cfg.seed, layer, ROLE_SHARED)
    gate = _tensor(rng, cfg, fmt, gs, cfg.I, cfg.D)
    up = _tensor(rng, cfg, fmt, gs, cfg.I, cfg.D)
    down = _tensor(rng, cfg, fmt, gs, cfg.D, cfg.I)
    return ExpertWeights(gate, up, down)


def gen_norm(cfg: Config, layer: int) -> np.ndarray:
    """rmsnorm weights gamma ~ N(1, 0.1), float32 [D]."""
    rng = _rng(cfg.seed, layer, ROLE_NORM)
    return rng.normal(1.0, 0.1, cfg.D).astype(np.float32)


def gen_router(cfg: Config, layer: int):
    rng = _rng(cfg.seed, layer, ROLE_ROUTER)
    W = rng.normal(0.0, cfg.router_w_std, (cfg.E, cfg.D)).astype(np.float32)
    b = rng.normal(0.0, cfg.router_b_std, cfg.E).astype(np.float32)
    return W, b


def gen_activations(cfg: Config, layer: int, S: Optional[int] = None):
    """Returns (x, dtype) with x float32 [S, D] or uint16 bf16 bits [S, D]."""
    S = cfg.S if S is None else S
    rng = _rng(cfg.seed, layer, ROLE_ACT)
    x = rng.standard_normal((S, cfg.D)).astype(np.float32)
    if cfg.x_dtype == "bf16":
        return round_f32_to_bf16_bits(x), "bf16"
    return x, "f32"


def gen_residual(cfg: Config, layer: int, S: Optional[int] = None) -> np.ndarray:
    S = cfg.S if S is None else S
    rng = _rng(cfg.seed, layer, ROLE_RESID)
    return rng.standard_normal((S, cfg.D)).astype(np.float32)


@dataclass
class LayerInputs:
    cfg: Config
    layer: int
    router_W: np.ndarray
    router_b: np.ndarray
    x: np.ndarray
    x_dtype: str
    residual: np.ndarray
    _experts: Dict[int, ExpertWeights] = field(default_factory=dict, repr=False)

    def expert(self, e: int) -> ExpertWeights:
        if e not in self._experts:
            self._experts[e] = gen_expert(self.cfg, self.layer, e)
        return self._experts[e]

    def drop_experts(self):
        self._experts.clear()


def gen_layer(cfg: Config, layer: int = 0) -> LayerInputs:
    W, b = gen_router(cfg, layer)
    x, dt = gen_activations(cfg, layer)
    r = gen_residual(cfg, layer)
    return LayerInputs(cfg=cfg, layer=layer, router_W=W, router_b=b, x=x, x_dtype=dt, residual=r)
