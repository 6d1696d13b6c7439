"""The five workloads the path is built and measured on.

Shapes follow the model the pages run (GLM-5.2-like decode MoE: model dim D,
expert intermediate I, E routed experts, top-K).  Router settings that a
workload leaves unstated default to: W_r ~ N(0, 0.02), bias ~ N(0, 0.1),
norm_topk on, routed_scale 1.0, top-p off.  Expert row/group scales are
lognormal(ln 0.01, 0.5) everywhere.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

FMT_ROW = 2      # per-row int4: one f32 scale per output row
FMT_GROUP = 4    # group-wise int4: one f32 scale per (row, column group)


@dataclass(frozen=True)
class Config:
    name: str
    D: int                 # model dim (gate/up columns, down rows)
    I: int                 # expert intermediate (gate/up rows, down columns)
    E: int                 # routed experts per layer
    K: int                 # top-K
    S: int                 # tokens per decode step
    formats: str           # "row" | "group" | "mix_even_odd" | "mix_halves"
    gs: int                # group size for group-wise experts (0 for per-row only)
    x_dtype: str           # "f32" | "bf16"
    topp: float            # 0 => off
    norm_topk: bool
    routed_scale: float
    seed: int
    layers: int = 1        # distinct layers (weights) a benchmark cycles through
    router_w_std: float = 0.02
    router_b_std: float = 0.1
    scale_mu: float = -4.605170185988091   # ln(0.01)
    scale_sigma: float = 0.5
    notes: str = field(default="", compare=False)

    @property
    def max_rows(self) -> int:
        return self.S * self.K


CONFIGS = {
    "tiny": Config(
        name="tiny", D=256, I=128, E=8, K=2, S=1, formats="row", gs=0,
        x_dtype="f32", topp=0.0, norm_topk=True, routed_scale=1.0, seed=0,
        notes="launch-bound smoke case"),
    "medium": Config(
        name="medium", D=4096, I=1536, E=64, K=8, S=1, formats="row", gs=0,
        x_dtype="bf16", topp=0.95, norm_topk=True, routed_scale=2.5, seed=1,
        layers=8, notes="decode S=1, per-row int4, bf16 activations"),
    "mix": Config(
        name="mix", D=4096, I=2000, E=64, K=8, S=1, formats="mix_even_odd", gs=64,
        x_dtype="f32", topp=0.0, norm_topk=True, routed_scale=1.0, seed=2,
        layers=8, notes="even experts g64, odd per-row; down has a 16-wide tail group"),
    "small_batch": Config(
        name="small_batch", D=6144, I=2048, E=256, K=8, S=4, formats="group", gs=64,
        x_dtype="bf16", topp=0.0, norm_topk=True, routed_scale=2.5, seed=3,
        layers=2, notes="S=4 union of up to 32 distinct experts, 1-4 rows each"),
    "sustained": Config(
        name="sustained", D=7168, I=2048, E=64, K=64, S=1, formats="mix_halves", gs=64,
        x_dtype="f32", topp=0.0, norm_topk=True, routed_scale=1.0, seed=4,
        layers=16, notes="all 64 experts taken per launch; experts 0-31 g64, 32-63 per-row"),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg
