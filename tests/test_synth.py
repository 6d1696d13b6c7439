"""Seeded input generators: determinism, independence of draw order, bf16 rounding, shapes."""

import numpy as np

from synth import CONFIGS, expert_format, gen_expert, gen_layer, get_config, round_f32_to_bf16_bits


def test_bf16_rounding_ties_to_even():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -7 + 2 ** -9], np.float32)
    assert round_f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_expert_draws_do_not_depend_on_order():
    cfg = get_config("tiny")
    a = gen_expert(cfg, 0, 5)
    gen_expert(cfg, 0, 1)
    b = gen_expert(cfg, 0, 5)
    assert np.array_equal(a.down.packed, b.down.packed) and np.array_equal(a.gate.scales, b.gate.scales)
    c = gen_expert(cfg, 1, 5)
    assert not np.array_equal(a.gate.packed, c.gate.packed)


def test_layer_shapes_and_formats():
    for name, cfg in CONFIGS.items():
        if cfg.D * cfg.I * cfg.E > 1 << 27:
            cfg = get_config(name, E=4, K=min(cfg.K, 4))
        L = gen_layer(cfg, 0)
        assert L.router_W.shape == (cfg.E, cfg.D) and L.router_W.dtype == np.float32
        assert L.x.shape == (cfg.S, cfg.D)
        assert L.x.dtype == (np.uint16 if cfg.x_dtype == "bf16" else np.float32)
        ew = L.expert(0)
        fmt, gs = expert_format(cfg, 0)
        assert ew.gate.packed.shape == (cfg.I, cfg.D // 2)
        assert ew.down.packed.shape == (cfg.D, cfg.I // 2)
        ng = -(-cfg.I // gs) if (fmt == 4 and gs) else 1
        assert ew.down.scales.shape == (cfg.D * ng,)


def test_format_mixes():
    mix = CONFIGS["mix"]
    assert [expert_format(mix, e)[0] for e in range(4)] == [4, 2, 4, 2]
    sus = CONFIGS["sustained"]
    assert expert_format(sus, 31) == (4, 64) and expert_format(sus, 32) == (2, 0)
