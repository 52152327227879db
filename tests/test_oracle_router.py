"""Pins of the oracle's router projection and optional shared-expert gate,
each fixed by something other than the oracle's own formula: exact rational
brute force on dyadic inputs, one-hot activations reading a weight column, a
closed form of the logistic function, and special cases of the layer."""
from fractions import Fraction
import math

import numpy as np

import oracle
from workload import f32_to_bf16_bits, make_weights, small_config, make_activations


def _dyadic(rng, shape, num, den):
    # small integers / power of two: exact in bf16, products and sums exact in fp64
    return (rng.integers(-num, num + 1, shape) / den).astype(np.float32)


def _exact_dot(a_row, b_row):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(a_row, b_row))


def test_router_logits_equal_exact_rational_dot_products():
    rng = np.random.default_rng(5)
    x = _dyadic(rng, (3, 64), 7, 8)
    wr = _dyadic(rng, (5, 64), 15, 32)
    got = oracle.router_logits(f32_to_bf16_bits(x), f32_to_bf16_bits(wr))
    assert got.shape == (3, 5)                      # [T, E]: W_r is [E, H], not [H, E]
    for t in range(3):
        for e in range(5):
            assert Fraction(got[t, e]) == _exact_dot(x[t], wr[e])


def test_router_one_hot_activation_reads_a_weight_column():
    rng = np.random.default_rng(6)
    H, E = 128, 9
    wr_bits = f32_to_bf16_bits(rng.standard_normal((E, H)).astype(np.float32))
    cols = [0, 17, 127]
    x = np.zeros((3, H), np.float32)
    x[np.arange(3), cols] = 1.0
    got = oracle.router_logits(f32_to_bf16_bits(x), wr_bits)
    w = oracle.bf16_bits_to_f64(wr_bits)
    for t, c in enumerate(cols):
        assert np.array_equal(got[t], w[:, c])


def test_shared_gate_closed_forms():
    rng = np.random.default_rng(7)
    H = 64
    wg = _dyadic(rng, H, 15, 64)
    x = _dyadic(rng, (4, H), 7, 8)
    x[0] = 0.0
    g = oracle.shared_gate(f32_to_bf16_bits(x), f32_to_bf16_bits(wg))
    g_neg = oracle.shared_gate(f32_to_bf16_bits(-x), f32_to_bf16_bits(wg))
    assert g[0] == 0.5                               # sigmoid(0)
    assert np.allclose(g + g_neg, 1.0, rtol=0, atol=1e-15)
    for t in range(1, 4):
        z = float(_exact_dot(x[t], wg))
        assert math.isclose(g[t], 0.5 * (1.0 + math.tanh(z / 2.0)), rel_tol=1e-14)
        assert (g[t] > 0.5) == (z > 0)


def test_layer_shared_weight_special_cases():
    cfg = small_config(12, 128, 64, 6, 2, 64, seed=2)
    w = make_weights(cfg, seed=4, cache=False)
    x_bits, logits = make_activations(cfg)
    base = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, cfg.k, w.sh_gate, w.sh_up,
                            w.sh_down)
    ones = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, cfg.k, w.sh_gate, w.sh_up,
                            w.sh_down, shared_w=np.ones(12))
    zero = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, cfg.k, w.sh_gate, w.sh_up,
                            w.sh_down, shared_w=np.zeros(12))
    routed_only = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, cfg.k)
    assert np.array_equal(ones["y"], base["y"])
    assert np.array_equal(zero["y"], routed_only["y"])
    half = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, cfg.k, w.sh_gate, w.sh_up,
                            w.sh_down, shared_w=np.full(12, 0.5))
    assert np.allclose(half["y"], routed_only["y"] + 0.5 * base["shared_out"], rtol=0, atol=1e-12)
