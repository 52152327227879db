"""Pins of the oracle's expert FFN, shared expert and combine (runs on CPU).

P-ffn1: brute-force dense computation (every expert on every token, a dense
[T, E] gate matrix that is zero off the top-k) equals the grouped oracle.
P-ffn2: one expert, k = 1, no shared expert, with exactly representable
(dyadic) weights: the SwiGLU identities
    y(x) + y(-x) = (G * U) Wd^T          (silu(z) - silu(-z) = z)
    y(x) - y(-x) = (G tanh(G/2) * U) Wd^T (silu(z) + silu(-z) = z tanh(z/2))
with G = x Wg^T, U = x Wu^T built independently of the oracle's dequant,
plus a non-square shape that rejects a transposed operand.
"""
import numpy as np
import pytest

import oracle
from workload import QMat, pack_nibbles, f32_to_bf16_bits, small_config, make_weights, make_activations


def _dyadic_qmat(rng, N, K, s_exp_base):
    """Codes, power-of-two scales per (row, group) and bias -8*s: W = (q - 8) * s exactly."""
    q = rng.integers(0, 16, (1, N, K), dtype=np.uint8)
    exps = s_exp_base + rng.integers(0, 3, (1, N, K // 64))
    s_bits = ((127 + exps) << 7).astype(np.uint16)
    b_bits = (s_bits | 0x8000) + (3 << 7)
    W = (q[0].astype(np.float64) - 8.0) * np.repeat(2.0 ** exps[0].astype(np.float64), 64, axis=1)
    return QMat(pack_nibbles(q), s_bits, b_bits), W


def _one_expert_case(seed, H=128, I=64):
    rng = np.random.default_rng(seed)
    g, Wg = _dyadic_qmat(rng, I, H, -7)
    u, Wu = _dyadic_qmat(rng, I, H, -7)
    d, Wd = _dyadic_qmat(rng, H, I, -7)
    T = 9
    xv = rng.integers(-2, 3, (T, H)).astype(np.float32)
    return (g, u, d), (Wg, Wu, Wd), xv


def _y(x_f32, mats, k=1):
    T = x_f32.shape[0]
    logits = np.zeros((T, 1), np.float32)
    r = oracle.moe_layer(f32_to_bf16_bits(x_f32), logits, *mats, k)
    return r["y"]


def test_swiglu_identities_one_expert():
    mats, (Wg, Wu, Wd), xv = _one_expert_case(3)
    yp = _y(xv, mats)
    ym = _y(-xv, mats)
    G = xv.astype(np.float64) @ Wg.T
    U = xv.astype(np.float64) @ Wu.T
    assert np.max(np.abs(G)) > 0.5   # identities are exercised away from zero
    ref_sum = (G * U) @ Wd.T
    ref_diff = (G * np.tanh(G / 2.0) * U) @ Wd.T
    scale = max(1.0, np.max(np.abs(ref_sum)))
    assert np.max(np.abs((yp + ym) - ref_sum)) < 1e-12 * scale
    assert np.max(np.abs((yp - ym) - ref_diff)) < 1e-12 * scale


def test_one_hot_input_reads_weight_column():
    # x = e_i: G[n] = Wg[n, i], U[n] = Wu[n, i]; output is the SwiGLU of two columns.
    mats, (Wg, Wu, Wd), _ = _one_expert_case(4)
    H = Wg.shape[1]
    for i in (0, 63, 64, 127):
        x = np.zeros((1, H), np.float32)
        x[0, i] = 1.0
        y = _y(x, mats)
        y_neg = _y(-x, mats)
        ref_sum = (Wg[:, i] * Wu[:, i]) @ Wd.T
        assert np.max(np.abs((y + y_neg)[0] - ref_sum)) < 1e-12 * max(1.0, np.max(np.abs(ref_sum)))


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs((s[1] - s[2]) - 1.0) < 1e-15          # silu(z) - silu(-z) = z
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-12


def test_transposed_operand_rejected():
    mats, _, xv = _one_expert_case(5, H=128, I=64)
    g, u, d = mats
    with pytest.raises(ValueError):
        # swapping gate and down (shapes [64,128] vs [128,64]) must not silently work
        _y(xv, (d, u, g))


def _dense_masked(x_bits, logits, w, k):
    """Every expert on every token; gate matrix zero off the top-k."""
    x = oracle.bf16_bits_to_f64(x_bits)
    T, E = logits.shape
    idx, wts = oracle.route_topk(logits, k)
    gm = np.zeros((T, E))
    gm[np.arange(T)[:, None], idx] = wts
    y = np.zeros_like(x)
    for e in range(E):
        Wg = oracle.dequant(w.gate.codes[e], w.gate.scales[e], w.gate.biases[e])
        Wu = oracle.dequant(w.up.codes[e], w.up.scales[e], w.up.biases[e])
        Wd = oracle.dequant(w.down.codes[e], w.down.scales[e], w.down.biases[e])
        y += gm[:, e:e + 1] * oracle.swiglu_ffn(x, Wg, Wu, Wd)
    if w.sh_gate is not None:
        Wg = oracle.dequant(w.sh_gate.codes[0], w.sh_gate.scales[0], w.sh_gate.biases[0])
        Wu = oracle.dequant(w.sh_up.codes[0], w.sh_up.scales[0], w.sh_up.biases[0])
        Wd = oracle.dequant(w.sh_down.codes[0], w.sh_down.scales[0], w.sh_down.biases[0])
        y += oracle.swiglu_ffn(x, Wg, Wu, Wd)
    return y


@pytest.mark.parametrize("shape", [
    (64, 256, 128, 16, 2, 128),     # the tiny workload's shape
    (37, 128, 64, 8, 3, 0),         # ragged T, no shared expert
    (5, 128, 64, 4, 4, 64),         # k = E
])
def test_dense_masked_equals_grouped(shape):
    T, H, I, E, k, I_sh = shape
    cfg = small_config(T, H, I, E, k, I_sh, seed=11)
    w = make_weights(cfg, seed=2, cache=False)
    x_bits, logits = make_activations(cfg)
    r = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, k, w.sh_gate, w.sh_up, w.sh_down)
    yd = _dense_masked(x_bits, logits, w, k)
    assert np.max(np.abs(r["y"] - yd)) <= 1e-12 * np.max(np.abs(yd))


def test_shared_expert_adds_with_weight_one():
    cfg = small_config(16, 128, 64, 4, 2, 64, seed=12)
    w = make_weights(cfg, seed=3, cache=False)
    x_bits, logits = make_activations(cfg)
    with_sh = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, 2, w.sh_gate, w.sh_up, w.sh_down)
    no_sh = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, 2)
    assert np.array_equal(with_sh["y"] - no_sh["y"], with_sh["shared_out"]) or \
        np.max(np.abs(with_sh["y"] - no_sh["y"] - with_sh["shared_out"])) < 1e-12


def test_chunks_are_independent_calls():
    cfg = small_config(48, 128, 64, 8, 2, 64, seed=13)
    w = make_weights(cfg, seed=4, cache=False)
    x_bits, logits = make_activations(cfg)
    args = (w.gate, w.up, w.down, 2, w.sh_gate, w.sh_up, w.sh_down)
    y_full = oracle.moe_layer(x_bits, logits, *args)["y"]
    y_ch, parts = oracle.moe_layer_chunked(x_bits, logits, *args, chunk=16)
    assert len(parts) == 3
    # token-wise independence: identical up to fp summation order
    assert np.max(np.abs(y_full - y_ch)) < 1e-12 * np.max(np.abs(y_full))
    y_one, parts1 = oracle.moe_layer_chunked(x_bits, logits, *args, chunk=48)
    assert len(parts1) == 1 and np.array_equal(y_one, y_full)
