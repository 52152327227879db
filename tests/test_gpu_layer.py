"""GPU layer parity through the C ABI: one-hot dequant probes (bit-exact),
small ragged layers checked element by element, the tiny workload, the
chunked driver and the decode entry points on small shapes, within
|gpu - oracle| <= 2e-2 * max|oracle| + 1e-3.  The full-size workloads are
checked on every token in test_gpu_workloads.py."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
import oracle
from gpu_cases import (DEV, announce, assert_close_layer, assert_routing_matches, oracle_layer,
                       require_gpu, run_layer, tol_ok, bf16_bits_to_f64)
from workload import (CONFIGS, QMat, LayerWeights, make_activations, make_weights, pack_nibbles,
                      small_config, f32_to_bf16_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------------------
# One-hot probes: bit-exact check of the dequantization inside both GEMMs
# ---------------------------------------------------------------------------

def _probe_weights(H, I, seed):
    """Gate = 256 everywhere (silu(256) = 256 exactly in fp32 and fp64); up random;
    down zero except one random entry per row (column c % I), bias = -8 * scale."""
    rng = np.random.default_rng(seed)
    gq = np.ones((1, I, H), np.uint8)
    g = QMat(pack_nibbles(gq), np.full((1, I, H // 64), 0x4380, np.uint16),   # s = 256
             np.zeros((1, I, H // 64), np.uint16))
    uq = rng.integers(0, 16, (1, I, H), dtype=np.uint8)
    us = f32_to_bf16_bits(rng.uniform(0.01, 0.5, (1, I, H // 64)).astype(np.float32))
    ub = f32_to_bf16_bits(rng.uniform(-2.0, 2.0, (1, I, H // 64)).astype(np.float32))
    u = QMat(pack_nibbles(uq), us, ub)
    dq = np.full((1, H, I), 8, np.uint8)
    q_nz = rng.integers(0, 16, H).astype(np.uint8)
    q_nz[q_nz == 8] = 3
    dq[0, np.arange(H), np.arange(H) % I] = q_nz
    ds = f32_to_bf16_bits(rng.uniform(0.001, 0.02, (1, H, I // 64)).astype(np.float32))
    s_val = (ds.astype(np.uint32) << 16).view(np.float32)
    db = f32_to_bf16_bits(np.float32(-8.0) * s_val)
    d = QMat(pack_nibbles(dq), ds, db)
    return LayerWeights(g, u, d, None, None, None)


@pytest.mark.parametrize("H,I,block_rows,prepack", [(256, 128, 32, False), (512, 256, 16, False),
                                                     (2048, 512, 64, False), (2048, 512, 32, False),
                                                     (2048, 512, 32, True), (512, 256, 16, True)])
def test_one_hot_probe_bit_exact(H, I, block_rows, prepack):
    """prepack: tile-packed codes with packed gate/up scale|bias words."""
    T = 96
    w = _probe_weights(H, I, seed=H + I)
    x = np.zeros((T, H), np.float32)
    cols = (np.arange(T) * 37 + 5) % H
    x[np.arange(T), cols] = 1.0
    x_bits = f32_to_bf16_bits(x)
    logits = np.zeros((T, 1), np.float32)
    cfg = small_config(T, H, I, 1, 1, 0)
    announce(f"one-hot probe H={H} I={I} br={block_rows} prepack={prepack}")
    layer = bq.MoeLayer(w, H, I, 0, 1, 1, DEV, block_rows=block_rows, prepack=prepack)
    got = run_layer(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits, block_rows)
    want = oracle.f32_to_bf16_rne_bits(ref["y"].astype(np.float32))
    assert np.count_nonzero(ref["y"]) > T * H // 2
    assert np.array_equal(got["y"], want)
    assert np.array_equal(got["expert_out"], want)   # k = 1, weight 1: rows are the tokens


# ---------------------------------------------------------------------------
# Small layers, every element
# ---------------------------------------------------------------------------

SMALL = [
    # T,   H,    I,   E,  k, I_sh, block_rows
    (64, 256, 128, 16, 2, 128, 32),       # the tiny workload's shape
    (200, 512, 256, 32, 4, 256, 32),      # several tiles per expert, ragged tails
    (37, 256, 128, 8, 3, 0, 16),          # ragged T, no shared expert
    (130, 384, 192, 12, 2, 320, 64),      # K not a multiple of 256; I_sh != I
    (70, 384, 128, 8, 2, 128, 32),        # down columns: a partial second group of 256
    (301, 256, 128, 4, 2, 128, 32),       # ~150 rows per expert: 64-row down items (block pairs)
    (3000, 256, 128, 64, 8, 128, 32),     # one call above 2048 tokens: batched routing reloads
    (200, 128, 64, 4, 4, 64, 32),         # paired down items with I = 64; k = 4 chunk routing
    (1, 2048, 512, 256, 8, 512, 32),      # batch-1 decode shape
    (9, 128, 64, 4, 4, 64, 16),           # k = E
    (50, 64, 64, 1000, 20, 64, 32),       # smallest H and I, largest E, k > 16 (radix top-k)
    # experts of 65-200 rows at H = 512 / 1024 (64-row paired down items)
    (301, 512, 128, 4, 2, 128, 32),       # ~150 rows per expert
    (200, 1024, 256, 4, 4, 256, 32),      # ~200 rows per expert, two down column groups
    (520, 512, 128, 8, 1, 0, 32),         # no shared expert, ~65 rows per expert
    (130, 512, 256, 2, 2, 128, 32),       # I_sh < I
    # large hidden sizes: gate/up scale tables of 36 and 81 KB of LDS per workgroup
    (96, 4096, 256, 8, 2, 256, 32),
    (96, 7168, 256, 8, 2, 256, 32),
    (70, 7168, 2048, 4, 2, 0, 32),        # down K = 2048: the K-chunked down kernel
]


@pytest.mark.parametrize("T,H,I,E,k,I_sh,br", SMALL)
def test_small_layer_parity(T, H, I, E, k, I_sh, br):
    cfg = small_config(T, H, I, E, k, I_sh, seed=T + E)
    w = make_weights(cfg, seed=T * 7 + 1, cache=False)
    x_bits, logits = make_activations(cfg)
    announce(f"small layer T={T} H={H} I={I} E={E} k={k} I_sh={I_sh} br={br}")
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=br)
    got = run_layer(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits, br)
    assert_routing_matches(got["routing"], logits, k, br)
    ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
    assert ok, f"expert_out {ratio:.3f}"
    if I_sh:
        ok, ratio = tol_ok(bf16_bits_to_f64(got["shared_out"]), ref["shared_out"])
        assert ok, f"shared_out {ratio:.3f}"
    assert_close_layer(got["y"], ref["y"])


# Packed layers (tile-packed codes, packed gate/up scale|bias words) whose experts
# average at least 48 rows: several full row blocks per expert and ragged last blocks,
# the down GEMM on 64-row paired items, the shared expert over every token.
LARGE_GROUPS = [
    (301, 256, 128, 4, 2, 128, 32),       # ~150 rows per expert, T not a multiple of 64
    (200, 128, 64, 4, 4, 64, 32),         # H = 128: one K-chunk
    (301, 512, 128, 4, 2, 128, 32),
    (200, 1024, 256, 4, 4, 256, 32),      # two gate/up column tiles
    (520, 512, 128, 8, 1, 0, 32),         # no shared expert, ~65 rows per expert
    (130, 512, 256, 2, 2, 128, 32),       # I_sh < I
    (3000, 256, 128, 64, 8, 128, 32),     # above 2048 tokens
    (97, 2048, 512, 2, 1, 512, 32),       # the layer's H and I; 97 shared rows: a ragged slot
]


@pytest.mark.parametrize("T,H,I,E,k,I_sh,br", LARGE_GROUPS)
def test_large_groups_parity_packed(T, H, I, E, k, I_sh, br):
    assert T * k >= 48 * E
    cfg = small_config(T, H, I, E, k, I_sh, seed=T + E + 5)
    w = make_weights(cfg, seed=T * 7 + 3, cache=False)
    x_bits, logits = make_activations(cfg)
    announce(f"large groups, packed T={T} H={H} I={I} E={E} k={k} I_sh={I_sh}")
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=br, prepack=True)
    got = run_layer(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits, br)
    assert_routing_matches(got["routing"], logits, k, br)
    ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
    assert ok, f"expert_out {ratio:.3f}"
    if I_sh:
        ok, ratio = tol_ok(bf16_bits_to_f64(got["shared_out"]), ref["shared_out"])
        assert ok, f"shared_out {ratio:.3f}"
    assert_close_layer(got["y"], ref["y"])


def test_one_expert_takes_every_token_packed():
    """Packed layer, E = 8: expert 3 gets all 330 rows (ten full 32-row blocks and a
    ragged eleventh; in the down GEMM five 64-row items and a 10-row leader), experts
    5..7 stay empty."""
    T, H, I, E, k, I_sh = 330, 512, 128, 8, 2, 128
    cfg = small_config(T, H, I, E, k, I_sh, seed=81)
    w = make_weights(cfg, seed=82, cache=False)
    x_bits, logits = make_activations(cfg)
    logits = logits.copy()
    logits[:, 3] += np.float32(50.0)
    logits[:, 5:] -= np.float32(50.0)
    announce("one expert takes every token, packed")
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, prepack=True)
    got = run_layer(layer, x_bits, logits)
    assert int(got["routing"]["counts"][3]) == T
    assert np.all(got["routing"]["counts"][5:] == 0)
    ref = oracle_layer(w, cfg, x_bits, logits)
    assert_routing_matches(got["routing"], logits, k)
    ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
    assert ok, f"expert_out {ratio:.3f}"
    ok, ratio = tol_ok(bf16_bits_to_f64(got["shared_out"]), ref["shared_out"])
    assert ok, f"shared_out {ratio:.3f}"
    assert_close_layer(got["y"], ref["y"])


def test_one_expert_takes_every_token():
    """Expert 3's logit is raised for every token: it gets all T rows (10 full
    32-row blocks and a ragged 11th), the second choices spread over the rest,
    and several experts stay empty."""
    T, H, I, E, k, I_sh = 330, 256, 128, 16, 2, 128
    cfg = small_config(T, H, I, E, k, I_sh, seed=77)
    w = make_weights(cfg, seed=78, cache=False)
    x_bits, logits = make_activations(cfg)
    logits = logits.copy()
    logits[:, 3] += np.float32(50.0)
    logits[:, 8:] -= np.float32(50.0)      # experts 8..15 never chosen
    announce("one expert takes every token")
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV)
    got = run_layer(layer, x_bits, logits)
    assert int(got["routing"]["counts"][3]) == T
    assert np.all(got["routing"]["counts"][8:] == 0)
    ref = oracle_layer(w, cfg, x_bits, logits)
    assert_routing_matches(got["routing"], logits, k)
    assert_close_layer(got["y"], ref["y"])


def test_one_expert_takes_every_token_h512():
    """A skewed layer at H = 512: expert 3 gets every token (330 rows: ten full 32-row
    blocks and a ragged eleventh), the second choices spread thinly, several experts stay
    empty."""
    T, H, I, E, k, I_sh = 330, 512, 128, 16, 2, 128
    cfg = small_config(T, H, I, E, k, I_sh, seed=79)
    w = make_weights(cfg, seed=80, cache=False)
    x_bits, logits = make_activations(cfg)
    logits = logits.copy()
    logits[:, 3] += np.float32(50.0)
    logits[:, 8:] -= np.float32(50.0)
    announce("one expert takes every token, H = 512")
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV)
    got = run_layer(layer, x_bits, logits)
    assert int(got["routing"]["counts"][3]) == T
    ref = oracle_layer(w, cfg, x_bits, logits)
    assert_routing_matches(got["routing"], logits, k)
    ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
    assert ok, f"expert_out {ratio:.3f}"
    assert_close_layer(got["y"], ref["y"])


def test_tiny_workload_full():
    cfg = CONFIGS["tiny"]
    w = make_weights(cfg, seed=0)
    x_bits, logits = make_activations(cfg)
    announce("tiny workload")
    layer = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    got = run_layer(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits)
    assert_routing_matches(got["routing"], logits, cfg.k)
    assert_close_layer(got["y"], ref["y"])


def test_chunked_driver_matches_unchunked_small():
    cfg = small_config(100, 256, 128, 16, 2, 128, seed=21)
    w = make_weights(cfg, seed=5, cache=False)
    x_bits, logits = make_activations(cfg)
    layer = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    x = bq.bf16_from_bits(x_bits, DEV)
    lg = torch.from_numpy(logits).to(DEV)
    announce("chunked driver T=100 chunk=32")
    y = torch.empty((100, cfg.H), dtype=torch.bfloat16, device=DEV)
    layer.forward_chunked(x, lg, 32, y)
    torch.cuda.synchronize()
    ref, _ = oracle.moe_layer_chunked(x_bits, logits, w.gate, w.up, w.down, 2, w.sh_gate, w.sh_up,
                                      w.sh_down, chunk=32)
    assert_close_layer(bq.bf16_to_bits(y), ref)
    # per-chunk calls through the three entry points give the same bits
    parts = []
    for t0 in range(0, 100, 32):
        parts.append(run_layer(layer, x_bits[t0:t0 + 32], logits[t0:t0 + 32])["y"])
    assert np.array_equal(np.concatenate(parts), bq.bf16_to_bits(y))


def test_split_phases_equal_grouped_gemm():
    cfg = small_config(150, 512, 256, 32, 4, 256, seed=31)
    w = make_weights(cfg, seed=9, cache=False)
    x_bits, logits = make_activations(cfg)
    layer = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    announce("split gateup/down vs grouped gemm")
    got = run_layer(layer, x_bits, logits)
    b = layer.buffers(cfg.T)
    eo = torch.empty_like(b["expert_out"])
    so = torch.empty_like(b["shared_out"])
    x = bq.bf16_from_bits(x_bits, DEV)
    bq.moe_expert_gateup_q4(x, cfg.I, cfg.I_sh, cfg.E, cfg.k, 32, b["routing"], layer.gate, layer.up,
                            layer.sh_gate, layer.sh_up, b["gemm_ws"])
    bq.moe_expert_down_q4(cfg.T, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, 32, b["routing"], layer.down,
                          layer.sh_down, eo, so, b["gemm_ws"])
    torch.cuda.synchronize()
    assert np.array_equal(bq.bf16_to_bits(eo), got["expert_out"])
    assert np.array_equal(bq.bf16_to_bits(so), got["shared_out"])


# ---------------------------------------------------------------------------
# Fused single-launch decode (one token per call)
# ---------------------------------------------------------------------------

def _decode_one(layer, x_bits_row, logits_row, ws=None, with_routing=True):
    x = bq.bf16_from_bits(x_bits_row, DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits_row)).to(DEV)
    r = bq.DeviceRouting(1, layer.E, layer.k, layer.block_rows, DEV) if with_routing else None
    y = torch.empty((1, layer.H), dtype=torch.bfloat16, device=DEV)
    ws = layer.decode(x, lg, y, routing=r, ws=ws)
    torch.cuda.synchronize()
    return bq.bf16_to_bits(y), (r.to_host() if r is not None else None), ws


@pytest.fixture(scope="module")
def big_layer():
    cfg = CONFIGS["prefill512"]
    w = make_weights(cfg, seed=0)
    return w, bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)


def test_fused_decode_sequential_equals_single(big_layer):
    w, layer = big_layer
    cfg = CONFIGS["decode"]
    x_bits, logits = make_activations(cfg)
    n = 40
    x = bq.bf16_from_bits(x_bits[:n], DEV)
    lg = torch.from_numpy(logits[:n]).to(DEV)
    y = torch.empty((n, cfg.H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(bq.decode_workspace_bytes(cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k),
                     dtype=torch.uint8, device=DEV)
    announce("fused decode sequential x40")
    bq.moe_decode_q4_sequential(x, lg, cfg.I, cfg.I_sh, cfg.k, *layer.weight_mats(), y, ws)
    torch.cuda.synchronize()
    ys = bq.bf16_to_bits(y)
    for t in (0, 17, 39):
        y1, _, _ = _decode_one(layer, x_bits[t:t + 1], logits[t:t + 1], with_routing=False)
        assert np.array_equal(ys[t:t + 1], y1)     # same kernel, deterministic


@pytest.mark.parametrize("H,I,E,k,I_sh", [
    (256, 128, 16, 2, 128),      # the tiny layer's shape
    (512, 256, 100, 7, 0),       # no shared expert, E not a multiple of 64
    (384, 192, 8, 1, 320),       # I_sh != I, k = 1
    (256, 1024, 64, 16, 768),    # k + 1 > 12 experts per down workgroup, K of down > 512
    (4096, 64, 8, 2, 64),        # H > 2048: several K passes per gate/up row
    (128, 128, 256, 64, 128),    # the largest k
    (64, 64, 1000, 20, 64),      # the largest E (16 logits per lane), k > 16, smallest H and I
    (7168, 256, 8, 2, 256),      # large H
    (7168, 2048, 4, 2, 0),       # large H and I, no shared expert
])
def test_fused_decode_small_shapes(H, I, E, k, I_sh):
    cfg = small_config(6, H, I, E, k, I_sh, seed=E + k)
    w = make_weights(cfg, seed=E * 3 + k, cache=False)
    x_bits, logits = make_activations(cfg)
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV)
    for t in range(cfg.T):
        announce(f"fused decode small H={H} I={I} E={E} k={k} I_sh={I_sh} t={t}")
        y, r, _ = _decode_one(layer, x_bits[t:t + 1], logits[t:t + 1])
        ref = oracle_layer(w, cfg, x_bits[t:t + 1], logits[t:t + 1])
        assert_routing_matches(r, logits[t:t + 1], k)
        assert_close_layer(y, ref["y"])


# ---------------------------------------------------------------------------
# Property-based layer cases (hypothesis, derandomized: every run draws the same
# examples): random shapes within the ABI's rules, both code layouts, every block
# height; routing bit-exact and every output element within the tolerance.
# ---------------------------------------------------------------------------
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402


@settings(max_examples=24, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(T=st.integers(1, 260), h64=st.integers(1, 16), i64=st.integers(1, 8),
       E=st.integers(1, 48), kq=st.floats(0.0, 1.0), sh64=st.integers(0, 6),
       br=st.sampled_from([16, 32, 64]), tiles=st.booleans(), seed=st.integers(0, 2 ** 20))
def test_layer_property_random_shapes(T, h64, i64, E, kq, sh64, br, tiles, seed):
    H, I, I_sh = 64 * h64, 64 * i64, 64 * sh64
    k = 1 + int(kq * (min(E, 10) - 1))
    cfg = small_config(T, H, I, E, k, I_sh, seed=seed)
    w = make_weights(cfg, seed=seed + 1, cache=False)
    x_bits, logits = make_activations(cfg)
    announce(f"layer property T={T} H={H} I={I} E={E} k={k} I_sh={I_sh} br={br} "
             f"tiles={tiles} seed={seed}")
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=br, prepack=tiles)
    got = run_layer(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits, br)
    assert_routing_matches(got["routing"], logits, k, br)
    ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
    assert ok, f"expert_out {ratio:.3f}"
    if I_sh:
        ok, ratio = tol_ok(bf16_bits_to_f64(got["shared_out"]), ref["shared_out"])
        assert ok, f"shared_out {ratio:.3f}"
    assert_close_layer(got["y"], ref["y"])
