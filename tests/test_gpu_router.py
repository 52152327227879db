"""Router projection and the gated combine on the GPU against the oracle.

The logits are fp32 sums of H exact bf16 x bf16 products, so each may differ
from the fp64 oracle by at most about H * 2^-24 * sum_h |x_h w_h|; the test
takes that bound per element.  Selection is a decision taken on fp32 values,
so the routing is checked bit for bit by running the oracle's top-k on the
GPU's own logits.  Whole layers (router -> route -> GEMMs -> gated combine)
are checked within the layer tolerance."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
import oracle
from gpu_cases import (DEV, announce, assert_close_layer, assert_routing_matches, gpu_route,
                       oracle_layer, require_gpu)
from workload import CONFIGS, make_activations, make_router, make_weights, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _router_gpu(x_bits, wr_bits, wg_bits=None):
    T, H = x_bits.shape
    E = wr_bits.shape[0]
    x = bq.bf16_from_bits(x_bits, DEV)
    wr = bq.bf16_from_bits(wr_bits, DEV)
    wg = None if wg_bits is None else bq.bf16_from_bits(wg_bits, DEV)
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    g = None if wg_bits is None else torch.full((T,), float("nan"), dtype=torch.float32, device=DEV)
    bq.moe_router(x, wr, lg, wg, g)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), (None if g is None else g.cpu().numpy())


def _check_logits(got, x_bits, wr_bits):
    want = oracle.router_logits(x_bits, wr_bits)
    H = x_bits.shape[1]
    abs_sum = np.abs(oracle.bf16_bits_to_f64(x_bits)) @ np.abs(oracle.bf16_bits_to_f64(wr_bits)).T
    bound = 2.0 * H * 2.0 ** -24 * abs_sum + 1e-30
    assert np.all(np.isfinite(got))
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= bound), f"max err / bound = {np.max(err / bound):.3f}"
    return want


@pytest.mark.parametrize("T,H,E,gated", [
    (512, 2048, 256, True),     # the prefill layer
    (1, 2048, 256, True),       # batch-1 decode
    (37, 384, 100, False),      # ragged T, E not a multiple of 16
    (16, 64, 1000, True),       # smallest H, largest E
    (1000, 256, 100, False),    # 32 x 32 tiles: ragged T and E
    (384, 128, 31, True),       # first size on 32 x 32 tiles; E + gate = one row tile
])
def test_router_logits_and_gate(T, H, E, gated):
    cfg = small_config(T, H, 64, E, 1, 0, seed=T + E)
    x_bits, _ = make_activations(cfg)
    wr_bits, wg_bits = make_router(cfg, seed=E)
    announce(f"router T={T} H={H} E={E} gated={gated}")
    got, g = _router_gpu(x_bits, wr_bits, wg_bits if gated else None)
    want = _check_logits(got, x_bits, wr_bits)
    if gated:
        g_want = oracle.shared_gate(x_bits, wg_bits)
        # logit error bound (as above) through sigmoid' <= 1/4, plus fp32 exp/divide rounding
        xw = np.abs(oracle.bf16_bits_to_f64(x_bits)) @ np.abs(oracle.bf16_bits_to_f64(wg_bits))
        bound = 0.25 * 2.0 * H * 2.0 ** -24 * xw + 1e-6
        assert np.all(np.abs(g - g_want) <= bound)
    assert want.shape == got.shape


def test_routing_on_router_logits_is_exact():
    cfg = CONFIGS["prefill512"]
    x_bits, _ = make_activations(cfg)
    wr_bits, _ = make_router(cfg)
    announce("route on GPU router logits (512 tokens)")
    logits, _ = _router_gpu(x_bits, wr_bits)
    got = gpu_route(logits, cfg.k)
    assert_routing_matches(got, logits, cfg.k)     # the oracle selects on the same fp32 values


@pytest.mark.parametrize("T,H,I,E,k,I_sh", [
    (64, 256, 128, 16, 2, 128),
    (200, 512, 256, 32, 4, 256),
])
def test_layer_with_router_and_gated_shared_expert(T, H, I, E, k, I_sh):
    cfg = small_config(T, H, I, E, k, I_sh, seed=3 * T)
    w = make_weights(cfg, seed=T + H, cache=False)
    x_bits, _ = make_activations(cfg)
    wr_bits, wg_bits = make_router(cfg, seed=T)
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV)
    x = bq.bf16_from_bits(x_bits, DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    g = torch.empty(T, dtype=torch.float32, device=DEV)
    announce(f"router + gated layer T={T} H={H} I={I} E={E} k={k}")
    bq.moe_router(x, bq.bf16_from_bits(wr_bits, DEV), lg, bq.bf16_from_bits(wg_bits, DEV), g)
    b = layer.forward(x, lg)                       # route, GEMMs, ungated combine
    y_gated = torch.empty_like(b["y"])
    bq.moe_combine_gated(b["expert_out"], b["shared_out"], g, b["routing"], k, y_gated)
    torch.cuda.synchronize()
    logits = lg.cpu().numpy()
    ref = oracle_layer(w, cfg, x_bits, logits)
    ref_g = oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, k, w.sh_gate, w.sh_up,
                             w.sh_down, shared_w=oracle.shared_gate(x_bits, wg_bits))
    assert_routing_matches(b["routing"].to_host(), logits, k)
    assert_close_layer(bq.bf16_to_bits(b["y"]), ref["y"])
    assert_close_layer(bq.bf16_to_bits(y_gated), ref_g["y"], what="gated y")
