"""The unfused baseline (weights expanded to bf16 in memory, then the grouped
GEMM over bf16 weights) against the oracle: the expansion bit-exact, one-hot
probes through the bf16 GEMM bit-exact, whole layers within the tolerance."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
import oracle
from gpu_cases import (DEV, announce, assert_close_layer, assert_routing_matches, layer_to_host,
                       oracle_layer, require_gpu, run_layer)
from test_gpu_layer import _probe_weights
from workload import make_activations, make_weights, small_config, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run_unfused(layer, x_bits, logits):
    x = bq.bf16_from_bits(x_bits, DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    bufs = layer.forward_unfused(x, lg)
    torch.cuda.synchronize()
    return layer_to_host(bufs)


def test_dequant_expansion_bit_exact_and_skips_unrouted():
    cfg = small_config(64, 256, 128, 16, 2, 128, seed=3)
    w = make_weights(cfg, seed=11, cache=False)
    m = bq.DeviceQMat.from_host(w.gate, DEV)
    out = torch.full((16, 128, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    counts = torch.tensor([0, 3, 1, 0] * 4, dtype=torch.int32, device=DEV)
    announce("dequant expansion E=16 N=128 K=256")
    bq.moe_dequant_q4_bf16(m, 16, 128, 256, out, counts)
    torch.cuda.synchronize()
    got = bq.bf16_to_bits(out)
    want = oracle.dequant_bf16_bits(w.gate.codes, w.gate.scales, w.gate.biases)
    on = counts.cpu().numpy() > 0
    assert np.array_equal(got[on], want[on])
    assert np.all(got[~on] == 0x40E0)                 # bf16 7.0: rows left as they were
    bq.moe_dequant_q4_bf16(m, 16, 128, 256, out)      # counts NULL: every expert
    torch.cuda.synchronize()
    assert np.array_equal(bq.bf16_to_bits(out), want)


@pytest.mark.parametrize("H,I,block_rows", [(256, 128, 32), (2048, 512, 64)])
def test_unfused_one_hot_probe_bit_exact(H, I, block_rows):
    T = 96
    w = _probe_weights(H, I, seed=H + I)
    x = np.zeros((T, H), np.float32)
    x[np.arange(T), (np.arange(T) * 37 + 5) % H] = 1.0
    x_bits = f32_to_bf16_bits(x)
    logits = np.zeros((T, 1), np.float32)
    cfg = small_config(T, H, I, 1, 1, 0)
    announce(f"unfused one-hot probe H={H} I={I} br={block_rows}")
    layer = bq.MoeLayer(w, H, I, 0, 1, 1, DEV, block_rows=block_rows)
    got = _run_unfused(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits, block_rows)
    want = oracle.f32_to_bf16_rne_bits(ref["y"].astype(np.float32))
    assert np.array_equal(got["y"], want)


@pytest.mark.parametrize("T,H,I,E,k,I_sh,block_rows", [
    (64, 256, 128, 16, 2, 128, 32),       # the tiny workload's shape
    (200, 512, 256, 32, 4, 256, 32),      # several tiles per expert, ragged tails
    (37, 256, 128, 8, 3, 0, 16),          # ragged T, no shared expert
    (130, 384, 192, 12, 2, 320, 64),      # I_sh != I
])
def test_unfused_layer_matches_oracle_and_fused(T, H, I, E, k, I_sh, block_rows):
    cfg = small_config(T, H, I, E, k, I_sh, seed=T + E)
    w = make_weights(cfg, seed=T * 7 + H, cache=False)
    x_bits, logits = make_activations(cfg)
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=block_rows)
    announce(f"unfused layer T={T} H={H} I={I} E={E} k={k} I_sh={I_sh} br={block_rows}")
    got = _run_unfused(layer, x_bits, logits)
    ref = oracle_layer(w, cfg, x_bits, logits, block_rows)
    assert_routing_matches(got["routing"], logits, k, block_rows)
    assert_close_layer(got["y"], ref["y"])
    fused = run_layer(layer, x_bits, logits)
    # same bf16 weights; the K-chunking (and so the fp32 summation order) differs
    assert_close_layer(got["y"], oracle.bf16_bits_to_f64(fused["y"]), what="unfused vs fused y")
