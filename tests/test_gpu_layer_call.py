"""moe_layer_q4 (route, grouped GEMM and combine in one call) against the same
three steps called one after another on one stream.  Both run the same kernels
on the same inputs, so every output must be bit-identical.  The layer itself is
checked against the oracle by the parity tests, which call moe_layer_q4."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
from gpu_cases import DEV, announce, layer_to_host, oracle_layer, assert_close_layer, require_gpu
from workload import make_activations, make_weights, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _layer(T, H, I, E, k, I_sh, seed, br=32):
    cfg = small_config(T, H, I, E, k, I_sh, seed=seed)
    w = make_weights(cfg, seed=seed + 1, cache=False)
    x_bits, logits = make_activations(cfg)
    layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=br, prepack=True)
    x = bq.bf16_from_bits(x_bits, DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    return cfg, w, layer, x, lg, x_bits, logits


def _both(layer, x, lg, stream=None):
    a = layer_to_host(layer.forward(x, lg, stream=stream))
    b = layer_to_host(layer.forward_three_calls(x, lg, stream=stream))
    return a, b


def _assert_same(a, b):
    assert a.keys() == b.keys()
    for key in a:
        va, vb = a[key], b[key]
        if isinstance(va, dict):
            _assert_same(va, vb)
        elif va is not None:
            assert np.array_equal(np.asarray(va), np.asarray(vb)), key


@pytest.mark.parametrize("T,H,I,E,k,I_sh,br", [
    (512, 512, 256, 64, 8, 256, 32),    # the prefill shape, scaled down
    (40, 256, 128, 16, 2, 128, 32),     # T <= 64: the one-launch routing path
    (300, 256, 128, 32, 4, 0, 16),      # no shared expert
    (700, 384, 192, 48, 6, 320, 64),    # I_sh != I, 64-row blocks
])
def test_layer_call_equals_three_calls(T, H, I, E, k, I_sh, br):
    cfg, w, layer, x, lg, x_bits, logits = _layer(T, H, I, E, k, I_sh, seed=T + E, br=br)
    announce(f"moe_layer_q4 vs three calls T={T} H={H} I={I} E={E} k={k} I_sh={I_sh} br={br}")
    a, b = _both(layer, x, lg)
    torch.cuda.synchronize()
    _assert_same(a, b)
    s = np.arange(0, T, max(1, T // 16))
    ref = oracle_layer(w, cfg, x_bits[s], logits[s], block_rows=br)
    assert_close_layer(a["y"][s], ref["y"])


def test_back_to_back_calls_on_a_side_stream():
    """Several calls in a row on a non-default stream, alternating two inputs:
    each call's y equals its own three-call result."""
    cfg, w, layer, x, lg, x_bits, logits = _layer(256, 256, 128, 32, 4, 128, seed=5)
    x2 = torch.flip(x, dims=[0]).contiguous()
    lg2 = torch.flip(lg, dims=[0]).contiguous()
    want1 = layer_to_host(layer.forward_three_calls(x, lg))["y"]
    want2 = layer_to_host(layer.forward_three_calls(x2, lg2))["y"]
    s = torch.cuda.Stream()
    ys = [torch.empty_like(x) for _ in range(6)]
    announce("moe_layer_q4 x6 back to back on a side torch stream")
    with torch.cuda.stream(s):
        for i, y in enumerate(ys):
            if i % 2 == 0:
                layer.forward(x, lg, out=y, stream=s)
            else:
                layer.forward(x2, lg2, out=y, stream=s)
    torch.cuda.synchronize()
    for i, y in enumerate(ys):
        assert np.array_equal(bq.bf16_to_bits(y), want1 if i % 2 == 0 else want2), i


def test_layer_call_under_graph_capture():
    """Replays of a captured layer call, with eager work in between, reproduce
    the eager result (the path records no memset node)."""
    cfg, w, layer, x, lg, x_bits, logits = _layer(200, 256, 128, 32, 4, 128, seed=9)
    want = layer_to_host(layer.forward_three_calls(x, lg))["y"]
    y = torch.empty_like(x)
    s = torch.cuda.Stream()
    announce("moe_layer_q4 graph capture")
    with torch.cuda.stream(s):
        layer.forward(x, lg, out=y, stream=s)     # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer.forward(x, lg, out=y, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bq.bf16_to_bits(y), want), rep
        layer.forward_three_calls(x, lg)         # eager work between replays
        torch.cuda.synchronize()
