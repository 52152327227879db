"""Full-size workloads checked on EVERY token against the oracle, in the
tile-packed code layout the bench times and in the row-major one:

  prefill512 / prefill2048  one layer call each (y and expert_out per element;
                            routing bit-exact);
  skew8192                  the bounded-chunk driver, all four 2048-token chunks
                            (the tolerance normaliser is each chunk's max|y|);
  decode                    all 1000 tokens through moe_decode_q4 (two launches
                            per token): the T = 1 routing arrays bit-exact and y
                            per token (normaliser: the token's max|y|);
  cold decode               the bench's cold run: token t on layer copy t mod 4,
                            copies 1-3 with code words XOR-ed by a per-copy
                            constant, replayed from a captured graph.

The oracle computes each token independently, so one oracle call over a set of
tokens gives every token's reference (decode tokens share one batched call)."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
import oracle
from gpu_cases import (DEV, announce, assert_routing_matches, bf16_bits_to_f64, oracle_layer,
                       require_gpu, run_layer, tol_ok)
from workload import CONFIGS, QMat, LayerWeights, make_activations, make_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def layers():
    cfg = CONFIGS["prefill512"]
    w = make_weights(cfg, seed=0)
    rows = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    tiles = bq.MoeLayer.from_device(bq.prepacked_mats(rows.weight_mats()),
                                    cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    torch.cuda.synchronize()
    return w, {"rows": rows, "tiles": tiles}


def _check_per_token(y_bits, y_ref, what):
    """Every token within 2e-2 * max|y[t]| + 1e-3 (the per-call normaliser of one token)."""
    got = bf16_bits_to_f64(y_bits)
    bound = 2e-2 * np.max(np.abs(y_ref), axis=1, keepdims=True) + 1e-3
    ratio = np.abs(got - y_ref) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, f"{what}: token {worst[0]} column {worst[1]} at {ratio.max():.3f} x bound"


@pytest.mark.parametrize("name", ["prefill512", "prefill2048"])
def test_prefill_every_token(layers, name):
    w, L = layers
    cfg = CONFIGS[name]
    x_bits, logits = make_activations(cfg)
    announce(f"oracle {name} (all {cfg.T} tokens)")
    ref = oracle_layer(w, cfg, x_bits, logits)
    for layout, layer in L.items():
        announce(f"workload {name} every token, {layout} layout")
        got = run_layer(layer, x_bits, logits)
        assert_routing_matches(got["routing"], logits, cfg.k)
        ok, ratio = tol_ok(bf16_bits_to_f64(got["y"]), ref["y"])
        assert ok, f"{layout} y: {ratio:.3f} x bound"
        ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
        assert ok, f"{layout} expert_out: {ratio:.3f} x bound"
        ok, ratio = tol_ok(bf16_bits_to_f64(got["shared_out"]), ref["shared_out"])
        assert ok, f"{layout} shared_out: {ratio:.3f} x bound"


def test_skewed_chunks_every_token(layers):
    w, L = layers
    cfg = CONFIGS["skew8192"]
    x_bits, logits = make_activations(cfg)
    x = bq.bf16_from_bits(x_bits, DEV)
    lg = torch.from_numpy(logits).to(DEV)
    announce("oracle skew8192 (four chunks of 2048)")
    ref_y, parts = oracle.moe_layer_chunked(x_bits, logits, w.gate, w.up, w.down, cfg.k,
                                            w.sh_gate, w.sh_up, w.sh_down, chunk=cfg.chunk)
    # the skew really is skewed: one expert takes most tokens of a chunk, many are empty
    counts = parts[0]["counts"]
    assert counts.max() > 0.9 * cfg.chunk and np.count_nonzero(counts == 0) > 64
    for layout, layer in L.items():
        announce(f"skew8192 chunked, {layout} layout")
        y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=DEV)
        layer.forward_chunked(x, lg, cfg.chunk, y)
        torch.cuda.synchronize()
        y_bits = bq.bf16_to_bits(y)
        for c0 in range(0, cfg.T, cfg.chunk):
            ok, ratio = tol_ok(bf16_bits_to_f64(y_bits[c0:c0 + cfg.chunk]), ref_y[c0:c0 + cfg.chunk])
            assert ok, f"{layout} chunk {c0}: {ratio:.3f} x bound"


def _decode_tokens(layer_of, x_bits, logits, tokens, k, block_rows=32, graph=False):
    """moe_decode_q4 per token (token t on layer_of(t)), with the T = 1 routing arrays;
    returns y bits [n, H] and the routing arrays per token (None under a graph)."""
    n = len(tokens)
    H = x_bits.shape[1]
    x = bq.bf16_from_bits(np.ascontiguousarray(x_bits[tokens]), DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits[tokens])).to(DEV)
    L0 = layer_of(tokens[0])
    ws = torch.empty(bq.decode_workspace_bytes(H, L0.I, L0.I_sh, L0.E, k), dtype=torch.uint8,
                     device=DEV)
    y = torch.zeros((n, H), dtype=torch.bfloat16, device=DEV)
    routes = None if graph else [bq.DeviceRouting(1, L0.E, k, block_rows, DEV) for _ in range(n)]

    def calls():
        for i, t in enumerate(tokens):
            L = layer_of(t)
            bq.moe_decode_q4(x[i:i + 1], lg[i:i + 1], L.I, L.I_sh, k, block_rows,
                             *L.decode_mats(), None if graph else routes[i], y[i:i + 1], ws)

    if graph:
        calls()                                   # eager first: the replay must match it
        torch.cuda.synchronize()
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        for rep in range(2):
            y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
        del g
    else:
        calls()
    torch.cuda.synchronize()
    return bq.bf16_to_bits(y), (None if graph else [r.to_host() for r in routes])


def test_decode_every_token(layers):
    w, L = layers
    cfg = CONFIGS["decode"]
    x_bits, logits = make_activations(cfg)
    announce("oracle decode (1000 tokens, one batched call)")
    ref = oracle_layer(w, cfg, x_bits, logits)
    tokens = list(range(cfg.T))
    for layout, layer in L.items():
        announce(f"decode all {cfg.T} tokens, {layout} layout")
        y, routes = _decode_tokens(lambda t: layer, x_bits, logits, tokens, cfg.k)
        for t in tokens:
            assert_routing_matches(routes[t], logits[t:t + 1], cfg.k)
        _check_per_token(y, ref["y"], f"decode {layout}")


def _xor_codes(w: LayerWeights, c: int) -> LayerWeights:
    x = lambda m: None if m is None else QMat(m.codes ^ np.uint32(c), m.scales, m.biases)  # noqa: E731
    return LayerWeights(x(w.gate), x(w.up), x(w.down), x(w.sh_gate), x(w.sh_up), x(w.sh_down))


def test_cold_decode_copies_from_a_graph(layers):
    """The bench's cold decode: copies 1-3 are made on the device from copy 0 by XOR-ing every
    code word with 0x01010101 * copy; token t runs on copy t mod 4, replayed from a graph."""
    w, L = layers
    cfg = CONFIGS["decode"]
    x_bits, logits = make_activations(cfg)
    base = L["tiles"]
    copies = [base] + [
        bq.MoeLayer.from_device(
            [None if m is None else bq.DeviceQMat(
                m.codes ^ (0x01010101 * i), m.scales.clone(),
                None if m.biases is None else m.biases.clone(), m.layout,
                plain=None if m.plain is None else tuple(t.clone() for t in m.plain))
             for m in base.weight_mats()], cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
        for i in range(1, 4)]
    tokens = list(range(64))
    announce("cold decode: 64 tokens over 4 layer copies, graph replay")
    y, _ = _decode_tokens(lambda t: copies[t % 4], x_bits, logits, tokens, cfg.k, graph=True)
    for i in range(4):
        wi = w if i == 0 else _xor_codes(w, 0x01010101 * i)
        sel = tokens[i::4]
        announce(f"oracle cold copy {i} ({len(sel)} tokens)")
        ref = oracle_layer(wi, cfg, x_bits[sel], logits[sel])
        _check_per_token(y[i::4], ref["y"], f"cold copy {i}")
