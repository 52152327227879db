"""Random layer shapes through the C ABI against the oracle: routing bit-exact,
expert_out / shared_out / y within 2e-2 * max|oracle| + 1e-3, in all three
weight layouts and block heights, with the bounded-chunk driver at a random
chunk size and the batch-1 decode entry for the smallest T.

The default run draws MOE_SWEEP_CASES = 40 cases from MOE_SWEEP_SEED = 0 (the
same cases every run); set either variable for a longer or a fresh sweep.
Shapes are capped so that the oracle's dense fp64 weights stay small."""
import os

import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
from gpu_cases import (DEV, announce, assert_close_layer, assert_routing_matches, oracle_layer,
                       require_gpu, run_layer, tol_ok, bf16_bits_to_f64)
from workload import make_activations, make_weights, small_config

pytestmark = pytest.mark.gpu

CASES = int(os.environ.get("MOE_SWEEP_CASES", "40"))
SEED = int(os.environ.get("MOE_SWEEP_SEED", "0"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _draw(rng):
    T = int(rng.choice([rng.integers(1, 5), rng.integers(1, 300), rng.integers(300, 1200)],
                       p=[0.2, 0.6, 0.2]))
    H = 64 * int(rng.integers(1, 25))
    I = 64 * int(rng.integers(1, 13))
    E = int(rng.choice([rng.integers(1, 40), rng.integers(40, 300), rng.integers(300, 1001)],
                       p=[0.5, 0.4, 0.1]))
    k = int(rng.integers(1, min(E, 16) + 1)) if rng.random() < 0.9 else int(rng.integers(1, min(E, 64) + 1))
    while E * 3 * H * I > 6e7 and (H > 64 or I > 64):
        if H >= I:
            H = max(64, (H // 2) // 64 * 64)
        else:
            I = max(64, (I // 2) // 64 * 64)
    I_sh = 64 * int(rng.integers(0, 9))
    br = int(rng.choice([16, 32, 64]))
    layout = str(rng.choice(["rows", "codes", "packed"]))
    chunk = int(rng.integers(16, T + 1)) if T > 64 and rng.random() < 0.5 else 0
    return T, H, I, E, k, I_sh, br, layout, chunk, int(rng.integers(0, 2 ** 20))


def test_random_layer_shapes():
    rng = np.random.default_rng(SEED)
    for case in range(CASES):
        T, H, I, E, k, I_sh, br, layout, chunk, s = _draw(rng)
        tag = (f"sweep case {case} T={T} H={H} I={I} E={E} k={k} I_sh={I_sh} br={br} "
               f"layout={layout} chunk={chunk} seed={s}")
        announce(tag)
        cfg = small_config(T, H, I, E, k, I_sh, seed=s)
        w = make_weights(cfg, seed=s + 1, cache=False)
        x_bits, logits = make_activations(cfg)
        prepack = {"rows": False, "codes": "codes", "packed": True}[layout]
        layer = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=br, prepack=prepack)
        got = run_layer(layer, x_bits, logits)
        ref = oracle_layer(w, cfg, x_bits, logits, br)
        assert_routing_matches(got["routing"], logits, k, br)
        ok, ratio = tol_ok(bf16_bits_to_f64(got["expert_out"]), ref["expert_out"])
        assert ok, f"{tag}: expert_out {ratio:.3f}"
        if I_sh:
            ok, ratio = tol_ok(bf16_bits_to_f64(got["shared_out"]), ref["shared_out"])
            assert ok, f"{tag}: shared_out {ratio:.3f}"
        assert_close_layer(got["y"], ref["y"], what=f"{tag}: y")
        x = bq.bf16_from_bits(x_bits, DEV)
        lg = torch.from_numpy(np.ascontiguousarray(logits)).to(DEV)
        if chunk:
            yc = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
            layer.forward_chunked(x, lg, chunk, yc)
            torch.cuda.synchronize()
            assert_close_layer(bq.bf16_to_bits(yc), ref["y"], what=f"{tag}: chunked y")
        if T <= 4:
            for t in range(T):
                y = torch.empty((1, H), dtype=torch.bfloat16, device=DEV)
                layer.decode(x[t:t + 1], lg[t:t + 1], y)
                torch.cuda.synchronize()
                assert_close_layer(bq.bf16_to_bits(y)[0], ref["y"][t], what=f"{tag}: decode token {t}")
