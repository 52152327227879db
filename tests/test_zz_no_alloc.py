"""moe_decode_q4_noalloc (the decode entry point that allocates nothing: its
workspace is the library's device-resident scratch array) gives bit for bit
what moe_decode_q4 gives with a caller workspace, through the C ABI, on two
calls in a row, the second on a smaller layer; its size limit is enforced."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
from gpu_cases import DEV, announce, require_gpu
from workload import CONFIGS, make_activations, make_weights, small_config

pytestmark = pytest.mark.gpu


def _layer_inputs(cfg, wseed, t):
    w = make_weights(cfg, seed=wseed, cache=False)
    x_bits, logits = make_activations(cfg)
    layer = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV, prepack=True)
    x = bq.bf16_from_bits(np.ascontiguousarray(x_bits[t:t + 1]), DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits[t:t + 1])).to(DEV)
    return layer, x, lg


def _both(layer, x, lg):
    """(y, routing) from moe_decode_q4 with a fresh workspace, then from the no-alloc entry."""
    E, k, H = layer.E, layer.k, layer.H
    out = []
    for noalloc in (False, True):
        r = bq.DeviceRouting(1, E, k, 32, DEV)
        y = torch.full((1, H), float("nan"), dtype=torch.bfloat16, device=DEV)
        if noalloc:
            bq.moe_decode_q4_noalloc(x, lg, layer.I, layer.I_sh, k, 32, *layer.weight_mats(), r, y)
        else:
            ws = torch.empty(bq.decode_workspace_bytes(H, layer.I, layer.I_sh, E, k),
                             dtype=torch.uint8, device=DEV)
            bq.moe_decode_q4(x, lg, layer.I, layer.I_sh, k, 32, *layer.weight_mats(), r, y, ws)
        torch.cuda.synchronize()
        out.append((bq.bf16_to_bits(y), r.to_host()))
    return out


def test_noalloc_decode_equals_workspace_decode_twice():
    require_gpu()
    big = CONFIGS["prefill512"]
    small = small_config(4, 256, 128, 16, 2, 128, seed=3)
    for name, cfg, wseed, t in (("full-size layer", big, 0, 7), ("smaller layer", small, 11, 2)):
        announce(f"no-alloc decode, {name}")
        layer, x, lg = _layer_inputs(cfg, wseed, t)
        (y_ws, r_ws), (y_na, r_na) = _both(layer, x, lg)
        assert not np.isnan((y_na.astype(np.uint32) << 16).view(np.float32)).any()
        assert np.array_equal(y_na, y_ws), name
        for key in r_ws:
            assert np.array_equal(r_na[key], r_ws[key]), (name, key)


def test_noalloc_rejects_shapes_past_its_scratch():
    require_gpu()
    limit = bq.decode_noalloc_max_bytes()
    assert limit == 256 * 1024
    # k = 64 experts of I = 2048: (k + 1) * I * 2 bytes of h is far past the scratch
    assert bq.decode_workspace_bytes(2048, 2048, 2048, 256, 64) > limit
    L = bq.lib()
    fake = ctypes.c_void_p(0x10000)
    m = bq.MoeQ4Mat(fake.value, fake.value, fake.value, 0)
    mats = [ctypes.byref(m)] * 6
    st = L.moe_decode_q4_noalloc(fake, fake, 2048, 2048, 2048, 256, 64, 32, *mats, None, fake, None)
    assert st == bq.MOE_ERR_WORKSPACE
