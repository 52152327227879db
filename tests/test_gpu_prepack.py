"""Tile-packed code words (moe_q4_prepack) and packed scale|bias words
(moe_q4_pack_scales): each repack is exactly the permutation the header
documents, and every output of the layer and of decode is bit-identical in
the three layouts (row-major; tile-packed codes; tile-packed codes with packed
gate/up scale|bias words): only the addresses change, not the arithmetic or
its order."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
from gpu_cases import DEV, announce, layer_to_host, require_gpu, run_layer
from workload import CONFIGS, make_activations, make_weights, small_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _packed_reference(codes, N, K):
    """The header's formula, word by word: (e, n, c) -> e*N*K/8 + ((n/64)*(K/64) + c/8)*512
    + ((n%64)/16)*128 + (n%16)*8 + c%8."""
    n_exp = codes.shape[0]
    out = np.empty(codes.size, codes.dtype)
    e, n, c = np.meshgrid(np.arange(n_exp), np.arange(N), np.arange(K // 8), indexing="ij")
    to = (e * N * (K // 8) + ((n // 64) * (K // 64) + c // 8) * 512 + ((n % 64) // 16) * 128
          + (n % 16) * 8 + c % 8)
    out[to.reshape(-1)] = codes.reshape(-1)
    return out


@pytest.mark.parametrize("n_exp,N,K", [(3, 128, 192), (2, 64, 64), (1, 512, 2048)])
def test_prepack_is_the_documented_permutation(n_exp, N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 2 ** 32, (n_exp, N, K // 8), dtype=np.uint32)
    src = torch.from_numpy(codes.view(np.int32)).to(DEV)
    dst = torch.zeros_like(src)
    announce(f"prepack permutation {n_exp}x{N}x{K}")
    assert bq.lib().moe_q4_prepack(src.data_ptr(), n_exp, N, K, dst.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(-1)
    want = _packed_reference(codes, N, K)
    assert np.array_equal(got, want)
    assert np.array_equal(np.sort(got), np.sort(codes.reshape(-1)))


@pytest.mark.parametrize("n_exp,N,K", [(3, 128, 192), (2, 64, 64), (1, 512, 2048)])
def test_pack_scales_is_the_documented_order(n_exp, N, K):
    """dst[((n/64)*(K/64) + g)*64 + n%64] = scale bits | bias bits << 16, n = e*N + n'."""
    rng = np.random.default_rng(N * 3 + K)
    G = K // 64
    sc = rng.integers(0, 2 ** 16, (n_exp, N, G), dtype=np.uint16)
    bi = rng.integers(0, 2 ** 16, (n_exp, N, G), dtype=np.uint16)
    s_d = torch.from_numpy(sc.view(np.int16)).to(DEV)
    b_d = torch.from_numpy(bi.view(np.int16)).to(DEV)
    dst = torch.zeros((n_exp, N, G), dtype=torch.int32, device=DEV)
    announce(f"pack scales {n_exp}x{N}x{K}")
    assert bq.lib().moe_q4_pack_scales(s_d.data_ptr(), b_d.data_ptr(), n_exp, N, K,
                                       dst.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(-1)
    rows = np.arange(n_exp * N)
    n, g = np.meshgrid(rows, np.arange(G), indexing="ij")
    want = np.empty(n_exp * N * G, np.uint32)
    want[((n // 64) * G + g) * 64 + n % 64] = (sc.reshape(-1, G).astype(np.uint32)
                                              | (bi.reshape(-1, G).astype(np.uint32) << 16))
    assert np.array_equal(got, want)


SHAPES = [
    # T,   H,    I,   E,  k, I_sh, block_rows
    (64, 256, 128, 16, 2, 128, 32),
    (200, 512, 256, 32, 4, 256, 32),
    (37, 256, 128, 8, 3, 0, 16),
    (130, 384, 192, 12, 2, 320, 64),      # K = 192 and 320: the 64-K chunk path
    (70, 384, 512, 8, 2, 512, 32),        # down K = 512 over whole-K tiles, partial column group
    (301, 320, 512, 4, 2, 512, 32),       # 64-row down items (block pairs), partial column group
]


@pytest.mark.parametrize("T,H,I,E,k,I_sh,block_rows", SHAPES)
def test_layer_outputs_identical_in_both_layouts(T, H, I, E, k, I_sh, block_rows):
    cfg = small_config(T, H, I, E, k, I_sh, seed=T + 1)
    w = make_weights(cfg, seed=T + H + 1, cache=False)
    x_bits, logits = make_activations(cfg)
    rows = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=block_rows)
    tiles = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=block_rows, prepack="codes")
    packed = bq.MoeLayer(w, H, I, I_sh, E, k, DEV, block_rows=block_rows, prepack=True)
    assert tiles.gate.layout == bq.LAYOUT_TILES
    assert packed.gate.layout == bq.LAYOUT_TILES_SB and packed.down.layout == bq.LAYOUT_TILES
    announce(f"layouts T={T} H={H} I={I} E={E} k={k} I_sh={I_sh} br={block_rows}")
    a = run_layer(rows, x_bits, logits)
    for L in (tiles, packed):
        b = run_layer(L, x_bits, logits)
        for key in ("y", "expert_out") + (("shared_out",) if I_sh else ()):
            assert np.array_equal(a[key], b[key]), (L.gate.layout, key)
    # decode: token by token through the two-launch path (MoeLayer.decode gives the packed
    # layer's plain-scale view; the packed matrices are also passed to moe_decode_q4 as is)
    ws = torch.empty(bq.decode_workspace_bytes(H, I, I_sh, E, k), dtype=torch.uint8, device=DEV)
    for t in (0, T - 1):
        ys = []
        x = bq.bf16_from_bits(x_bits[t:t + 1], DEV)
        lg = torch.from_numpy(np.ascontiguousarray(logits[t:t + 1])).to(DEV)
        for L in (rows, tiles, packed):
            y = torch.empty((1, H), dtype=torch.bfloat16, device=DEV)
            L.decode(x, lg, y)
            torch.cuda.synchronize()
            ys.append(bq.bf16_to_bits(y))
        y = torch.empty((1, H), dtype=torch.bfloat16, device=DEV)
        bq.moe_decode_q4(x, lg, I, I_sh, k, block_rows, *packed.weight_mats(), None, y, ws)
        torch.cuda.synchronize()
        ys.append(bq.bf16_to_bits(y))
        assert np.array_equal(ys[0], ys[1]), f"decode token {t} (tiles)"
        assert np.array_equal(ys[0], ys[2]), f"decode token {t} (packed layer, plain view)"
        assert np.array_equal(ys[0], ys[3]), f"decode token {t} (packed scale|bias words)"


@pytest.mark.parametrize("name", ["prefill512", "prefill2048"])
def test_prefill_identical_in_both_layouts(name):
    """The bench times the tile-packed order; the full-size workloads must give
    the row-major order's outputs bit for bit (2048 tokens also takes the
    64-row paired down items)."""
    cfg = CONFIGS[name]
    w = make_weights(cfg, seed=0)
    rows = bq.MoeLayer(w, cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    tiles = bq.MoeLayer.from_device(bq.prepacked_mats(rows.weight_mats(), pack_scales=False),
                                    cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    packed = bq.MoeLayer.from_device(bq.prepacked_mats(rows.weight_mats()),
                                     cfg.H, cfg.I, cfg.I_sh, cfg.E, cfg.k, DEV)
    x_bits, logits = make_activations(cfg)
    announce(f"layouts {name}")
    a = run_layer(rows, x_bits, logits)
    for L in (tiles, packed):
        b = run_layer(L, x_bits, logits)
        assert np.array_equal(a["y"], b["y"]), L.gate.layout
        assert np.array_equal(a["expert_out"], b["expert_out"]), L.gate.layout
    # batch-1 decode over the same full-size weights, as the bench times it
    for t in (0, cfg.T // 2, cfg.T - 1):
        ys = []
        for L in (rows, tiles, packed):
            xt = bq.bf16_from_bits(x_bits[t:t + 1], DEV)
            lg = torch.from_numpy(np.ascontiguousarray(logits[t:t + 1])).to(DEV)
            y = torch.empty((1, cfg.H), dtype=torch.bfloat16, device=DEV)
            L.decode(xt, lg, y)
            torch.cuda.synchronize()
            ys.append(bq.bf16_to_bits(y))
        assert np.array_equal(ys[0], ys[1]), f"decode token {t}"
        assert np.array_equal(ys[0], ys[2]), f"decode token {t} (packed scales)"
