"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare with the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import bit_quantized_grouped_amd as bq
import oracle
from workload import bf16_bits_to_f32

DEV = "cuda:0"


def announce(msg: str):
    """Name the case on stderr before a GPU step (survives output capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    bq.lib()   # raises if the HIP library is missing


def gpu_route(logits_np: np.ndarray, k: int, block_rows: int = 32) -> dict:
    T, E = logits_np.shape
    logits = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).to(DEV)
    r = bq.DeviceRouting(T, E, k, block_rows, DEV)
    ws = torch.empty(max(bq.route_workspace_bytes(T, E, k, block_rows), 256), dtype=torch.uint8,
                     device=DEV)
    bq.moe_route(logits, k, block_rows, r, ws)
    torch.cuda.synchronize()
    return r.to_host()


def assert_routing_matches(got: dict, logits_np: np.ndarray, k: int, block_rows: int = 32):
    T, E = logits_np.shape
    idx, w = oracle.route_topk(logits_np, k)
    g = oracle.group(idx, E, block_rows)
    assert np.array_equal(got["topk_idx"], idx), "topk_idx"
    assert np.max(np.abs(got["topk_w"].astype(np.float64) - w)) <= 1e-6, "topk_w"
    for key in ("counts", "offsets", "sorted_assign", "assign_row", "block_expert", "block_row"):
        assert np.array_equal(got[key], g[key]), key
    assert int(got["n_blocks"][0]) == int(g["n_blocks"]), "n_blocks"


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def tol_ok(got: np.ndarray, ref: np.ndarray, rel: float = 2e-2, abs_: float = 1e-3):
    """|got - ref| <= rel * max|ref| + abs_ per element; returns (ok, worst excess ratio)."""
    bound = rel * float(np.max(np.abs(ref))) + abs_
    err = np.abs(got - ref)
    return bool(np.all(err <= bound)), float(np.max(err) / bound)


def assert_close_layer(y_bits: np.ndarray, y_ref: np.ndarray, what: str = "y"):
    ok, ratio = tol_ok(bf16_bits_to_f64(y_bits), y_ref)
    assert ok, f"{what}: max error is {ratio:.3f} x the bound"
    return ratio


def layer_to_host(bufs: dict) -> dict:
    out = dict(routing=bufs["routing"].to_host(), y=bq.bf16_to_bits(bufs["y"]),
               expert_out=bq.bf16_to_bits(bufs["expert_out"]))
    if bufs["shared_out"] is not None:
        out["shared_out"] = bq.bf16_to_bits(bufs["shared_out"])
    return out


def run_layer(layer: "bq.MoeLayer", x_bits: np.ndarray, logits: np.ndarray) -> dict:
    x = bq.bf16_from_bits(x_bits, DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    bufs = layer.forward(x, lg)
    torch.cuda.synchronize()
    return layer_to_host(bufs)


def oracle_layer(w, cfg, x_bits, logits, block_rows=32):
    return oracle.moe_layer(x_bits, logits, w.gate, w.up, w.down, cfg.k, w.sh_gate, w.sh_up,
                            w.sh_down, block_rows=block_rows)
