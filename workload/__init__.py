"""Seeded synthetic inputs for the 4-bit MoE layer (test and bench infrastructure).

This module only draws and stores inputs: random codes, scales, biases,
activations and router logits, in the storage formats the layer consumes
(codes packed eight per uint32 with the lowest-k nibble in the low bits;
scales, biases and activations as bf16 bit patterns in uint16).  It holds
none of the layer's arithmetic: no dequantization, routing, FFN or combine.
Both the CPU oracle and the HIP path are fed from here and from nowhere else.

bf16 storage rounding uses torch's CPU float32 -> bfloat16 conversion
(round to nearest even); the oracle has its own, separately pinned, rounding.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

GROUP = 64  # weights per (scale, bias) pair along K


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens in the workload (all chunks together)
    H: int            # hidden size
    I: int            # routed expert intermediate size
    E: int            # routed experts
    k: int            # experts per token
    I_sh: int         # shared expert intermediate size (0 = no shared expert)
    act_seed: int     # seed of the activation / logit generator
    chunk: int = 0    # bounded-chunk size (0 = one call over all T tokens)
    per_token: bool = False   # decode: T independent single-token calls
    zipf_s: float = 0.0       # > 0: per-expert popularity bias on the logits

    @property
    def call_tokens(self) -> int:
        """Tokens seen by one layer call."""
        if self.per_token:
            return 1
        if self.chunk:
            return min(self.chunk, self.T)
        return self.T


# The five workloads: a tiny correctness layer, two prefill sizes, batch-1
# decode over 1000 tokens, and a Zipf-skewed 8192-token prefill run in
# bounded chunks of 2048.  Configs 2-5 share one layer (same weights).
CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, H=256, I=128, E=16, k=2, I_sh=128, act_seed=0),
    "prefill512": LayerConfig("prefill512", T=512, H=2048, I=512, E=256, k=8, I_sh=512, act_seed=1),
    "prefill2048": LayerConfig("prefill2048", T=2048, H=2048, I=512, E=256, k=8, I_sh=512, act_seed=2),
    "decode": LayerConfig("decode", T=1000, H=2048, I=512, E=256, k=8, I_sh=512, act_seed=3,
                          per_token=True),
    "skew8192": LayerConfig("skew8192", T=8192, H=2048, I=512, E=256, k=8, I_sh=512, act_seed=4,
                            chunk=2048, zipf_s=1.1),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Pack codes [..., K] (values 0..15) into uint32 words [..., K/8].

    Nibble i of word c holds code 8c+i (bits 4i..4i+3, lowest k in the low bits).
    """
    K = q.shape[-1]
    assert K % 8 == 0
    q8 = q.reshape(*q.shape[:-1], K // 8, 8)
    out = np.zeros(q8.shape[:-1], np.uint32)
    for i in range(8):
        out |= q8[..., i].astype(np.uint32) << np.uint32(4 * i)
    return out


@dataclasses.dataclass
class QMat:
    """One 4-bit matrix set [n_exp, N, K]: packed codes and bf16 scale/bias bits."""
    codes: np.ndarray   # uint32 [n_exp, N, K/8]
    scales: np.ndarray  # uint16 [n_exp, N, K/64]
    biases: np.ndarray  # uint16 [n_exp, N, K/64]

    @property
    def shape(self):
        n_exp, N, K8 = self.codes.shape
        return n_exp, N, K8 * 8


def draw_qmat(rng: np.random.Generator, n_exp: int, N: int, K: int) -> QMat:
    """Codes uniform 0..15, scales bf16(U(0.005, 0.02)), biases = -8 * scale (exact)."""
    assert K % GROUP == 0
    q = rng.integers(0, 16, (n_exp, N, K), dtype=np.uint8)
    codes = pack_nibbles(q)
    del q
    s32 = rng.uniform(0.005, 0.02, (n_exp, N, K // GROUP)).astype(np.float32)
    s_bits = f32_to_bf16_bits(s32)
    s_val = (s_bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    b_bits = f32_to_bf16_bits(np.float32(-8.0) * s_val)
    return QMat(codes, s_bits, b_bits)


@dataclasses.dataclass
class LayerWeights:
    gate: QMat      # [E, I, H]
    up: QMat        # [E, I, H]
    down: QMat      # [E, H, I]
    sh_gate: QMat | None   # [1, I_sh, H]
    sh_up: QMat | None
    sh_down: QMat | None   # [1, H, I_sh]

    def nbytes(self) -> int:
        tot = 0
        for m in (self.gate, self.up, self.down, self.sh_gate, self.sh_up, self.sh_down):
            if m is not None:
                tot += m.codes.nbytes + m.scales.nbytes + m.biases.nbytes
        return tot


_WEIGHT_CACHE: dict = {}


def make_weights(cfg: LayerConfig, seed: int = 0, cache: bool = True) -> LayerWeights:
    """Draw one layer's weights with default_rng(seed), in the order
    gate, up, down, shared gate, shared up, shared down."""
    key = (cfg.H, cfg.I, cfg.E, cfg.I_sh, seed)
    if cache and key in _WEIGHT_CACHE:
        return _WEIGHT_CACHE[key]
    rng = np.random.default_rng(seed)
    gate = draw_qmat(rng, cfg.E, cfg.I, cfg.H)
    up = draw_qmat(rng, cfg.E, cfg.I, cfg.H)
    down = draw_qmat(rng, cfg.E, cfg.H, cfg.I)
    if cfg.I_sh:
        sg = draw_qmat(rng, 1, cfg.I_sh, cfg.H)
        su = draw_qmat(rng, 1, cfg.I_sh, cfg.H)
        sd = draw_qmat(rng, 1, cfg.H, cfg.I_sh)
    else:
        sg = su = sd = None
    w = LayerWeights(gate, up, down, sg, su, sd)
    if cache:
        _WEIGHT_CACHE.clear()
        _WEIGHT_CACHE[key] = w
    return w


def make_router(cfg: LayerConfig, seed: int = 100):
    """Router weights bf16 [E, H] and a shared-expert gate row bf16 [H] (uint16
    bit patterns), drawn N(0, 1/H) with default_rng(seed) so that router
    logits over N(0, 1) activations are about N(0, 1) like the drawn logits."""
    rng = np.random.default_rng(seed)
    scale = np.float32(1.0 / np.sqrt(cfg.H))
    wr = f32_to_bf16_bits(rng.standard_normal((cfg.E, cfg.H), dtype=np.float32) * scale)
    wg = f32_to_bf16_bits(rng.standard_normal(cfg.H, dtype=np.float32) * scale)
    return wr, wg


def zipf_bias(E: int, s: float, perm: np.ndarray) -> np.ndarray:
    """Per-expert log-popularity bias: expert perm[i] gets rank i+1 and bias -s*ln(rank)."""
    rank = np.empty(E, np.int64)
    rank[perm] = np.arange(1, E + 1)
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def make_activations(cfg: LayerConfig):
    """Return (x_bits uint16 [T, H], logits float32 [T, E]) for all T tokens."""
    rng = np.random.default_rng(cfg.act_seed)
    perm = rng.permutation(cfg.E) if cfg.zipf_s > 0 else None
    x_bits = f32_to_bf16_bits(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))
    logits = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if perm is not None:
        logits = (logits + zipf_bias(cfg.E, cfg.zipf_s, perm)).astype(np.float32)
    return x_bits, logits


def small_config(T: int, H: int, I: int, E: int, k: int, I_sh: int, seed: int = 0,
                 name: str = "custom") -> LayerConfig:
    return LayerConfig(name, T=T, H=H, I=I, E=E, k=k, I_sh=I_sh, act_seed=seed)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 values (exact).  Storage helper for
    callers that need to display or compare stored inputs."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("math", "np", "torch",
                                                                      "dataclasses", "annotations")]
