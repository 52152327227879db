"""Plain CPU oracle of the 4-bit grouped MoE layer.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in __graft_entry__ and the cpu_baseline
leg of bench.py may import or call this module.  The product path (the HIP
library and its Python binding) never does, and shares no code with it.

What it computes, and where the pages say so.  The pages are three news
reports on Perplexity's "Lily" engine:
  [P1] dothoosh.com, "Perplexity Lily: 1.35x faster decode for Qwen3.6 on
       Apple silicon" (Persian);
  [P2] aikraft.ru, "Perplexity open-sources Lily, a Rust/Metal inference
       engine for Qwen3.6" (Russian);
  [P3] droneth.or.th, post on Lily (Thai).

* Weights are 4-bit groupwise-affine: each run of 64 weights shares one bf16
  scale and one bf16 bias ([P1] "Prefill optimizations", fused-dequantization
  bullet; [P3] "A big model that touches only part of its weights per
  token").  The engine expands them to bf16 because its tensor units take
  bf16, and accumulates in FP32 ([P3], same section).  Dequantization here is
  w = bf16_rne(fp32(q * scale + bias)), widened to fp64.
* A router scores 256 experts, keeps 8, and one shared expert sees every
  token ([P1] "Model specification"; [P2] "Qwen3.6-35B-A3B architecture";
  [P3] same section as above).  Selection is by descending fp32 logit with
  ties to the lower expert index; the k weights are the softmax over the k
  selected logits (equal to the full softmax renormalised over the top k).
* Routing is histogram -> prefix scan -> scatter -> block map ([P1]
  "Prefill optimizations", GPU-resident routing bullet; [P3] ablation
  paragraph).  Grouping here is the plain definition: bincount, exclusive
  cumulative sum, stable sort by expert, and 32-row tiles per expert
  ([P1] tiling bullet, 16 -> 32-row tiles).
* Each expert is a SwiGLU FFN (silu(x Wg^T) * (x Wu^T)) Wd^T with no biases;
  the layer output is the routing-weighted sum of the k expert outputs plus
  the shared expert's output with weight 1 (unless the optional gate is on).
* Long prompts run in bounded chunks ([P1] "Prefill optimizations", memory
  bullet): each chunk is an independent layer call.
* The router's scores are a plain projection of the token's activations,
  logits = x W_r^T in fp64 ([P1] "Model specification"); an optional
  per-token shared-expert weight sigmoid(x . w_g) (not named by the pages,
  off unless asked) scales the shared expert's output.

Readings taken where the pages are silent are listed in the design notes of
the repository; every one of them is applied here and nowhere else.

All floating point after dequantization is fp64.  Routing decisions are
taken on the fp32 logits exactly as stored (comparisons are exact).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


# ----------------------------------------------------------------------------
# bf16 helpers (own implementation; pinned by the hand-worked groups)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 values; exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_rne_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, round-to-nearest-even on the 16 dropped bits.

    Inputs are finite; overflow past the bf16 range rounds to infinity as
    IEEE rounding does.
    """
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


# ----------------------------------------------------------------------------
# Dequantization ([P1] "Prefill optimizations"; [P3] "A big model ...")
# ----------------------------------------------------------------------------

def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint32 words [..., K/8] -> 4-bit codes [..., K]; code 8c+i is bits 4i..4i+3 of word c."""
    w = np.asarray(codes, dtype=np.uint32)
    shifts = (np.arange(8, dtype=np.uint32) * np.uint32(4))
    q = (w[..., None] >> shifts) & np.uint32(0xF)
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8).astype(np.uint8)


def dequant_bf16_bits(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """Dequantized weights as bf16 bit patterns [..., N, K].

    For weight (n, k): q = code, s = scales[n, k // 64], b = biases[n, k // 64];
    value = fp32(q * s + b) rounded once to fp32 (q * s is exact in fp32),
    then rounded to bf16 with round-to-nearest-even.
    """
    q = unpack_codes(codes).astype(np.float32)
    K = q.shape[-1]
    s = bf16_bits_to_f64(scales).astype(np.float32)
    b = bf16_bits_to_f64(biases).astype(np.float32)
    assert s.shape[-1] * GROUP == K, "one scale per 64 weights along K"
    s_full = np.repeat(s, GROUP, axis=-1)
    b_full = np.repeat(b, GROUP, axis=-1)
    v32 = q * s_full + b_full          # float32 arithmetic: exact product, one rounding
    return f32_to_bf16_rne_bits(v32)


def dequant(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """Dequantized weights [..., N, K] as fp64 (bf16-valued)."""
    return bf16_bits_to_f64(dequant_bf16_bits(codes, scales, biases))


# ----------------------------------------------------------------------------
# Routing ([P1] "Model specification", "Prefill optimizations"; [P3])
# ----------------------------------------------------------------------------

def route_topk(logits: np.ndarray, k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Selection repeats k times: take the largest remaining logit, the lowest
    expert index on ties (-0.0 and +0.0 are equal), and remove it.
    Weights: exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k chosen,
    in fp64 from the fp32 logits.
    Returns idx int32 [T, k] (slot order = selection order) and w fp64 [T, k].
    """
    L = np.array(logits, dtype=np.float32, copy=True)
    T, E = L.shape
    assert 1 <= k <= E
    L64 = L.astype(np.float64) + 0.0          # canonical +0.0; values exact
    avail = np.ones((T, E), dtype=bool)
    idx = np.empty((T, k), np.int32)
    rows = np.arange(T)
    for j in range(k):
        masked = np.where(avail, L64, -np.inf)
        best = masked.max(axis=1)
        # lowest index among the maxima of the remaining experts
        is_best = avail & (L64 == best[:, None])
        pick = np.argmax(is_best, axis=1)
        idx[:, j] = pick
        avail[rows, pick] = False
    sel = L64[rows[:, None], idx]
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    return idx, w


def max_blocks(T: int, E: int, k: int, block_rows: int) -> int:
    """Upper bound on the number of row blocks: ceil(T*k/BR) + min(E, T*k)."""
    n = T * k
    return -(-n // block_rows) + min(E, n)


def group(idx: np.ndarray, E: int, block_rows: int = 32) -> dict:
    """Histogram, exclusive scan, stable scatter and block map of the assignments.

    Assignment a = t*k + j goes to expert idx[t, j].
    counts[e]       = number of assignments to e
    offsets         = exclusive prefix sum of counts, length E+1
    sorted_assign   = assignments ordered by expert, ascending a inside an expert
    assign_row[a]   = row of a in that order (inverse permutation)
    block map       = for e ascending, i < ceil(counts[e]/BR): (e, offsets[e] + BR*i);
                      entries past n_blocks are -1
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_assign = np.argsort(flat, kind="stable").astype(np.int32)
    assign_row = np.empty_like(sorted_assign)
    assign_row[sorted_assign] = np.arange(flat.size, dtype=np.int32)
    mb = max_blocks(T, E, k, block_rows)
    block_expert = np.full(mb, -1, np.int32)
    block_row = np.full(mb, -1, np.int32)
    nb = 0
    for e in range(E):
        for i in range(-(-int(counts[e]) // block_rows)):
            block_expert[nb] = e
            block_row[nb] = offsets[e] + block_rows * i
            nb += 1
    return dict(counts=counts, offsets=offsets, sorted_assign=sorted_assign,
                assign_row=assign_row, block_expert=block_expert, block_row=block_row,
                n_blocks=np.int32(nb))


# ----------------------------------------------------------------------------
# Expert FFN and combine
# ----------------------------------------------------------------------------

def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """Router scores ([P1] "Model specification": a router scores the 256
    experts for every token): logits[t, e] = sum_h x[t, h] * W_r[e, h], with
    x bf16 [T, H] and W_r bf16 [E, H] (uint16 bit patterns), in fp64."""
    return bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(wr_bits).T


def shared_gate(x_bits: np.ndarray, wg_bits: np.ndarray) -> np.ndarray:
    """Optional per-token weight of the shared expert, g[t] = sigmoid(x[t] . w_g)
    (w_g bf16 [H]), in fp64.  The pages name no such gate (the shared expert
    sees every token); this is the common sigmoid-gated form, off unless asked."""
    z = bf16_bits_to_f64(x_bits) @ bf16_bits_to_f64(wg_bits)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) in fp64."""
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """(silu(X Wg^T) * (X Wu^T)) Wd^T; W matrices are [N_out, K_in]."""
    G = X @ Wg.T
    U = X @ Wu.T
    return (silu(G) * U) @ Wd.T


def _mat(m, e: int):
    return dequant(m.codes[e], m.scales[e], m.biases[e])


def moe_layer(x_bits: np.ndarray, logits: np.ndarray, gate, up, down, k: int,
              sh_gate=None, sh_up=None, sh_down=None, block_rows: int = 32,
              shared_w=None) -> dict:
    """One layer call over T tokens.

    x_bits: uint16 [T, H] bf16 activations; logits: float32 [T, E].
    gate/up: objects with .codes [E, I, H/8], .scales/.biases [E, I, H/64];
    down: .codes [E, H, I/8], .scales/.biases [E, H, I/64]; shared matrices
    likewise with one expert.
    shared_w: optional fp64 [T] weight of the shared expert per token (default 1).
    Returns dict with routing arrays, topk_w, expert_out (fp64 [T*k, H],
    sorted-row order, unweighted), shared_out (fp64 [T, H], unweighted) and
    y (fp64 [T, H]).
    """
    x = bf16_bits_to_f64(x_bits)
    T, H = x.shape
    E = logits.shape[1]
    idx, w = route_topk(logits, k)
    g = group(idx, E, block_rows)
    expert_out = np.zeros((T * k, H))
    for e in range(E):
        lo, hi = int(g["offsets"][e]), int(g["offsets"][e + 1])
        if hi == lo:
            continue
        tokens = g["sorted_assign"][lo:hi] // k
        expert_out[lo:hi] = swiglu_ffn(x[tokens], _mat(gate, e), _mat(up, e), _mat(down, e))
    shared_out = np.zeros((T, H))
    if sh_gate is not None:
        shared_out = swiglu_ffn(x, _mat(sh_gate, 0), _mat(sh_up, 0), _mat(sh_down, 0))
    y = np.zeros((T, H))
    for j in range(k):
        y += w[:, j:j + 1] * expert_out[g["assign_row"][np.arange(T) * k + j]]
    y += shared_out if shared_w is None else np.asarray(shared_w)[:, None] * shared_out
    out = dict(topk_idx=idx, topk_w=w, expert_out=expert_out, shared_out=shared_out, y=y)
    out.update(g)
    return out


def moe_layer_chunked(x_bits, logits, gate, up, down, k, sh_gate=None, sh_up=None,
                      sh_down=None, chunk: int = 2048, block_rows: int = 32):
    """Bounded chunks: independent layer calls over consecutive token ranges.

    Returns (y fp64 [T, H], list of per-chunk result dicts)."""
    T = x_bits.shape[0]
    parts, ys = [], []
    for t0 in range(0, T, chunk):
        r = moe_layer(x_bits[t0:t0 + chunk], logits[t0:t0 + chunk], gate, up, down, k,
                      sh_gate, sh_up, sh_down, block_rows)
        parts.append(r)
        ys.append(r["y"])
    return np.concatenate(ys, axis=0), parts
