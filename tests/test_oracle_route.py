"""Pins of the oracle's routing (runs on CPU).

P-rt1: top-k equals a full sort with key (-logit, expert) on every token of
every workload, plus hand-derived tie cases.  Softmax weights pinned by the
two-expert logistic identity, the full-softmax renormalisation (scipy), and
ratio / shift invariants.  P-rt2: grouping invariants on every workload.
P-rt3: special cases and hand-derived grouping fixtures.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from conftest import golden_lines
from workload import CONFIGS, make_activations


def _parse_f32(tok):
    return np.float32(float(tok))


def test_topk_tie_fixture():
    for ln in golden_lines("topk_ties.txt"):
        k_s, logit_s, want_s = [p.strip() for p in ln.split("|")]
        L = np.array([[_parse_f32(t) for t in logit_s.split()]], np.float32)
        idx, w = oracle.route_topk(L, int(k_s))
        assert idx[0].tolist() == [int(t) for t in want_s.split()], ln


def _full_sort_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_topk_equals_full_sort_all_configs(name):
    cfg = CONFIGS[name]
    _, logits = make_activations(cfg)
    # every token for the prefill configs; a stride through the larger ones keeps this quick
    step = 1 if cfg.T <= 2048 else 3
    L = logits[::step]
    idx, _ = oracle.route_topk(L, cfg.k)
    for t in range(L.shape[0]):
        assert idx[t].tolist() == _full_sort_topk(L[t], cfg.k)


def test_weights_two_experts_logistic():
    rng = np.random.default_rng(5)
    L = rng.standard_normal((200, 10)).astype(np.float32)
    idx, w = oracle.route_topk(L, 2)
    for t in range(200):
        d = float(L[t, idx[t, 1]]) - float(L[t, idx[t, 0]])
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(d))) < 1e-15
        assert abs(w[t, 1] - 1.0 / (1.0 + math.exp(-d))) < 1e-15


def test_weights_equal_renormalised_full_softmax():
    _, logits = make_activations(CONFIGS["prefill512"])
    idx, w = oracle.route_topk(logits, 8)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    psel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    ref = psel / psel.sum(axis=1, keepdims=True)
    assert np.max(np.abs(ref - w)) < 1e-12
    assert np.all(w > 0)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-12
    # weights follow the selection order (non-increasing)
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_weights_invariants():
    rng = np.random.default_rng(7)
    L = rng.integers(-8, 8, (50, 32)).astype(np.float32) / np.float32(4)
    idx, w = oracle.route_topk(L, 4)
    idx2, w2 = oracle.route_topk(L + np.float32(1.0), 4)   # exact shift
    assert np.array_equal(idx, idx2)
    assert np.max(np.abs(w - w2)) < 1e-14
    for t in range(50):
        for a in range(4):
            for b in range(4):
                r = math.exp(float(L[t, idx[t, a]]) - float(L[t, idx[t, b]]))
                assert abs(w[t, a] / w[t, b] - r) < 1e-12 * max(1.0, r)


def test_equal_logits_and_k_equals_E():
    L = np.zeros((3, 16), np.float32)
    idx, w = oracle.route_topk(L, 5)
    assert idx.tolist() == [[0, 1, 2, 3, 4]] * 3
    assert np.allclose(w, 0.2, atol=1e-15, rtol=0)
    rng = np.random.default_rng(1)
    L = rng.standard_normal((4, 16)).astype(np.float32)
    idx, w = oracle.route_topk(L, 16)
    for t in range(4):
        assert idx[t].tolist() == list(np.argsort(-L[t], kind="stable"))
    g = oracle.group(idx, 16, 32)
    assert g["counts"].tolist() == [4] * 16


def _check_group_invariants(idx, E, br, g):
    T, k = idx.shape
    n = T * k
    counts, offsets = g["counts"], g["offsets"]
    sa, ar = g["sorted_assign"], g["assign_row"]
    assert counts.sum() == n
    assert offsets[0] == 0 and offsets[-1] == n
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(sa), np.arange(n))
    assert np.array_equal(ar[sa], np.arange(n))
    # every token exactly k times
    assert np.array_equal(np.bincount(sa // k, minlength=T), np.full(T, k))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = sa[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    nb = int(g["n_blocks"])
    assert nb == sum(-(-int(c) // br) for c in counts)
    be, brw = g["block_expert"], g["block_row"]
    covered = np.zeros(n, np.int32)
    for b in range(nb):
        e = be[b]
        r0 = brw[b]
        r1 = min(r0 + br, offsets[e + 1])
        assert offsets[e] <= r0 < offsets[e + 1]
        covered[r0:r1] += 1
        if b > 0:
            assert (be[b - 1], brw[b - 1]) < (e, r0)
    assert np.all(covered == 1)
    assert np.all(be[nb:] == -1) and np.all(brw[nb:] == -1)
    assert len(be) == oracle.max_blocks(T, E, k, br)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_group_invariants_all_configs(name):
    cfg = CONFIGS[name]
    _, logits = make_activations(cfg)
    T = cfg.call_tokens
    # first call of each workload (first chunk / first decode token), plus a second
    for t0 in (0, T if cfg.T >= 2 * T else 0):
        L = logits[t0:t0 + T]
        idx, _ = oracle.route_topk(L, cfg.k)
        for br in (16, 32, 64):
            _check_group_invariants(idx, cfg.E, br, oracle.group(idx, cfg.E, br))


def test_decode_token_gives_k_one_row_blocks():
    _, logits = make_activations(CONFIGS["decode"])
    idx, _ = oracle.route_topk(logits[:1], 8)
    g = oracle.group(idx, 256, 32)
    assert int(g["n_blocks"]) == 8
    assert g["block_row"][:8].tolist() == list(range(8))
    assert g["block_expert"][:8].tolist() == sorted(idx[0].tolist())


def _kv(lines):
    out = {}
    for ln in lines:
        key, *vals = ln.split()
        out[key] = [int(v) for v in vals]
    return out


def test_grouping_fixture():
    f = _kv(golden_lines("grouping.txt"))
    idx = np.array(f["idx"], np.int32).reshape(4, 2)
    g = oracle.group(idx, 3, 2)
    for key in ("counts", "offsets", "sorted_assign", "assign_row", "block_expert", "block_row"):
        assert g[key].tolist() == f[key], key
    assert int(g["n_blocks"]) == f["n_blocks"][0]


def test_block_map_counts_fixture():
    f = _kv(golden_lines("block_map_counts.txt"))
    counts = f["counts"]
    rng = np.random.default_rng(0)
    flat = np.repeat(np.arange(len(counts)), counts)
    rng.shuffle(flat)
    idx = flat.reshape(-1, 1).astype(np.int32)          # k = 1
    g = oracle.group(idx, len(counts), 32)
    assert g["counts"].tolist() == counts
    assert g["offsets"].tolist() == f["offsets"]
    assert g["block_expert"].tolist() == f["block_expert"]
    assert g["block_row"].tolist() == f["block_row"]
    assert int(g["n_blocks"]) == f["n_blocks"][0]
