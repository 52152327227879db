"""Pins of the oracle's dequantization (runs on CPU).

P-dq1/P-dq2: hand-worked groups, including bf16 ties that separate
round-to-nearest-even from truncation and from round-half-away.
P-dq3: nibble order.  P-dq4: storage format size.
Exact-rational brute force: q*s+b rounded to fp32 then to bf16 by a slow
Fraction-based rounding written here, on random groups.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import golden_lines
from workload import pack_nibbles


def test_hand_worked_groups():
    rows = [ln.split() for ln in golden_lines("dequant_groups.txt")]
    assert len(rows) >= 20
    for s_hex, b_hex, q, w_hex in rows:
        codes = np.zeros((1, 8), np.uint32)   # one row of 64 weights
        qs = np.zeros(64, np.uint8)
        qs[5] = int(q)
        codes[0] = pack_nibbles(qs[None, :])[0]
        s = np.array([[int(s_hex, 16)]], np.uint16)
        b = np.array([[int(b_hex, 16)]], np.uint16)
        w = oracle.dequant_bf16_bits(codes, s, b)
        assert w.shape == (1, 64)
        assert int(w[0, 5]) == int(w_hex, 16), (s_hex, b_hex, q, hex(int(w[0, 5])))


def test_rne_tie_breaks_distinguish_modes():
    # fp32 0x3d8f8000 is a bf16 tie: nearest-even gives 0x3d90 (truncation 0x3d8f).
    v = np.array([0x3D8F8000, 0xBCFA8000, 0xBC7A8000, 0x3F808000, 0x3F818000], np.uint32).view(np.float32)
    got = oracle.f32_to_bf16_rne_bits(v)
    assert [hex(int(g)) for g in got] == ["0x3d90", "0xbcfa", "0xbc7a", "0x3f80", "0x3f82"]


def test_nibble_order():
    for ln in golden_lines("nibble_order.txt"):
        parts = ln.split()
        word = int(parts[0], 16)
        want = [int(p) for p in parts[1:]]
        got = oracle.unpack_codes(np.array([word], np.uint32))
        assert got.tolist() == want


def test_storage_format_bytes_per_weight():
    # 4-bit code + one bf16 scale + one bf16 bias per 64 weights = 4.5 bits.
    # The pages' checkpoint: 19.4 GB at 4 bit vs 70 GB at bf16 (ratio 0.277 vs 4.5/16 = 0.281).
    bits = 4 + 2 * 16 / 64
    assert bits == 4.5
    assert abs(19.4 / 70 - bits / 16) < 0.005
    # per expert at H=2048, I=512: gate+up [512, 2048] and down [2048, 512]
    n_w = 3 * 512 * 2048
    assert n_w * bits / 8 == 1_769_472


def _round_to_format(v: Fraction, mant_bits: int) -> Fraction:
    """Nearest value with `mant_bits` fraction bits of significand (normal range), ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - mant_bits)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def _bf16_bits_to_fraction(bits: int) -> Fraction:
    f = np.array([bits << 16], np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def test_exact_rational_brute_force():
    rng = np.random.default_rng(123)
    n_rows, K = 6, 128
    q = rng.integers(0, 16, (n_rows, K), dtype=np.uint8)
    # scales and biases over several binades, not tied to -8*s, so rounding ties and
    # non-ties both occur
    s_f = (rng.uniform(0.5, 2.0, (n_rows, 2)) * 2.0 ** rng.integers(-12, 2, (n_rows, 2))).astype(np.float32)
    b_f = (rng.uniform(-2.0, 2.0, (n_rows, 2)) * 2.0 ** rng.integers(-10, 1, (n_rows, 2))).astype(np.float32)
    # truncate to bf16 patterns (any pattern is a valid input)
    s_bits = (s_f.view(np.uint32) >> 16).astype(np.uint16)
    b_bits = (b_f.view(np.uint32) >> 16).astype(np.uint16)
    got = oracle.dequant_bf16_bits(pack_nibbles(q), s_bits, b_bits)
    for n in range(n_rows):
        for kk in range(K):
            s = _bf16_bits_to_fraction(int(s_bits[n, kk // 64]))
            b = _bf16_bits_to_fraction(int(b_bits[n, kk // 64]))
            exact = int(q[n, kk]) * s + b
            v32 = _round_to_format(exact, 23)
            v16 = _round_to_format(v32, 7)
            assert _bf16_bits_to_fraction(int(got[n, kk])) == v16, (n, kk)


def test_group_axis_is_k_within_output_row():
    # Scales differ per (row, group): W[n, k] must use scales[n, k // 64].
    N, K = 3, 192
    q = np.full((N, K), 9, np.uint8)            # (q - 8) = 1 -> w = s exactly
    s_bits = np.zeros((N, K // 64), np.uint16)
    for n in range(N):
        for g in range(K // 64):
            s_bits[n, g] = 0x3F80 + ((n * 3 + g) << 7)   # 2^(n*3+g): exact powers of two
    b_bits = (s_bits | 0x8000) + (3 << 7)            # -8 * s
    w = oracle.dequant(pack_nibbles(q), s_bits, b_bits)
    for n in range(N):
        for kk in range(K):
            assert w[n, kk] == 2.0 ** (n * 3 + kk // 64)
