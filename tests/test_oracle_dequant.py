"""Pins for the oracle's dequantisation (CPU only).

The fp16 dequantised weight is read as round-to-nearest-even of the exact
product (q - z) * s. The oracle gets it from float64 arithmetic and numpy's
float16 cast; here it is checked over the whole input domain (31 code
differences x all 65 536 fp16 scale bit patterns) against an independent
integer implementation of IEEE 754 binary16 rounding, and on samples and all
ties against exact rationals.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _fp16_fields(bits):
    bits = np.asarray(bits, dtype=np.int64)
    return (bits >> 15) & 1, (bits >> 10) & 0x1F, bits & 0x3FF


def _bit_length(a):
    a = np.asarray(a, dtype=np.int64)
    out = np.zeros(a.shape, dtype=np.int64)
    for b in range(63):
        out += (a >= (np.int64(1) << b)).astype(np.int64)
    return out


def int_rne_product(d, s_bits):
    """binary16 bits of RNE(d * s) for integer d and fp16 bit pattern s,
    by integer arithmetic only. NaN results are returned as 0x7E00."""
    d = np.asarray(d, dtype=np.int64)
    sign_s, exp_s, frac_s = _fp16_fields(s_bits)
    d, sign_s, exp_s, frac_s = np.broadcast_arrays(d, sign_s, exp_s, frac_s)
    # s = (-1)^sign * m * 2^e
    normal = exp_s > 0
    m = np.where(normal, frac_s + 1024, frac_s)
    e = np.where(normal, exp_s - 25, -24)
    P = np.abs(d) * m
    neg = (d < 0).astype(np.int64) ^ sign_s
    out = np.zeros(d.shape, dtype=np.int64)

    special = exp_s == 31
    nan_in = special & (frac_s != 0)
    inf_in = special & (frac_s == 0)

    nb = _bit_length(P)
    ulp = np.maximum(nb - 1 + e - 10, -24)
    sh = ulp - e  # bits to drop (<= 0 means exact)
    R = np.where(sh <= 0, P << np.maximum(-sh, 0), 0)
    shp = np.maximum(sh, 0)
    q = P >> shp
    rem = P - (q << shp)
    half = np.where(shp > 0, np.int64(1) << np.maximum(shp - 1, 0), 0)
    up = (shp > 0) & ((rem > half) | ((rem == half) & (q & 1 == 1)))
    R = np.where(sh > 0, q + up.astype(np.int64), R)
    # normalise carry into the next binade
    carry = R >= 2048
    R = np.where(carry, R >> 1, R)
    ulp = np.where(carry, ulp + 1, ulp)
    sub = (ulp == -24) & (R < 1024)
    E = ulp + 25
    enc = np.where(sub, R, (E << 10) | (R - 1024))
    enc = np.where(~sub & (E >= 31), 0x7C00, enc)
    enc = np.where(P == 0, 0, enc)
    out = enc | (neg << 15)
    # d == 0 gives +0 from the subtraction; +0 * s carries s's sign.
    out = np.where((d == 0) & ~special, sign_s << 15, out)
    out = np.where(inf_in & (d != 0), 0x7C00 | (neg << 15), out)
    out = np.where(inf_in & (d == 0), 0x7E00, out)
    out = np.where(nan_in, 0x7E00, out)
    return out.astype(np.int64)


def _oracle_bits(d, s_bits):
    """Run the oracle on a layout that realises code difference d per row."""
    d = np.asarray(d, dtype=np.int64)
    s_bits = np.asarray(s_bits, dtype=np.uint16)
    # K = 1 group of G = 1 row is not allowed (G >= 1 fine for the oracle);
    # use q = max(d, 0), z = max(-d, 0) so q - z = d with 0 <= q, z <= 15.
    q = np.maximum(d, 0).astype(np.uint8).reshape(1, -1)
    z = np.maximum(-d, 0).astype(np.uint8).reshape(1, -1)
    s = s_bits.view(np.float16).reshape(1, -1)
    w = oracle.dequant16(q, z, s, 1)
    return w.view(np.uint16).astype(np.int64).reshape(-1)


def _is_nan_bits(b):
    b = np.asarray(b)
    return ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)


def test_full_domain_against_integer_rounding():
    s_all = np.arange(65536, dtype=np.int64)
    for d in range(-15, 16):
        ref = int_rne_product(np.full(65536, d), s_all)
        got = _oracle_bits(np.full(65536, d), s_all)
        nan_ref = _is_nan_bits(ref)
        nan_got = _is_nan_bits(got)
        assert np.array_equal(nan_ref, nan_got), d
        assert np.array_equal(ref[~nan_ref], got[~nan_got]), d


def _frac_round16(value: Fraction) -> int:
    """Reference binary16 RNE of an exact rational (finite inputs)."""
    if value == 0:
        return 0
    neg = value < 0
    a = -value if neg else value
    # candidates: enumerate neighbouring fp16 values by bisection over bits
    lo, hi = 0, 0x7C00  # non-negative fp16 patterns are ordered
    def val(b):
        if b == 0x7C00:
            return None
        ex, fr = b >> 10, b & 0x3FF
        return Fraction(fr, 1 << 24) if ex == 0 else Fraction(1024 + fr, 1 << 10) * Fraction(2) ** (ex - 15)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if val(mid) <= a:
            lo = mid
        else:
            hi = mid
    vlo = val(lo)
    vhi = val(hi) if hi != 0x7C00 else Fraction(65536)  # 2^16 = overflow threshold step
    if a - vlo < vhi - a:
        b = lo
    elif a - vlo > vhi - a:
        b = hi
    else:
        b = lo if lo % 2 == 0 else hi
    return b | (0x8000 if neg else 0)


def test_sample_and_ties_against_fractions():
    rng = np.random.default_rng(7)
    d = rng.integers(-15, 16, size=20000)
    s = rng.integers(0, 0x7C00, size=20000) | (rng.integers(0, 2, size=20000) << 15)
    got = _oracle_bits(d, s)
    for di, si, gi in zip(d[:4000], s[:4000], got[:4000]):
        if di == 0:
            continue
        sv = float(np.uint16(si).view(np.float16))
        ref = _frac_round16(Fraction(int(di)) * Fraction(sv))
        assert ref == gi, (di, hex(si), hex(gi), hex(ref))
    # all exact ties: the product lies halfway between two fp16 values
    ties = 0
    s_all = np.arange(0x7C00, dtype=np.int64)
    for di in range(1, 16):
        sign_s, exp_s, frac_s = _fp16_fields(s_all)
        m = np.where(exp_s > 0, frac_s + 1024, frac_s)
        P = di * m
        nb = _bit_length(P)
        e = np.where(exp_s > 0, exp_s - 25, -24)
        sh = np.maximum(nb - 1 + e - 10, -24) - e
        tie_mask = (sh > 0) & ((P & ((np.int64(1) << np.maximum(sh, 1)) - 1)) == (np.int64(1) << np.maximum(sh - 1, 0)))
        idx = np.nonzero(tie_mask)[0]
        got = _oracle_bits(np.full(idx.size, di), s_all[idx])
        for si, gi in zip(s_all[idx][::7], got[::7]):
            sv = float(np.uint16(si).view(np.float16))
            assert _frac_round16(Fraction(di) * Fraction(sv)) == gi
            ties += 1
    assert ties > 1000


def test_power_of_two_scales_are_exact():
    # s = 2^-e makes (q - z) * s exactly representable: no rounding at all.
    for e in range(0, 14):
        s = np.full((1, 16), 2.0 ** -e, dtype=np.float16)
        q = np.arange(16, dtype=np.uint8).reshape(1, 16)
        z = np.full((1, 16), 7, np.uint8)
        w = oracle.dequant16(q, z, s, 1).astype(np.float64)
        assert np.array_equal(w[0], (np.arange(16) - 7) * 2.0 ** -e)


def test_signed_zero_and_specials():
    q = np.array([[3, 3, 3, 0]], np.uint8)
    z = np.array([[3, 3, 3, 0]], np.uint8)
    s = np.array([[-0.5, 0.5, np.inf, np.nan]], np.float16)
    w = oracle.dequant16(q, z, s, 1)
    bits = w.view(np.uint16)[0]
    assert bits[0] == 0x8000 and bits[1] == 0x0000
    assert np.isnan(w[0, 2]) and np.isnan(w[0, 3])


def test_groups_index_rows():
    # Row k uses group k // G: a scale per group that is a distinct power of
    # two reveals the mapping.
    K, N, G = 256, 8, 64
    q = np.full((K, N), 9, np.uint8)
    z = np.full((K // G, N), 8, np.uint8)
    s = (2.0 ** -np.arange(K // G)).astype(np.float16)[:, None] * np.ones((1, N), np.float16)
    w = oracle.dequant64(q, z, s, G)
    for k in range(K):
        assert np.all(w[k] == 2.0 ** -(k // G))
    with pytest.raises(ValueError):
        oracle.dequant64(q, z, s, 96)
