"""Pins for the oracle's W4A8-FP8 form (CPU only).

* The E4M3 values: every one of the 256 codes against a table built
  independently from the format's description (subnormals m * 2^-9, normals
  (8 + m) * 2^(e - 10), largest finite 448, 0x7F / 0xFF NaN);
* encoding: every finite code round-trips; every midpoint between
  neighbours goes to the even code; random reals go to the nearest table
  entry (brute force over the table);
* the activation quantiser: each row's largest magnitude becomes +-448,
  zero rows give codes 0 and scale 0, scaling a row by a power of two keeps
  its codes and scales sx by the same power, the dequantised activations are
  within half a step of the inputs;
* the layer: exact rational brute force on tiny shapes, and agreement with
  the (separately pinned) W4A16 oracle to within the activations' rounding;
* planted mistakes (ties away from zero, truncation, exponent bias 8, the
  240 maximum of the other E4M3 variant, one scale for the whole tensor, the
  row scale dropped) each fail one of these pins.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import w4a8_oracle as w8


def _table():
    """Positive finite E4M3 values by code (0..126), from the format's description."""
    vals = {}
    for m in range(8):
        vals[m] = Fraction(m, 512)                       # exponent field 0: m * 2^-9
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                  # NaN
            vals[(e << 3) | m] = Fraction(8 + m, 1) * Fraction(2) ** (e - 10)
    return vals


TABLE = _table()


class _Impl:
    """The oracle functions under test (a planted mistake swaps some)."""
    value = staticmethod(w8.fp8_e4m3_value)
    encode = staticmethod(w8.fp8_e4m3_encode)
    quantize = staticmethod(w8.quantize_act_fp8)
    linear = staticmethod(w8.linear_w4a8_64)


def pin_values(impl):
    codes = np.arange(256, dtype=np.uint8)
    v = impl.value(codes)
    for c, f in TABLE.items():
        assert v[c] == float(f), c
        assert v[c | 0x80] == -float(f), c
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x7E] == 448.0


def pin_encode_round_trip_and_ties(impl):
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = impl.value(np.array(finite, np.uint8))
    assert np.array_equal(impl.encode(vals), np.array(finite, np.uint8))
    pos = sorted(TABLE.items(), key=lambda kv: kv[1])
    for (ca, a), (cb, b) in zip(pos, pos[1:]):
        mid = float((a + b) / 2)
        even = ca if ca % 2 == 0 else cb
        assert impl.encode(np.array([mid]))[0] == even, (ca, cb)
        assert impl.encode(np.array([-mid]))[0] == even | 0x80
        eps = float(b - a) / 64
        assert impl.encode(np.array([mid - eps]))[0] == ca
        assert impl.encode(np.array([mid + eps]))[0] == cb


def pin_encode_nearest(impl):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-460, 460, 4000), rng.uniform(-0.05, 0.05, 4000),
                        np.exp(rng.uniform(-12, 6, 2000)) * rng.choice([-1, 1], 2000)])
    grid = np.array(sorted(float(f) for f in TABLE.values()))
    codes = impl.encode(x)
    got = impl.value(codes)
    best = grid[np.argmin(np.abs(grid[None, :] - np.abs(x)[:, None]), axis=1)] * np.sign(x)
    assert np.array_equal(np.abs(got - x), np.abs(best - x))


def pin_quantizer(impl):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((6, 256)) * rng.uniform(0.01, 20, (6, 1))).astype(np.float16)
    x[3] = 0
    x[4, :] = np.float16(0.0)
    x[4, 17] = np.float16(-3.0)                        # one non-zero element
    codes, sx = impl.quantize(x)
    assert codes.dtype == np.uint8 and sx.dtype == np.float32
    for m in range(6):
        amax = np.max(np.abs(x[m].astype(np.float32)))
        if amax == 0:
            assert np.all(codes[m] == 0) and sx[m] == 0
            continue
        k = int(np.argmax(np.abs(x[m].astype(np.float32))))
        assert impl.value(codes[m, k:k + 1])[0] == np.sign(float(x[m, k])) * 448.0
        assert sx[m] == np.float32(amax / np.float32(448.0))
        xhat = impl.value(codes[m]) * float(sx[m])
        # half a step: 2^-4 relative for normal codes, 2^-10 of the scale below 2^-6
        bound = np.maximum(np.abs(x[m].astype(np.float64)) * 2.0 ** -4, 2.0 ** -10 * float(sx[m])) * 1.0001
        assert np.all(np.abs(xhat - x[m].astype(np.float64)) <= bound), m
    # a power of two on a row: same codes, scale times that power
    x2 = (x.astype(np.float32) * 8).astype(np.float16)
    c2, s2 = impl.quantize(x2)
    assert np.array_equal(c2, codes) and np.array_equal(s2, (sx * 8).astype(np.float32))


def pin_linear_bruteforce(impl):
    rng = np.random.default_rng(3)
    M, K, N, G = 2, 256, 8, 128
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    z = rng.integers(0, 16, (K // G, N)).astype(np.uint8)
    s = rng.uniform(0.001, 0.02, (K // G, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    codes, sx = impl.quantize(x)
    y = impl.linear(codes, sx, q, z, s, G)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for g in range(K // G):
                part = Fraction(0)
                for k in range(g * G, (g + 1) * G):
                    part += TABLE[int(codes[m, k]) & 0x7F] * (-1 if codes[m, k] & 0x80 else 1) * \
                        (int(q[k, n]) - int(z[g, n]))
                acc += Fraction(float(s[g, n])) * part
            want = acc * Fraction(float(sx[m]))
            assert abs(Fraction(float(y[m, n])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def pin_close_to_w4a16(impl):
    # The W4A8 layer differs from the W4A16 one only by the activations'
    # rounding: within 2^-4 (plus the subnormal half step) of the L1 scale.
    K, N, G = 512, 48, 128
    q, z, s = synth.layer(K, N, G, seed=4)
    x = synth.activations(5, K, seed=4)
    codes, sx = impl.quantize(x)
    y8 = impl.linear(codes, sx, q, z, s, G)
    y16 = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    absw = np.abs(oracle.dequant64(q, z, s, G))
    sub = (2.0 ** -10 * sx.astype(np.float64))[:, None] * absw.sum(axis=0)[None, :]
    assert np.all(np.abs(y8 - y16) <= 2.0 ** -4 * D * 1.0001 + sub)
    # and it is not the W4A16 result itself (the activations were rounded)
    assert np.max(np.abs(y8 - y16)) > 1e-4 * np.max(np.abs(y16))


PINS = [pin_values, pin_encode_round_trip_and_ties, pin_encode_nearest, pin_quantizer, pin_linear_bruteforce,
        pin_close_to_w4a16]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_w4a8(pin):
    pin(_Impl)


def test_error_scale_is_the_l1_sum():
    rng = np.random.default_rng(5)
    K, N, G = 256, 16, 128
    q, z, s = synth.layer(K, N, G, seed=5)
    codes = rng.integers(0, 256, (3, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x01
    sx = np.array([0.5, 1.0, 0.0], np.float32)
    D = w8.w4a8_l1_scale(codes, sx, q, z, s, G)
    xv = np.abs(w8.fp8_e4m3_value(codes) * sx[:, None].astype(np.float64))
    for m in range(3):
        for n in (0, 7, 15):
            want = sum(xv[m, k] * abs((int(q[k, n]) - int(z[k // G, n])) * float(s[k // G, n])) for k in range(K))
            assert abs(D[m, n] - want) <= 1e-12 * max(1.0, want)
    assert np.all(D[2] == 0)


# ---- planted mistakes ---------------------------------------------------------

def _encode_variant(ties_away=False, trunc=False, bias=7):
    def enc(v):
        v = np.asarray(v, np.float64)
        out = []
        for t in v:
            a = abs(t)
            best, bc = None, 0
            cands = []
            for c, f in TABLE.items():
                val = float(f) * 2.0 ** (7 - bias)
                cands.append((val, c))
            cands.sort()
            if trunc:
                lower = [c for val, c in cands if val <= a]
                bc = lower[-1] if lower else 0
            else:
                d = [(abs(val - a), c, val) for val, c in cands]
                md = min(x[0] for x in d)
                ties = [x for x in d if x[0] == md]
                if len(ties) > 1:
                    bc = max(ties, key=lambda x: x[2])[1] if ties_away else [x for x in ties if x[1] % 2 == 0][0][1]
                else:
                    bc = ties[0][1]
            out.append(bc | (0x80 if np.signbit(t) else 0))
        return np.array(out, np.uint8)
    return enc


def _value_bias8(code):
    return w8.fp8_e4m3_value(code) / 2.0


def _quantize_variant(maxv=448.0, per_tensor=False):
    def quant(x):
        x32 = np.asarray(x, np.float16).astype(np.float32)
        amax_rows = np.max(np.abs(x32), axis=1)
        codes = np.zeros(x32.shape, np.uint8)
        sx = np.zeros(x32.shape[0], np.float32)
        for m in range(x32.shape[0]):
            amax = np.max(amax_rows) if per_tensor else amax_rows[m]
            if amax == 0:
                continue
            inv = np.float32(maxv) / amax
            codes[m] = w8.fp8_e4m3_encode((x32[m] * inv).astype(np.float32).astype(np.float64))
            sx[m] = amax / np.float32(maxv)
        return codes, sx
    return quant


def _linear_no_rowscale(codes, sx, q, z, s, G):
    return w8.fp8_e4m3_value(codes) @ oracle.dequant64(q, z, s, G)


def _mutant(**fns):
    return type("M", (_Impl,), {k: staticmethod(v) for k, v in fns.items()})


MUTANTS = {
    "ties_away_from_zero": _mutant(encode=_encode_variant(ties_away=True)),
    "truncation": _mutant(encode=_encode_variant(trunc=True)),
    "exponent_bias_8": _mutant(value=_value_bias8),
    "max_240": _mutant(quantize=_quantize_variant(maxv=240.0)),
    "one_scale_per_tensor": _mutant(quantize=_quantize_variant(per_tensor=True)),
    "row_scale_dropped": _mutant(linear=_linear_no_rowscale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, ValueError, KeyError, IndexError):
            failed += 1
    assert failed >= 1, name
