"""Pins for the oracle's round-to-nearest group quantiser (CPU only).

The pages name the method (round-to-nearest, "RTN"; 4-bit codes in groups of
128 input channels) but print no formula; the oracle takes the asymmetric
min-max reading. It is pinned here by facts that do not depend on its code:

* weights that lie exactly on a grid (q0 - z0) * s0 with a power-of-two s0,
  with codes 0 and 15 present in every group, come back as exactly q0, z0, s0;
* on random groups that contain 0, every dequantised weight is within s/2 of
  the input (plus the fp16 rounding of s): the codes are the nearest grid
  points;
* quotients that fall exactly half-way between two codes round to the even
  one;
* constant groups (range 0) take the scale 1 and reproduce integer values;
* plausible mistakes (floor for rounding, 16 levels for 15, zero point with
  the wrong sign, zero point dropped, groups taken along the wrong axis,
  halves rounded away from zero) planted in copies of the quantiser each
  fail one of these pins.
"""
import numpy as np
import pytest

import oracle
import synth


def _exact_grid_case(K, N, G, seed):
    """Codes with 0 and 15 in every (group, column), z0 in 0..15, s0 = 2^-e."""
    rng = np.random.default_rng(seed)
    q0 = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
    for g in range(K // G):
        rows = rng.permutation(G)[:2] + g * G
        q0[rows[0], :] = 0
        q0[rows[1], :] = 15
    z0 = rng.integers(0, 16, size=(K // G, N)).astype(np.uint8)
    e = rng.integers(4, 12, size=(K // G, N))
    s0 = np.ldexp(1.0, -e).astype(np.float16)
    w = oracle.dequant64(q0, z0, s0, G)
    assert np.array_equal(w.astype(np.float16).astype(np.float64), w)  # exact in fp16
    return w.astype(np.float16), q0, z0, s0


def check_exact_grid(quantize):
    for K, N, G in [(128, 16, 32), (256, 24, 64), (256, 8, 128), (512, 16, 256)]:
        w, q0, z0, s0 = _exact_grid_case(K, N, G, seed=K + N + G)
        q, z, s = quantize(w, G)
        assert np.array_equal(q, q0) and np.array_equal(z, z0)
        assert np.array_equal(s.view(np.uint16), s0.view(np.uint16))


def check_error_bound(quantize):
    for K, N, G in [(256, 32, 32), (256, 32, 64), (512, 48, 128), (512, 16, 256)]:
        w = synth.dense_weights(K, N, seed=K * 7 + G)
        wg = w.astype(np.float64).reshape(K // G, G, N)
        assert np.all(wg.min(axis=1) <= 0) and np.all(wg.max(axis=1) >= 0)
        q, z, s = quantize(w, G)
        assert q.dtype == np.uint8 and q.max() <= 15 and z.max() <= 15
        wd = oracle.dequant64(q, z, s, G)
        srow = np.repeat(s.astype(np.float64), G, axis=0)
        # nearest grid point: s/2, plus at most 15 * 2^-11 * s from the fp16
        # rounding of s at the top of the range, plus float32 quotient rounding
        assert np.max(np.abs(wd - w.astype(np.float64)) / srow) <= 0.5 + 15 * 2.0 ** -11 + 1e-6
        # the range is covered: the scale is no smaller than needed
        rng = (wg.max(axis=1) - wg.min(axis=1)) / 15
        assert np.all(s.astype(np.float64) >= rng * (1 - 2.0 ** -11))


def check_half_way_rounds_to_even(quantize):
    G, N = 32, 4
    s0 = 2.0 ** -6
    z0 = np.array([4, 5, 7, 10])
    base = np.tile(np.arange(16, dtype=np.float64)[:, None], (2, 1))[:G]   # codes 0..15 twice
    w = (base - z0[None, :]) * s0
    # row 3: code 2.5 (between 2 and 3); row 5: code 3.5 (between 3 and 4)
    w[3, :] = (2.5 - z0) * s0
    w[5, :] = (3.5 - z0) * s0
    w16 = w.astype(np.float16)
    assert np.array_equal(w16.astype(np.float64), w)
    q, z, s = quantize(w16, G)
    assert np.array_equal(z[0], z0) and float(s[0, 0]) == s0
    # w/s - z0 is x.5 with x = 2 - z0 or 3 - z0; ties to even in the quotient
    for n in range(N):
        for row, c in ((3, 2.5), (5, 3.5)):
            t = c - z0[n]
            want = np.rint(t) + z0[n]            # numpy rint is round-half-even
            assert np.rint(t) % 2 == 0
            assert q[row, n] == want


def check_constant_groups(quantize):
    G = 64
    w = np.zeros((2 * G, 8), dtype=np.float16)
    w[:G, 1] = 3.0
    w[:G, 2] = -2.0
    w[G:, 3] = 7.0
    q, z, s = quantize(w, G)
    assert np.all(s == np.float16(1.0))
    wd = oracle.dequant64(q, z, s, G)
    assert np.array_equal(wd, w.astype(np.float64))


PINS = [check_exact_grid, check_error_bound, check_half_way_rounds_to_even, check_constant_groups]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_quantiser(pin):
    pin(oracle.quantize_rtn)


def test_quantise_then_dequant_round_trip_of_codes():
    # quantising the oracle's own dequantised weights returns the same codes
    # when the grid is exact (the W4A16 layer then sees the same weights)
    w, q0, z0, s0 = _exact_grid_case(256, 16, 128, seed=5)
    q, z, s = oracle.quantize_rtn(oracle.dequant16(q0, z0, s0, 128), 128)
    assert np.array_equal(oracle.dequant16(q, z, s, 128).view(np.uint16), w.view(np.uint16))


# ---- planted mistakes: each mutant must fail at least one pin ----------------

def _mutant(floor=False, levels=15, zero_sign=1, drop_zero=False, axis_n=False, half_away=False):
    def quantize(w, G):
        w = np.asarray(w, dtype=np.float16)
        K, N = w.shape
        if axis_n:
            wg = w.T.reshape(N // G if N % G == 0 else 1, -1, K).astype(np.float32)
            lo = np.repeat(wg.min(axis=1), 1, axis=0)
            hi = np.repeat(wg.max(axis=1), 1, axis=0)
            lo = np.resize(lo, (K // G, N)).astype(np.float32)
            hi = np.resize(hi, (K // G, N)).astype(np.float32)
            wg = w.reshape(K // G, G, N).astype(np.float32)
        else:
            wg = w.reshape(K // G, G, N).astype(np.float32)
            lo, hi = wg.min(axis=1), wg.max(axis=1)
        s16 = ((hi - lo) / np.float32(levels)).astype(np.float16)
        s16 = np.where(s16 == 0, np.float16(1.0), s16).astype(np.float16)
        sf = s16.astype(np.float32)
        rnd = np.floor if floor else (lambda a: np.sign(a) * np.floor(np.abs(a) + 0.5)) if half_away else np.rint
        z = np.zeros_like(lo) if drop_zero else np.clip(rnd(-zero_sign * lo / sf), 0, 15)
        q = np.clip(rnd(wg / sf[:, None, :]) + z[:, None, :], 0, 15)
        return q.reshape(K, N).astype(np.uint8), z.astype(np.uint8), s16
    return quantize


MUTANTS = {
    "floor": _mutant(floor=True),
    "sixteen_levels": _mutant(levels=16),
    "zero_sign": _mutant(zero_sign=-1),
    "drop_zero": _mutant(drop_zero=True),
    "groups_along_n": _mutant(axis_n=True),
    "half_away_from_zero": _mutant(half_away=True),
}


def test_unmutated_copy_passes():
    for pin in PINS:
        pin(_mutant())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    failed = 0
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError:
            failed += 1
    assert failed >= 1, name
