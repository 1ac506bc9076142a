"""Pins for the oracle's linear layer (CPU only).

* q == z everywhere gives y == 0;
* with exactly representable weights and activations, the oracle equals the
  dense matmul of the fp16 weights, exactly, and the exact rational sum;
* on tiny shapes, the exact rational triple loop (no numpy) agrees with the
  oracle to fp64 accuracy;
* plausible mistakes (group index taken modulo, zero point dropped, sign of
  the zero point flipped, transposed operand, wrong nibble order) are planted
  in copies of the oracle here and each one is caught by these pins.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _tiny(M, K, N, G, seed):
    q, z, s = synth.layer(K, N, G, seed=seed)
    # asymmetric scales (both signs) so sign errors cannot cancel
    rng = np.random.default_rng(seed + 100)
    s = (s.astype(np.float64) * rng.choice([-1.0, 1.0], size=s.shape)).astype(np.float16)
    x = synth.activations(M, K, seed=seed)
    return x, q, z, s


def test_q_equals_z_gives_zero():
    K, N, G = 256, 24, 64
    rng = np.random.default_rng(0)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    q = np.repeat(z, G, axis=0)
    s = rng.uniform(-0.02, 0.02, size=(K // G, N)).astype(np.float16)
    x = synth.activations(5, K)
    y = oracle.linear64(x, q, z, s, G)
    assert np.all(y == 0)


def exact_case(M, K, N, G, seed=0):
    """Weights (q - z) * 2^-6 and activations in {-1, 0, 1} with 8 non-zeros
    per row: every product and partial sum is exactly representable."""
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    s = np.full((K // G, N), 2.0 ** -6, np.float16)
    x = np.zeros((M, K), np.float16)
    for m in range(M):
        cols = rng.choice(K, size=min(8, K), replace=False)
        x[m, cols] = rng.choice([-1.0, 1.0], size=cols.size)
    return x, q, z, s


def test_exact_case_equals_dense_fp16_matmul():
    M, K, N, G = 9, 512, 40, 128
    x, q, z, s = exact_case(M, K, N, G)
    W16 = oracle.dequant16(q, z, s, G)
    y = oracle.linear64(x, q, z, s, G)
    dense = x.astype(np.float64) @ W16.astype(np.float64)
    assert np.array_equal(y, dense)
    # and the exact rational value (fractions), with no numpy arithmetic
    for m in range(M):
        for n in range(0, N, 7):
            acc = Fraction(0)
            for k in range(K):
                if x[m, k] != 0:
                    acc += Fraction(float(x[m, k])) * (int(q[k, n]) - int(z[k // G, n])) * Fraction(1, 64)
            assert Fraction(y[m, n]) == acc


CASES = [(1, 32, 8, 32), (2, 64, 16, 32), (3, 128, 24, 64), (9, 128, 8, 128), (2, 384, 16, 128),
         (3, 192, 8, 64)]


@pytest.mark.parametrize("M,K,N,G", CASES)
def test_bruteforce_tiny(M, K, N, G):
    x, q, z, s = _tiny(M, K, N, G, seed=M * 1000 + K + N + G)
    y = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    exact = oracle.linear_bruteforce(x, q, z, s, G)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(y[m, n]) - exact[m][n])
            assert err <= Fraction(1, 10 ** 15) * Fraction(D[m, n]) + Fraction(0), (m, n)


def test_linearity_and_locality():
    M, K, N, G = 4, 256, 16, 64
    x, q, z, s = _tiny(M, K, N, G, seed=5)
    y = oracle.linear64(x, q, z, s, G)
    # scaling x by a power of two scales y exactly
    y2 = oracle.linear64((x.astype(np.float64) * 4).astype(np.float16), q, z, s, G)
    assert np.array_equal(y2, 4 * y)
    # permuting columns of (q, z, s) permutes y
    perm = np.random.default_rng(1).permutation(N)
    yp = oracle.linear64(x, q[:, perm], z[:, perm], s[:, perm], G)
    assert np.array_equal(yp, y[:, perm])
    # changing one group's scales changes y by exactly that group's term
    s2 = s.copy()
    s2[2, :] = (s2[2, :].astype(np.float64) * 2).astype(np.float16)
    d = oracle.linear64(x, q, z, s2, G) - y
    rows = slice(2 * G, 3 * G)
    term = x[:, rows].astype(np.float64) @ ((q[rows].astype(np.float64) - z[2].astype(np.float64)) * s[2].astype(np.float64))
    assert np.allclose(d, term, rtol=0, atol=1e-12)


def test_normalised_error_metric():
    y64 = np.array([[1.0, 0.0, -2.0]])
    D = np.array([[10.0, 0.0, 4.0]])
    assert oracle.normalised_error(y64, y64, D) == 0.0
    assert oracle.normalised_error(np.array([[1.5, 0.0, -2.0]]), y64, D) == pytest.approx(0.05)
    assert oracle.normalised_error(np.array([[1.0, 1e-9, -2.0]]), y64, D) == float("inf")


# ---- planted mistakes: each mutant must fail at least one pin above ----------

def _mut_group_mod(x, q, z, s, G):
    K = q.shape[0]
    g = np.arange(K) % (K // G)
    return x.astype(np.float64) @ ((q.astype(np.float64) - z[g].astype(np.float64)) * s[g].astype(np.float64))


def _mut_drop_zero(x, q, z, s, G):
    g = np.arange(q.shape[0]) // G
    return x.astype(np.float64) @ (q.astype(np.float64) * s[g].astype(np.float64))


def _mut_zero_sign(x, q, z, s, G):
    g = np.arange(q.shape[0]) // G
    return x.astype(np.float64) @ ((q.astype(np.float64) + z[g].astype(np.float64)) * s[g].astype(np.float64))


def _mut_scale_after_sum(x, q, z, s, G):
    # scale taken from group 0 for every row
    return x.astype(np.float64) @ ((q.astype(np.float64) - np.repeat(z, G, 0).astype(np.float64)) * s[0].astype(np.float64))


def _mut_transpose_square(x, q, z, s, G):
    g = np.arange(q.shape[0]) // G
    w = (q.astype(np.float64) - z[g].astype(np.float64)) * s[g].astype(np.float64)
    return x.astype(np.float64) @ w.T if w.shape[0] == w.shape[1] else x.astype(np.float64) @ w[::-1]


@pytest.mark.parametrize("mutant", [_mut_group_mod, _mut_drop_zero, _mut_zero_sign,
                                    _mut_scale_after_sum, _mut_transpose_square])
def test_pins_catch_planted_mistakes(mutant):
    M, K, N, G = 3, 128, 16, 32
    x, q, z, s = _tiny(M, K, N, G, seed=11)
    exact = oracle.linear_bruteforce(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    y = mutant(x, q, z, s, G)
    worst = max(abs(Fraction(y[m, n]) - exact[m][n]) / Fraction(D[m, n])
                for m in range(M) for n in range(N) if D[m, n] > 0)
    assert worst > 1e-6


def test_pins_catch_wrong_nibble_order():
    # A canonical pack with most-significant-nibble-first order fails the
    # worked examples.
    def bad_pack(q):
        K, N = q.shape
        out = np.zeros((K // 8, N), np.uint32)
        for i in range(8):
            out |= q[i::8].astype(np.uint32) << np.uint32(4 * (7 - i))
        return out
    codes = np.arange(8, dtype=np.uint8).reshape(8, 1)
    assert int(bad_pack(codes)[0, 0]) != 0x76543210
    assert int(oracle.pack_canonical(codes)[0, 0]) == 0x76543210
