"""Pins for the oracle's gated epilogue y = silu(gate) * up (CPU only).

silu is pinned by facts independent of its code: the identity
silu(t) - silu(-t) = t, the closed form through tanh,
silu(t) = t/2 * (1 + tanh(t/2)), its limits, and the bound |silu'| <= 1.1
that the error scale relies on. The gated layer is pinned by an exactly
representable case in which the gate half and the up half give different
answers when swapped or interleaved, and by zero halves.
"""
import math

import numpy as np
import pytest

import oracle


def test_silu_identities():
    t = np.linspace(-40, 40, 8001)
    s = oracle.silu64(t)
    assert np.max(np.abs(s - oracle.silu64(-t) - t)) <= 1e-12
    tanh_form = t / 2 * (1 + np.tanh(t / 2))
    assert np.max(np.abs(s - tanh_form) / np.maximum(np.abs(t), 1e-300)) <= 1e-15
    assert oracle.silu64(np.array([0.0]))[0] == 0.0
    assert oracle.silu64(np.array([-1000.0]))[0] == 0.0
    assert oracle.silu64(np.array([1000.0]))[0] == 1000.0


def test_silu_derivative_bound():
    t = np.linspace(-30, 30, 600001)
    d = np.diff(oracle.silu64(t)) / np.diff(t)
    assert np.max(np.abs(d)) <= 1.1
    assert np.max(np.abs(d)) >= 1.09  # the bound is nearly tight (max ~1.0998 near t = 2.4)


def _exact_gated(N, gate_val, up_val):
    """x = e_0; W row 0: gate columns (q - z) * s = gate_val, up columns up_val
    (s = 1, small integers, so every value is exact)."""
    K, G = 32, 32
    q = np.zeros((K, N), np.uint8)
    z = np.zeros((K // G, N), np.uint8)
    s = np.ones((K // G, N), np.float16)
    z[0, :] = 8
    q[:, :] = 8                      # q == z: zero weight everywhere else
    q[0, : N // 2] = 8 + gate_val
    q[0, N // 2:] = 8 + up_val
    x = np.zeros((1, K), np.float16)
    x[0, 0] = 1.0
    return x, q, z, s, G


def test_gate_half_then_up_half():
    x, q, z, s, G = _exact_gated(16, 2, 1)
    y = oracle.linear_silu_mul64(x, q, z, s, G)
    assert y.shape == (1, 8)
    assert np.all(y == 2 / (1 + math.exp(-2)) * 1)
    swapped = 1 / (1 + math.exp(-1)) * 2          # up half taken as the gate
    assert abs(y[0, 0] - swapped) > 0.2


def test_zero_halves_give_zero():
    x, q, z, s, G = _exact_gated(16, 3, 0)
    assert np.all(oracle.linear_silu_mul64(x, q, z, s, G) == 0)
    x, q, z, s, G = _exact_gated(16, 0, 5)
    assert np.all(oracle.linear_silu_mul64(x, q, z, s, G) == 0)


def test_error_scale_covers_first_order_perturbations():
    rng = np.random.default_rng(4)
    K, N, G = 64, 16, 32
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    z = rng.integers(0, 16, (K // G, N)).astype(np.uint8)
    s = rng.uniform(0.01, 0.1, (K // G, N)).astype(np.float16)
    x = rng.standard_normal((3, K)).astype(np.float16)
    h = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    E = oracle.silu_mul_scale(x, q, z, s, G)
    y = oracle.linear_silu_mul64(x, q, z, s, G)
    for sign in (-1, 1):
        hp = h + sign * 1e-4 * D            # every pre-activation off by 1e-4 of its scale
        yp = oracle.silu64(hp[:, :8]) * hp[:, 8:]
        assert np.max(np.abs(yp - y) / E) <= 1.01e-4


# ---- planted mistakes ---------------------------------------------------------

def _swapped(x, q, z, s, G):
    h = oracle.linear64(x, q, z, s, G)
    n2 = h.shape[1] // 2
    return oracle.silu64(h[:, n2:]) * h[:, :n2]


def _interleaved(x, q, z, s, G):
    h = oracle.linear64(x, q, z, s, G)
    return oracle.silu64(h[:, 0::2]) * h[:, 1::2]


def _sigmoid_only(x, q, z, s, G):
    h = oracle.linear64(x, q, z, s, G)
    n2 = h.shape[1] // 2
    return 1 / (1 + np.exp(-h[:, :n2])) * h[:, n2:]


@pytest.mark.parametrize("mutant", [_swapped, _interleaved, _sigmoid_only])
def test_pins_catch_planted_mistakes(mutant):
    x, q, z, s, G = _exact_gated(16, 2, 1)
    want = 2 / (1 + math.exp(-2)) * 1
    assert np.max(np.abs(mutant(x, q, z, s, G) - want)) > 0.1
