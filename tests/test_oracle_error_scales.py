"""Two-sided pins for the error scales the GPU parity tests divide by (CPU only).

Every parity bar has the form |kernel - oracle| <= 2e-3 * scale, so a scale
that came out too large would silently loosen every test that uses it. Each
scale is therefore pinned from above as well as from below, on cases where
its value is known in closed form from exact rational arithmetic:

* ``l1_scale`` (the W4A16 layer's D = sum_k |x w|): equal to a Fraction triple
  loop; equal to the output itself when every product has the same sign;
  unchanged by sign flips of x and s.
* ``silu_mul_scale`` (the gated layer): equal to its closed form where the
  gate and up sums and their L1 norms are known exactly; zero where either
  half of the layer is identically zero.
* ``decode_error_scale`` (attention): with uniform probabilities (q = 0, or
  every key with the same product with q) equal to (1 + sigma) times the
  mean |v| plus |mean v| in closed form; on an empty cache (1 + sigma) 2|v|.

Plausible mistakes in each (a factor of 2, a looser norm, a missing absolute
value, a sum for a maximum, a dropped term, the two halves swapped) are
planted in copies of the oracle here, and each one fails at least one pin.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


# ---------------------------------------------------------------------------
# l1_scale
# ---------------------------------------------------------------------------

def _mixed_layer(M, K, N, G, seed):
    q, z, s = synth.layer(K, N, G, seed=seed)
    rng = np.random.default_rng(seed + 1)
    s = (s.astype(np.float64) * rng.choice([-1.0, 1.0], size=s.shape)).astype(np.float16)
    x = synth.activations(M, K, seed=seed)
    return x, q, z, s


def _l1_fraction(x, q, z, s, G):
    M, K = x.shape
    N = q.shape[1]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                w = (int(q[k, n]) - int(z[k // G, n])) * Fraction(float(s[k // G, n]))
                acc += abs(Fraction(float(x[m, k]))) * abs(w)
            out[m, n] = acc
    return out


def _same_sign_layer(K, N, G, seed, sign):
    """q >= z everywhere and s of one sign, x >= 0: every product x * w has
    the sign `sign`."""
    rng = np.random.default_rng(seed)
    z = rng.integers(0, 8, size=(K // G, N), dtype=np.uint8)
    q = (np.repeat(z, G, axis=0) + rng.integers(0, 8, size=(K, N))).astype(np.uint8)
    s = (sign * rng.uniform(0.001, 0.02, size=(K // G, N))).astype(np.float16)
    x = np.abs(synth.activations(4, K, seed=seed))
    return x, q, z, s


def l1_pins(fn):
    """Runs every l1_scale pin on `fn`; returns the names of the pins it fails."""
    failed = []
    x, q, z, s = _mixed_layer(3, 96, 16, 32, seed=3)
    D = fn(x, q, z, s, 32)
    exact = _l1_fraction(x, q, z, s, 32)
    if not all(abs(Fraction(float(D[m, n])) - exact[m, n]) <= Fraction(1, 10 ** 14) * exact[m, n]
               for m in range(3) for n in range(16)):
        failed.append("rational sum")
    for sign in (1.0, -1.0):
        xs, qs, zs, ss = _same_sign_layer(256, 24, 64, seed=4, sign=sign)
        y = oracle.linear64(xs, qs, zs, ss, 64)
        if not np.allclose(fn(xs, qs, zs, ss, 64), sign * y, rtol=1e-14, atol=0):
            failed.append(f"same-sign products ({sign:+.0f})")
    flipped = fn((-x.astype(np.float64)).astype(np.float16), q, z, (-s.astype(np.float64)).astype(np.float16), 32)
    if not np.array_equal(flipped, D):
        failed.append("sign flips")
    return failed


def test_l1_scale_pins():
    assert l1_pins(oracle.l1_scale) == []


def _w64(q, z, s, G):
    g = np.arange(q.shape[0]) // G
    return (q.astype(np.float64) - z[g].astype(np.float64)) * s[g].astype(np.float64)


def _l1_times_two(x, q, z, s, G):
    return 2 * oracle.l1_scale(x, q, z, s, G)


def _l1_norm_times_max(x, q, z, s, G):
    # the looser bound ||x_m||_1 * max_k |w_kn|
    ax = np.abs(x.astype(np.float64)).sum(axis=1)
    return ax[:, None] * np.abs(_w64(q, z, s, G)).max(axis=0)[None, :]


def _l1_no_abs_on_w(x, q, z, s, G):
    return np.abs(x.astype(np.float64)) @ _w64(q, z, s, G)


def _l1_no_abs_on_x(x, q, z, s, G):
    return x.astype(np.float64) @ np.abs(_w64(q, z, s, G))


def _l1_fp16_products(x, q, z, s, G):
    # products |x| |w| rounded to fp16 before the sum
    ax = np.abs(x.astype(np.float64))
    aw = np.abs(_w64(q, z, s, G))
    return (ax[:, :, None] * aw[None, :, :]).astype(np.float16).astype(np.float64).sum(axis=1)


def _l1_plus_constant(x, q, z, s, G):
    return oracle.l1_scale(x, q, z, s, G) + 1e-3


@pytest.mark.parametrize("mutant", [_l1_times_two, _l1_norm_times_max, _l1_no_abs_on_w, _l1_no_abs_on_x,
                                    _l1_fp16_products, _l1_plus_constant])
def test_l1_scale_pins_catch_planted_mistakes(mutant):
    assert l1_pins(mutant) != []


# ---------------------------------------------------------------------------
# silu_mul_scale
# ---------------------------------------------------------------------------

def _silu(t):
    return t / (1.0 + math.exp(-t))


def _gated_layer(K, NH, G, seed, gate_sign, up_sign, zero_half=None):
    """x >= 0; the gate half's products all have sign gate_sign, the up
    half's up_sign (or a half is identically zero: q == z)."""
    rng = np.random.default_rng(seed)
    N = 2 * NH
    z = rng.integers(0, 8, size=(K // G, N), dtype=np.uint8)
    q = (np.repeat(z, G, axis=0) + rng.integers(0, 8, size=(K, N))).astype(np.uint8)
    if zero_half == "gate":
        q[:, :NH] = np.repeat(z[:, :NH], G, axis=0)
    if zero_half == "up":
        q[:, NH:] = np.repeat(z[:, NH:], G, axis=0)
    sign = np.concatenate([np.full(NH, gate_sign), np.full(NH, up_sign)])
    s = (rng.uniform(0.001, 0.02, size=(K // G, N)) * sign[None, :]).astype(np.float16)
    x = np.abs(synth.activations(3, K, seed=seed))
    return x, q, z, s


def _exact_sums(x, q, z, s, G):
    """Exact layer sums h[m][n] as Fractions (pure Python)."""
    M, K = x.shape
    N = q.shape[1]
    return [[sum(Fraction(float(x[m, k])) * (int(q[k, n]) - int(z[k // G, n])) * Fraction(float(s[k // G, n]))
                 for k in range(K)) for n in range(N)] for m in range(M)]


def silu_pins(fn):
    failed = []
    K, NH, G = 64, 8, 32
    for gate_sign in (1.0, -1.0):
        x, q, z, s = _gated_layer(K, NH, G, seed=5, gate_sign=gate_sign, up_sign=1.0)
        h = _exact_sums(x, q, z, s, G)
        E = fn(x, q, z, s, G)
        for m in range(x.shape[0]):
            for i in range(NH):
                g, u = float(h[m][i]), float(h[m][NH + i])  # D_gate = |g|, D_up = |u| here
                want = 1.1 * abs(u) * abs(g) + abs(_silu(g)) * abs(u) + abs(_silu(g) * u)
                if not math.isclose(E[m, i], want, rel_tol=1e-12):
                    failed.append(f"closed form (gate sign {gate_sign:+.0f})")
                    break
            else:
                continue
            break
    for half in ("gate", "up"):
        x, q, z, s = _gated_layer(K, NH, G, seed=6, gate_sign=1.0, up_sign=-1.0, zero_half=half)
        if not np.all(fn(x, q, z, s, G) == 0):
            failed.append(f"zero {half} half")
    return failed


def test_silu_mul_scale_pins():
    assert silu_pins(oracle.silu_mul_scale) == []


def _silu_parts(x, q, z, s, G):
    h = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    n2 = h.shape[1] // 2
    return h[:, :n2], h[:, n2:], D[:, :n2], D[:, n2:]


def _silu_const_two(x, q, z, s, G):
    g, u, Dg, Du = _silu_parts(x, q, z, s, G)
    return 2.0 * np.abs(u) * Dg + np.abs(oracle.silu64(g)) * Du + np.abs(oracle.silu64(g) * u)


def _silu_swapped_halves(x, q, z, s, G):
    g, u, Dg, Du = _silu_parts(x, q, z, s, G)
    return 1.1 * np.abs(u) * Du + np.abs(oracle.silu64(g)) * Dg + np.abs(oracle.silu64(g) * u)


def _silu_no_output_term(x, q, z, s, G):
    g, u, Dg, Du = _silu_parts(x, q, z, s, G)
    return 1.1 * np.abs(u) * Dg + np.abs(oracle.silu64(g)) * Du


def _silu_times_two(x, q, z, s, G):
    return 2 * oracle.silu_mul_scale(x, q, z, s, G)


def _silu_plus_constant(x, q, z, s, G):
    return oracle.silu_mul_scale(x, q, z, s, G) + 1e-4


def _silu_sum_of_l1(x, q, z, s, G):
    # the cruder (|u| + |silu(g)|) (D_gate + D_up)
    g, u, Dg, Du = _silu_parts(x, q, z, s, G)
    return (np.abs(u) + np.abs(oracle.silu64(g))) * (Dg + Du) + np.abs(oracle.silu64(g) * u)


@pytest.mark.parametrize("mutant", [_silu_const_two, _silu_swapped_halves, _silu_no_output_term, _silu_times_two,
                                    _silu_plus_constant, _silu_sum_of_l1])
def test_silu_mul_scale_pins_catch_planted_mistakes(mutant):
    assert silu_pins(mutant) != []


# ---------------------------------------------------------------------------
# decode_error_scale
# ---------------------------------------------------------------------------

def _attn_uniform_case(L, D, a, c, nonneg, seed, Hq=4, Hkv=2, style="none"):
    """B = 1; q = a e_0 for every head; every key, cached and new, has
    component 0 equal to c (the others random), so every score equals
    scale * a * c and the probabilities are uniform. Values: integers in
    0..3 (nonneg) or in -3..3. With a = 0 the query is zero."""
    rng = np.random.default_rng(seed)
    S = L + 1
    qkv = np.zeros((1, (Hq + 2 * Hkv) * D))
    qkv[0, :Hq * D].reshape(Hq, D)[:, 0] = a
    k = rng.standard_normal((1, Hkv, S, D))
    k[..., 0] = c
    knew = rng.standard_normal((Hkv, D))
    knew[:, 0] = c
    qkv[0, Hq * D:(Hq + Hkv) * D] = knew.reshape(-1)
    lo = 0 if nonneg else -3
    vals = rng.integers(lo, 4, size=(1, Hkv, S, D)).astype(np.float64)
    vnew = rng.integers(lo, 4, size=(Hkv, D)).astype(np.float64)
    qkv[0, (Hq + Hkv) * D:] = vnew.reshape(-1)
    return (qkv.astype(np.float16), k.astype(np.float16), vals.astype(np.float16),
            np.array([L], np.int32), Hq, Hkv, style)


def _uniform_expected(qkv, k, v, lengths, Hq, Hkv, D, sigma):
    """(1 + sigma) (mean_j |v_j| + |mean_j v_j|) over the L cached values and
    the new one, per query head (head h reads kv head h // (Hq / Hkv))."""
    L = int(lengths[0])
    vnew = qkv[0, (Hq + Hkv) * D:].astype(np.float64).reshape(Hkv, D)
    E = np.zeros((1, Hq, D))
    for h in range(Hq):
        j = h // (Hq // Hkv)
        vals = np.concatenate([v[0, j, :L].astype(np.float64), vnew[j:j + 1]])
        n = Fraction(L + 1)
        for d in range(D):
            col = [Fraction(float(t)) for t in vals[:, d]]
            mean_abs = sum(abs(t) for t in col) / n
            abs_mean = abs(sum(col) / n)
            E[0, h, d] = float((1 + sigma) * (mean_abs + abs_mean))
    return E


def attention_scale_pins(fn):
    failed = []
    D = 64
    # q = 0: sigma = 0, uniform probabilities, L + 1 a power of two and not
    for L, nonneg in ((63, True), (63, False), (100, False)):
        case = _attn_uniform_case(L, D, 0.0, 0.5, nonneg, seed=L)
        qkv, k, v, lengths, Hq, Hkv, style = case
        E = fn(qkv, k, v, lengths, Hq, Hkv, D, 1e4, style)
        if not np.allclose(E, _uniform_expected(qkv, k, v, lengths, Hq, Hkv, D, Fraction(0)), rtol=1e-14, atol=0):
            failed.append(f"q = 0, L = {L}, nonneg {nonneg}")
    # q = a e_0 and every key with component 0 = c: sigma = scale |a c|
    for a, c, scale in ((-1.5, 0.75, None), (2.0, -1.25, None), (-1.5, 0.75, 0.25)):
        qkv, k, v, lengths, Hq, Hkv, style = _attn_uniform_case(31, D, a, c, False, seed=7)
        sc = Fraction(scale) if scale is not None else None
        E = fn(qkv, k, v, lengths, Hq, Hkv, D, 1e4, style, scale)
        sigma = (float(sc) if sc is not None else 1.0 / math.sqrt(D)) * abs(a * c)
        want = _uniform_expected(qkv, k, v, lengths, Hq, Hkv, D, Fraction(sigma))
        if not np.allclose(E, want, rtol=1e-13, atol=0):
            failed.append(f"sigma, a = {a}, c = {c}, scale {scale}")
    # empty cache: o = v_new, E = (1 + sigma) 2 |v_new|, sigma = scale sum_d |q_d k_d|
    rng = np.random.default_rng(9)
    Hq, Hkv = 2, 1
    qkv = rng.standard_normal((1, (Hq + 2 * Hkv) * D)).astype(np.float16)
    k = np.zeros((1, Hkv, 32, D), np.float16)
    E = fn(qkv, k, k, np.array([0], np.int32), Hq, Hkv, D, 1e4, "none")
    kn = [Fraction(float(t)) for t in qkv[0, Hq * D:(Hq + 1) * D]]
    vn = qkv[0, (Hq + 1) * D:].astype(np.float64)
    for h in range(Hq):
        qh = [Fraction(float(t)) for t in qkv[0, h * D:(h + 1) * D]]
        sigma = float(sum(abs(a * b) for a, b in zip(qh, kn))) / math.sqrt(D)
        if not np.allclose(E[0, h], (1 + sigma) * 2 * np.abs(vn), rtol=1e-13, atol=0):
            failed.append("empty cache")
            break
    return failed


def test_decode_error_scale_pins():
    assert attention_scale_pins(oracle.decode_error_scale) == []


def _attn_variant(sigma_kind="max_abs", probs="abs", o_term=True, factor=True, scale_kind="sqrt"):
    """A copy of the oracle's error scale with one of its parts changed."""
    def fn(qkv, k_cache, v_cache, lengths, Hq, Hkv, D, theta=1e4, style="half", scale=None):
        B = qkv.shape[0]
        g = Hq // Hkv
        if scale is None:
            scale = 1.0 / (np.sqrt(D) if scale_kind == "sqrt" else D)
        E = np.zeros((B, Hq, D))
        for b in range(B):
            L = int(lengths[b])
            q, kk, vv = oracle.split_qkv(qkv[b], Hq, Hkv, D)
            q_rot = oracle.rope64(q, L, theta, style)
            k_store = oracle.rope64(kk, L, theta, style).astype(np.float16).astype(np.float64)
            for h in range(Hq):
                j = h // g
                keys = np.concatenate([np.asarray(k_cache[b, j, :L], np.float64), k_store[j:j + 1]])
                vals = np.concatenate([np.asarray(v_cache[b, j, :L], np.float64), vv[j:j + 1]])
                p = oracle.softmax64(scale * (keys @ q_rot[h]))
                o = p @ vals
                if sigma_kind == "max_abs":
                    sigma = scale * np.max(np.abs(keys) @ np.abs(q_rot[h]))
                elif sigma_kind == "max_signed":
                    sigma = scale * np.max(keys @ q_rot[h])
                else:  # sum over positions
                    sigma = scale * np.sum(np.abs(keys) @ np.abs(q_rot[h]))
                pv = p @ np.abs(vals) if probs == "abs" else np.abs(p @ vals)
                E[b, h] = (1.0 + sigma if factor else 1.0) * (pv + (np.abs(o) if o_term else 0.0))
        return E
    return fn


def test_attention_variant_copy_is_the_oracle():
    # the unmodified copy passes, so the mutants below differ only in the planted part
    assert attention_scale_pins(_attn_variant()) == []


@pytest.mark.parametrize("kw", [dict(sigma_kind="max_signed"), dict(sigma_kind="sum"), dict(probs="signed"),
                                dict(o_term=False), dict(factor=False), dict(scale_kind="linear")],
                         ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_decode_error_scale_pins_catch_planted_mistakes(kw):
    assert attention_scale_pins(_attn_variant(**kw)) != []


def test_decode_error_scale_times_two_is_caught():
    assert attention_scale_pins(lambda *a, **k: 2 * oracle.decode_error_scale(*a, **k)) != []
