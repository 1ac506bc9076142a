"""Pins for the oracle's fused decode-step attention (CPU only).

The pages say only that the generation stage runs MHA/GQA/MQA attention with
the positional embedding fused in and pre-allocated key-value caches; the
oracle takes the textbook readings (rotary embedding, scaled dot-product
softmax attention, the new token appended at position lengths[b]). They are
pinned here by facts that do not depend on the oracle's code:

* the rotation equals multiplication of the pair (a + ib) by exp(i t) with
  complex numbers, the rates forming the geometric sequence from 1 down to
  theta^-(D-2)/D (numpy's geomspace), for both pairings;
* rotations compose: rope(rope(x, m), n) = rope(x, m + n); position 0 is the
  identity;
* the attention equals torch's scaled_dot_product_attention (fp64, CPU) on
  the cached keys plus the new rotated key, each query head on its group's
  key/value head;
* with an empty cache the output is the new value; with zero cached keys and
  values, the output fixes the new token's score in closed form, which must be
  the un-rotated q . k times the scale (rotation by the same angle keeps dot
  products);
* query heads of one group read the same key/value head; cached slots can be
  permuted (keys and values together) without changing the output;
* planted mistakes (clockwise rotation, wrong pairs, wrong rates, the key
  rotated at the wrong position, the new token left out, head h on kv head
  h % Hkv, no 1/sqrt(D), cached keys rotated again, q not rotated) each fail
  one of these pins.
"""
import numpy as np
import pytest

import oracle


def _case(B, Hq, Hkv, D, lengths, S=None, seed=0, qscale=1.0):
    rng = np.random.default_rng(seed)
    S = S or (max(lengths) + 1)
    qkv = rng.standard_normal((B, (Hq + 2 * Hkv) * D))
    qkv[:, :Hq * D] *= qscale
    kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    return qkv.astype(np.float16), kc, vc, np.asarray(lengths, np.int32)


# ---- pins, as functions of an implementation (rope64, decode_step64) --------

def pin_rope_complex(impl):
    rng = np.random.default_rng(1)
    for D, theta in ((8, 10000.0), (64, 10000.0), (128, 500000.0)):
        x = rng.standard_normal((3, D))
        rates = np.geomspace(1.0, theta ** (-(D - 2) / D), D // 2)
        for style, (a, b) in (("half", (np.arange(D // 2), np.arange(D // 2) + D // 2)),
                              ("interleaved", (np.arange(0, D, 2), np.arange(1, D, 2)))):
            for pos in (0, 1, 7, 1000, 32767):
                z = (x[:, a] + 1j * x[:, b]) * np.exp(1j * pos * rates)
                y = impl.rope64(x, pos, theta, style)
                assert np.allclose(y[:, a], z.real, rtol=0, atol=1e-9), (style, D, pos)
                assert np.allclose(y[:, b], z.imag, rtol=0, atol=1e-9), (style, D, pos)
        assert np.array_equal(impl.rope64(x, 5, theta, "none"), x)


def pin_rope_composition(impl):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 64))
    for style in ("half", "interleaved"):
        assert np.allclose(impl.rope64(x, 0, 1e4, style), x, rtol=0, atol=1e-15)
        for m, n in ((1, 2), (100, 37), (4000, 95)):
            lhs = impl.rope64(impl.rope64(x, m, 1e4, style), n, 1e4, style)
            assert np.allclose(lhs, impl.rope64(x, m + n, 1e4, style), rtol=0, atol=1e-9)


def _sdpa_reference(impl, qkv, kc, vc, lengths, Hq, Hkv, D, theta, style, scale):
    import torch
    import torch.nn.functional as F
    B = qkv.shape[0]
    g = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lengths[b])
        r = qkv[b].astype(np.float64)
        q = impl.rope64(r[:Hq * D].reshape(Hq, D), L, theta, style)
        k = impl.rope64(r[Hq * D:(Hq + Hkv) * D].reshape(Hkv, D), L, theta, style).astype(np.float16)
        v = r[(Hq + Hkv) * D:].reshape(Hkv, D)
        keys = np.concatenate([kc[b, :, :L].astype(np.float64), k[:, None].astype(np.float64)], axis=1)
        vals = np.concatenate([vc[b, :, :L].astype(np.float64), v[:, None]], axis=1)
        kt = torch.from_numpy(keys).repeat_interleave(g, dim=0)[None]
        vt = torch.from_numpy(vals).repeat_interleave(g, dim=0)[None]
        qt = torch.from_numpy(q)[None, :, None]
        out[b] = F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()
    return out


def pin_against_torch_sdpa(impl):
    for (B, Hq, Hkv, D, lengths, style, theta, qs) in (
            (2, 4, 4, 16, [5, 9], "half", 1e4, 1.0), (1, 8, 2, 32, [17], "interleaved", 5e5, 3.0),
            (3, 6, 1, 8, [0, 1, 12], "half", 1e4, 2.0), (2, 4, 2, 64, [33, 3], "none", 1e4, 1.0)):
        qkv, kc, vc, L = _case(B, Hq, Hkv, D, lengths, seed=B * D, qscale=qs)
        out, _, _ = impl.decode_step64(qkv, kc, vc, L, Hq, Hkv, D, theta, style)
        ref = _sdpa_reference(impl, qkv, kc, vc, L, Hq, Hkv, D, theta, style, 1 / np.sqrt(D))
        assert np.allclose(out, ref, rtol=0, atol=1e-12), (B, Hq, Hkv, D, style)


def pin_empty_cache_returns_value(impl):
    qkv, kc, vc, L = _case(2, 4, 2, 16, [0, 0], seed=3)
    out, _, v_new = impl.decode_step64(qkv, kc, vc, L, 4, 2, 16, 1e4, "half")
    assert np.array_equal(out, np.repeat(v_new.astype(np.float64), 2, axis=1))


def pin_new_token_score_closed_form(impl):
    # Cached keys and values all zero: o = v_new * e^s / (L + e^s) for the new
    # token's score s, which must be scale * q . k of the un-rotated vectors
    # (up to the fp16 rounding of the stored key).
    rng = np.random.default_rng(4)
    Hq, Hkv, D = 2, 1, 32
    for L, style in ((5, "half"), (11, "interleaved"), (300, "half")):
        qkv = (0.4 * rng.standard_normal((1, (Hq + 2 * Hkv) * D))).astype(np.float16)
        qkv[0, (Hq + Hkv) * D:] = 1.0  # v_new = 1 everywhere
        kc = np.zeros((1, Hkv, L + 1, D), np.float16)
        vc = np.zeros((1, Hkv, L + 1, D), np.float16)
        out, _, _ = impl.decode_step64(qkv, kc, vc, np.array([L]), Hq, Hkv, D, 1e4, style)
        q = qkv[0, :Hq * D].astype(np.float64).reshape(Hq, D)
        k = qkv[0, Hq * D:(Hq + Hkv) * D].astype(np.float64)
        for h in range(Hq):
            p = out[0, h, 0]
            assert np.allclose(out[0, h], p, rtol=0, atol=1e-12)
            with np.errstate(divide="ignore"):
                s_est = np.log(L * p / (1 - p))
            s_want = (q[h] @ k) / np.sqrt(D)
            assert abs(s_est - s_want) <= 2.0 ** -10 * np.abs(q[h]) @ np.abs(k) / np.sqrt(D) + 1e-9, (L, style, h)


def pin_group_mapping(impl):
    B, Hq, Hkv, D = 1, 12, 3, 8
    qkv, kc, vc, L = _case(B, Hq, Hkv, D, [6], seed=5)
    for j in range(Hkv):
        vc[0, j] = j + 1
        qkv[0, (Hq + Hkv + j) * D:(Hq + Hkv + j + 1) * D] = j + 1
    out, _, _ = impl.decode_step64(qkv, kc, vc, L, Hq, Hkv, D, 1e4, "half")
    for h in range(Hq):
        assert np.allclose(out[0, h], h // (Hq // Hkv) + 1, rtol=0, atol=1e-12), h


def pin_cached_slot_permutation(impl):
    qkv, kc, vc, L = _case(1, 4, 2, 16, [9], seed=6)
    out, _, _ = impl.decode_step64(qkv, kc, vc, L, 4, 2, 16, 1e4, "half")
    perm = np.random.default_rng(6).permutation(9)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, :9] = kc[:, :, perm]
    vc2[:, :, :9] = vc[:, :, perm]
    out2, _, _ = impl.decode_step64(qkv, kc2, vc2, L, 4, 2, 16, 1e4, "half")
    assert np.allclose(out, out2, rtol=0, atol=1e-13)


PINS = [pin_rope_complex, pin_rope_composition, pin_against_torch_sdpa, pin_empty_cache_returns_value,
        pin_new_token_score_closed_form, pin_group_mapping, pin_cached_slot_permutation]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_attention(pin):
    pin(oracle)


def test_appended_key_and_value():
    # The step appends the rotated key (fp16) and the value unchanged; the
    # rotated key keeps each pair's length.
    qkv, kc, vc, L = _case(2, 4, 2, 32, [3, 8], seed=7)
    _, k_new, v_new = oracle.decode_step64(qkv, kc, vc, L, 4, 2, 32, 1e4, "half")
    r = qkv.astype(np.float64)
    k = r[:, 4 * 32:6 * 32].reshape(2, 2, 32)
    assert np.array_equal(v_new, qkv[:, 6 * 32:].reshape(2, 2, 32))
    kn = k_new.astype(np.float64)
    pair_len = np.hypot(kn[..., :16], kn[..., 16:])
    assert np.allclose(pair_len, np.hypot(k[..., :16], k[..., 16:]), rtol=2 ** -10, atol=0)


def test_error_scale_covers_first_order_perturbations():
    # Perturb every rotated query element by a relative 2^-11 (the fp16
    # rounding the kernel applies); the output moves by at most 2^-11 E.
    Hq, Hkv, D = 4, 2, 32
    qkv, kc, vc, L = _case(2, Hq, Hkv, D, [20, 3], seed=8, qscale=2.0)
    out, _, _ = oracle.decode_step64(qkv, kc, vc, L, Hq, Hkv, D, 1e4, "half")
    E = oracle.decode_error_scale(qkv, kc, vc, L, Hq, Hkv, D, 1e4, "half")
    eps = 2.0 ** -11
    rng = np.random.default_rng(9)
    for _ in range(4):
        sign = rng.choice([-1.0, 1.0], size=(2, Hq, D))
        worst = 0.0
        for b in range(2):
            Lb = int(L[b])
            q = oracle.rope64(qkv[b, :Hq * D].astype(np.float64).reshape(Hq, D), Lb, 1e4, "half")
            q = q * (1 + eps * sign[b])
            k = oracle.rope64(qkv[b, Hq * D:(Hq + Hkv) * D].astype(np.float64).reshape(Hkv, D), Lb, 1e4, "half")
            v = qkv[b, (Hq + Hkv) * D:].astype(np.float64).reshape(Hkv, D)
            for h in range(Hq):
                j = h // (Hq // Hkv)
                keys = np.concatenate([kc[b, j, :Lb].astype(np.float64), k[j:j + 1].astype(np.float16).astype(np.float64)])
                vals = np.concatenate([vc[b, j, :Lb].astype(np.float64), v[j:j + 1]])
                o = oracle.softmax64(keys @ q[h] / np.sqrt(D)) @ vals
                worst = max(worst, float(np.max(np.abs(o - out[b, h]) / E[b, h])))
        assert worst <= 1.05 * eps


def test_decode_bytes():
    # two sequences, 10 and 20 cached tokens, 8 kv heads of 128: keys and
    # values 2 bytes each
    n = oracle.decode_bytes(2, [10, 20], 32, 8, 128)
    assert n == 30 * 8 * 128 * 4 + 2 * 2 * 48 * 128 + 2 * 2 * 32 * 128 + 4 * 2 * 8 * 128


# ---- planted mistakes: each mutant must fail at least one pin ----------------

class _Mutant:
    """A configurable copy of the oracle's rotation and decode step."""

    def __init__(self, clockwise=False, swap_pairs=False, rate_exponent=2.0, k_shift=0, drop_new=False,
                 gqa_mod=False, no_scale=False, rerotate_cache=False, q_plain=False):
        self.__dict__.update(locals())

    def rope64(self, x, pos, theta, style):
        x = np.asarray(x, dtype=np.float64)
        if style == "none":
            return x.copy()
        D = x.shape[-1]
        if self.swap_pairs:
            style = "interleaved" if style == "half" else "half"
        a, b = ((np.arange(D // 2), np.arange(D // 2) + D // 2) if style == "half"
                else (np.arange(0, D, 2), np.arange(1, D, 2)))
        ang = np.asarray(pos, np.float64)[..., None] * np.power(theta, -self.rate_exponent * np.arange(D // 2) / D)
        sn = -np.sin(ang) if self.clockwise else np.sin(ang)
        y = np.empty_like(x)
        y[..., a] = x[..., a] * np.cos(ang) - x[..., b] * sn
        y[..., b] = x[..., a] * sn + x[..., b] * np.cos(ang)
        return y

    def decode_step64(self, qkv, kc, vc, lengths, Hq, Hkv, D, theta=1e4, style="half", scale=None):
        B = qkv.shape[0]
        g = Hq // Hkv
        scale = 1.0 if self.no_scale else 1 / np.sqrt(D)
        out = np.zeros((B, Hq, D))
        k_new = np.zeros((B, Hkv, D), np.float16)
        v_new = np.zeros((B, Hkv, D), np.float16)
        for b in range(B):
            L = int(lengths[b])
            r = qkv[b].astype(np.float64)
            q = r[:Hq * D].reshape(Hq, D)
            q = q if self.q_plain else self.rope64(q, L, theta, style)
            k = self.rope64(r[Hq * D:(Hq + Hkv) * D].reshape(Hkv, D), L + self.k_shift, theta, style)
            k_new[b] = k.astype(np.float16)
            v = r[(Hq + Hkv) * D:].reshape(Hkv, D)
            v_new[b] = v.astype(np.float16)
            for h in range(Hq):
                j = h % Hkv if self.gqa_mod else h // g
                ck = kc[b, j, :L].astype(np.float64)
                if self.rerotate_cache:
                    ck = self.rope64(ck, np.arange(L), theta, style)
                keys, vals = ck, vc[b, j, :L].astype(np.float64)
                if not self.drop_new or L == 0:
                    keys = np.concatenate([keys, k_new[b, j:j + 1].astype(np.float64)])
                    vals = np.concatenate([vals, v[j:j + 1]])
                s = scale * (keys @ q[h])
                e = np.exp(s - s.max())
                out[b, h] = (e / e.sum()) @ vals
        return out, k_new, v_new


MUTANTS = {
    "clockwise": _Mutant(clockwise=True),
    "swapped_pairs": _Mutant(swap_pairs=True),
    "rate_exponent_i_over_D": _Mutant(rate_exponent=1.0),
    "key_at_next_position": _Mutant(k_shift=1),
    "new_token_left_out": _Mutant(drop_new=True),
    "head_modulo_kv_heads": _Mutant(gqa_mod=True),
    "no_softmax_scale": _Mutant(no_scale=True),
    "cached_keys_rotated_again": _Mutant(rerotate_cache=True),
    "query_not_rotated": _Mutant(q_plain=True),
}


def test_unmutated_copy_passes():
    for pin in PINS:
        pin(_Mutant())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    failed = 0
    for pin in PINS:
        try:
            pin(MUTANTS[name])
        except AssertionError:
            failed += 1
    assert failed >= 1, name
