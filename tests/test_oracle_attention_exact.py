"""The exact attention case and the mistakes it must catch (CPU only).

With every query 0, every score is 0 and every probability 1/(L+1); with
values that are odd integers in {-3, -1, 1, 3} and L + 1 a power of two, the
output sum_j v_j / (L + 1) is exact in binary arithmetic and the fp16 output
is fixed bit for bit (the kernel sums integers in fp32 and scales by a power
of two, both exact). The GPU test compares the kernel's output bits with the
oracle's on the bench's attention shapes.

These pins show, on the oracle and the CPU, that the comparison is
discriminating: the generated sums n stay below 1024 in magnitude, so with
L + 1 = 2^p the exact output n 2^-p is an fp16 number (at most 10
significant bits) below 2^(10-p), where an fp16 step is at most 2^-(p+1); a
change of n by any nonzero integer moves the output by at least 2^-p, two
fp16 steps or more; and copies of the oracle step with a
kernel-like mistake planted -- the last cached position dropped, a whole
32-position block dropped or read twice, the new token left out, the wrong
key/value head for a query head -- give different fp16 bits, at 1024 and
4096 positions per sequence.
"""
import numpy as np
import pytest

import oracle
import synth

EXACT_SHAPES = [
    # (workload, L): L + 1 a power of two, shapes of the bench's attention workloads
    (synth.AttnWorkload("mha", 1, 32, 32, 128, 0), 1023),
    (synth.AttnWorkload("mha", 1, 32, 32, 128, 0), 4095),
    (synth.AttnWorkload("gqa", 1, 32, 8, 128, 0, theta=500000.0), 4095),
    (synth.AttnWorkload("mqa", 1, 71, 1, 64, 0), 2047),
]


def _bits(out):
    return np.asarray(out, np.float64).astype(np.float16).view(np.uint16)


def _step(w, qkv, k, v, lengths):
    out, _, _ = oracle.decode_step64(qkv, k, v, lengths, w.Hq, w.Hkv, w.D, w.theta, w.rope)
    return out


@pytest.mark.parametrize("w,L", EXACT_SHAPES, ids=lambda a: getattr(a, "name", str(a)))
def test_exact_inputs_fix_every_output_bit(w, L):
    qkv, k, v, lengths = synth.attention_exact_inputs(w, L, seed=1)
    assert (L + 1) & L == 0
    vnew = qkv[:, (w.Hq + w.Hkv) * w.D:].astype(np.float64).reshape(w.B, w.Hkv, 1, w.D)
    sums = v[:, :, :L].astype(np.float64).sum(axis=2, keepdims=True) + vnew
    assert np.all(np.abs(sums) < 1024)
    out = _step(w, qkv, k, v, lengths)
    # the oracle's value is the exact mean (a dyadic rational)
    g = w.Hq // w.Hkv
    exact = np.repeat(sums / (L + 1), g, axis=1).reshape(w.B, w.Hq, w.D)
    assert np.array_equal(out, exact)
    # and it is exactly representable in fp16: no rounding decides the bits
    assert np.array_equal(out.astype(np.float16).astype(np.float64), out)


def _drop_positions(k, v, L, drop):
    keep = np.setdiff1d(np.arange(L), drop)
    return k[:, :, keep], v[:, :, keep], len(keep)


def _mutant_outputs(w, qkv, k, v, lengths):
    L = int(lengths[0])
    out = {}
    kk, vv, n = _drop_positions(k, v, L, [L - 1])
    out["last position dropped"] = _step(w, qkv, kk, vv, np.array([n], np.int32))
    blk = (L // 2) // 32 * 32
    kk, vv, n = _drop_positions(k, v, L, np.arange(blk, blk + 32))
    out["32-block dropped"] = _step(w, qkv, kk, vv, np.array([n], np.int32))
    idx = np.concatenate([np.arange(L), np.arange(blk, blk + 32)])
    out["32-block read twice"] = _step(w, qkv, k[:, :, idx], v[:, :, idx], np.array([L + 32], np.int32))
    # new token left out: softmax over the cached positions only (q = 0:
    # uniform over them)
    g = w.Hq // w.Hkv
    cached = v[:, :, :L].astype(np.float64).mean(axis=2)
    out["new token left out"] = np.repeat(cached[:, :, None, :], g, axis=2).reshape(w.B, w.Hq, w.D)
    if 1 < w.Hkv < w.Hq:
        # query head h reading kv head h % Hkv instead of h // (Hq / Hkv)
        ref = _step(w, qkv, k, v, lengths).reshape(w.B, w.Hkv, g, w.D)
        heads = np.arange(w.Hq)
        perm = ref[:, heads % w.Hkv, 0]  # kv head j's output is any of its query heads'
        out["kv head h % Hkv"] = perm
    return out


@pytest.mark.parametrize("w,L", EXACT_SHAPES[:3], ids=lambda a: getattr(a, "name", str(a)))
def test_exact_case_catches_planted_mistakes(w, L):
    qkv, k, v, lengths = synth.attention_exact_inputs(w, L, seed=1)
    ref = _bits(_step(w, qkv, k, v, lengths))
    for what, mutant in _mutant_outputs(w, qkv, k, v, lengths).items():
        assert not np.array_equal(_bits(mutant), ref), f"{what} gives the same fp16 bits"
        # and it changes the bits of most outputs, not of a lucky few
        frac = np.mean(_bits(mutant) != ref)
        assert frac > 0.5, f"{what}: only {frac:.2%} of the outputs change"
