"""Seeded random shapes and plans through awq_linear, awq_linear_silu_mul,
awq_linear_w4a8 and awq_attention_decode: every plan the library accepts must
meet the tolerance (any plan it rejects must be rejected before a launch,
with AWQ_ERR_PLAN)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, check_close, log, to_np16, upload_layer, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def random_plan(rng):
    if rng.random() < 0.3:
        return None
    if rng.random() < 0.6:
        p = {"path": 1, "waves": int(rng.choice([0, 1, 2, 4, 8, 16])), "x_stage": int(rng.choice([0, 1, 2])),
             "tpw": int(rng.choice([0, 1, 2, 4]))}
    else:
        p = {"path": 2, "tile": int(rng.choice([0, 1, 2, 3])), "split_k": int(rng.choice([0, 1, 2, 3, 7]))}
    return p


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_and_plans(awq, seed):
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.choice([32, 64, 128, 256]))
    K = G * int(rng.integers(1, max(2, 2048 // G) + 1))
    N = 32 * int(rng.integers(1, 20))
    M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 33, 64, 65, 130, 257]))
    gated = bool(rng.random() < 0.35)
    plan = random_plan(rng)
    planner = awq.linear_silu_mul_plan if gated else awq.linear_plan
    try:
        used = planner(M, K, N, G, plan)
    except awq.AWQError as e:
        assert e.status == -7, e  # only plan errors for valid shapes
        log(f"random seed={seed} M={M} K={K} N={N} G={G} gated={gated} plan={plan}: rejected")
        return
    log(f"random seed={seed} M={M} K={K} N={N} G={G} gated={gated} plan={plan} -> {used}")
    q, z, s = synth.layer(K, N, G, seed=seed)
    x = synth.activations(M, K, seed=seed, outlier_frac=0.01 if K >= 100 else 0.0)
    qw, zw, sd = upload_layer(q, z, s)
    if gated:
        y = to_np16(awq.linear_silu_mul(x_dev(x), qw, sd, zw, N, G, plan=plan)).astype(np.float64)
        ref = oracle.linear_silu_mul64(x, q, z, s, G)
        E = oracle.silu_mul_scale(x, q, z, s, G)
        assert np.all(np.isfinite(y))
        err = float(np.max(np.abs(y - ref)[E > 0] / E[E > 0]))
        assert err <= TOL, err
    else:
        y = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G, plan=plan))
        check_close(y, oracle.linear64(x, q, z, s, G), oracle.l1_scale(x, q, z, s, G), what=f"seed {seed}")


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_split(awq, seed):
    # the streamed decode kernel with K split over workgroups, plain and gated
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.choice([32, 64, 128, 256]))
    K = G * int(rng.integers(1, max(2, 4096 // G) + 1))
    N = 32 * int(rng.integers(1, 20))
    M = int(rng.choice([1, 2, 5, 8, 16, 17, 31, 32]))
    gated = bool(rng.random() < 0.35)
    plan = {"path": 1, "x_stage": 2, "waves": int(rng.choice([4, 8])), "tpw": int(rng.choice([1, 2, 4])),
            "split_k": int(rng.choice([2, 3, 4, 6, 16]))}
    planner = awq.linear_silu_mul_plan if gated else awq.linear_plan
    try:
        used = planner(M, K, N, G, plan)
    except awq.AWQError as e:
        assert e.status == -7, e
        log(f"random split seed={seed} M={M} K={K} N={N} G={G} gated={gated} plan={plan}: rejected")
        return
    log(f"random split seed={seed} M={M} K={K} N={N} G={G} gated={gated} plan={plan} -> {used}")
    q, z, s = synth.layer(K, N, G, seed=seed + 50)
    x = synth.activations(M, K, seed=seed + 50)
    qw, zw, sd = upload_layer(q, z, s)
    if gated:
        y = to_np16(awq.linear_silu_mul(x_dev(x), qw, sd, zw, N, G, plan=plan)).astype(np.float64)
        ref = oracle.linear_silu_mul64(x, q, z, s, G)
        E = oracle.silu_mul_scale(x, q, z, s, G)
        assert np.all(np.isfinite(y))
        assert float(np.max(np.abs(y - ref)[E > 0] / E[E > 0])) <= TOL
    else:
        y = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G, plan=plan))
        check_close(y, oracle.linear64(x, q, z, s, G), oracle.l1_scale(x, q, z, s, G), what=f"seed {seed}")


@pytest.mark.parametrize("seed", range(12))
def test_random_w4a8(awq, seed):
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([32, 64, 128, 256]))
    step = max(G, 128)  # K % 128 == 0 and K % G == 0
    K = step * int(rng.integers(1, max(2, 2048 // step) + 1))
    N = 8 * int(rng.integers(1, 80))
    M = int(rng.choice([1, 2, 7, 16, 33, 64, 130, 257, 513]))
    plan = None if rng.random() < 0.4 else {"tile": int(rng.choice([2, 3])),
                                            "split_k": int(rng.choice([0, 1, 2, 3, 5]))}
    try:
        used = awq.linear_w4a8_plan(M, K, N, G, plan)
    except awq.AWQError as e:
        assert e.status == -7, e
        log(f"random w4a8 seed={seed} M={M} K={K} N={N} G={G} plan={plan}: rejected")
        return
    log(f"random w4a8 seed={seed} M={M} K={K} N={N} G={G} plan={plan} -> {used}")
    q, z, s = synth.layer(K, N, G, seed=seed)
    x = synth.activations(M, K, seed=seed, outlier_frac=0.01)
    qw, zw, sd = upload_layer(q, z, s)
    y = to_np16(awq.linear_w4a8(x_dev(x), qw, sd, zw, N, G, plan=plan)).astype(np.float64)
    codes, sx = oracle.quantize_act_fp8(x)
    y64 = oracle.linear_w4a8_64(codes, sx, q, z, s, G)
    D = oracle.w4a8_l1_scale(codes, sx, q, z, s, G)
    assert np.all(np.isfinite(y))
    assert np.all(y[D == 0] == 0)
    err = float(np.max(np.abs(y - y64) / np.where(D > 0, D, 1.0)))
    assert err <= TOL, f"normalised error {err:.3e}"


@pytest.mark.parametrize("seed", range(12))
def test_random_attention(awq, seed):
    from tests.test_gpu_attention import _inputs, check_step, run_step
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7, 16, 20]))
    Hq = Hkv * g
    B = int(rng.integers(1, 5))
    S = 32 * int(rng.integers(1, 40))
    max_cached = int(rng.integers(0, S))
    lengths = rng.integers(0, max_cached + 1, B).astype(np.int32)
    rope = str(rng.choice(["none", "half", "interleaved"]))
    theta = float(rng.choice([10000.0, 500000.0]))
    steps = int(rng.choice([0, 0, 1, 2, 3]))
    log(f"random attention seed={seed} B={B} Hq={Hq} Hkv={Hkv} D={D} S={S} max_cached={max_cached} "
        f"lengths={lengths.tolist()} rope={rope} steps={steps}")
    qkv, kc, vc = _inputs(B, Hq, Hkv, D, S, 4000 + seed)
    got = run_step(awq, qkv, kc, vc, lengths, Hq, Hkv, max_cached, rope, theta, steps=steps)
    check_step(qkv, kc, vc, lengths, Hq, Hkv, rope, theta, got, what=f"seed {seed}")

