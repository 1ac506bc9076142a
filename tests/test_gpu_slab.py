"""Slab variant of the decode path (x_stage 3: eight waves on the same
bands, activations staged per two-band slab in LDS) against the fp64 oracle:
one and two 16-row tiles, an odd number of bands (half-used last slab),
groups of 128, 256 and 512 rows, partial column tiles and column groups,
K splits from 1 to 5 with one, two and four tiles per wave; the automatic plans on
the shapes where they choose it, q == z, and the no-alloc entry point."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_close, log, to_np16, upload_layer, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


SLAB_SHAPES = [
    # (M, K, N, G)
    (1, 128, 16, 128), (5, 384, 40, 128), (16, 1024, 136, 256), (17, 512, 264, 128),
    (32, 1280, 520, 128), (3, 4096, 1000, 128), (32, 11008, 72, 128), (8, 2560, 4104, 512),
]


@pytest.mark.parametrize("M,K,N,G", SLAB_SHAPES)
def test_slab_plans(awq, M, K, N, G):
    log(f"slab M={M} K={K} N={N} G={G}")
    q, z, s = synth.layer(K, N, G, seed=M + K + 3)
    x = synth.activations(M, K, seed=N + 3)
    y64 = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    qw, zw, sd = upload_layer(q, z, s)
    xd = x_dev(x)
    for tpw in (1, 2, 4):
        for split in (0, 1, 2, 3, 5):
            plan = {"path": 1, "x_stage": 3, "tpw": tpw, "split_k": split}
            log(f"  plan {plan} -> {awq.linear_plan(M, K, N, G, plan)}")
            y = to_np16(awq.linear(xd, qw, sd, zw, N, G, plan=plan))
            check_close(y, y64, D, what=f"{plan}")


def test_slab_q_equals_z_is_zero(awq):
    M, K, N, G = 20, 1024, 264, 128
    log("slab q == z")
    rng = np.random.default_rng(1)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    q = np.repeat(z, G, axis=0)
    s = rng.uniform(-0.02, 0.02, size=(K // G, N)).astype(np.float16)
    x = synth.activations(M, K, seed=1)
    qw, zw, sd = upload_layer(q, z, s)
    for plan in ({"path": 1, "x_stage": 3, "tpw": 2, "split_k": 3}, {"path": 1, "x_stage": 3, "tpw": 4}):
        y = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G, plan=plan))
        assert np.all(y.astype(np.float64) == 0)


@pytest.mark.parametrize("M,K,N", [(32, 4096, 16384), (24, 1024, 16384), (17, 2048, 16520)])
def test_slab_automatic_plans(awq, M, K, N):
    # wide layers above 16 rows, on which the automatic plan picks the slab
    # variant, against the oracle on sampled columns (the large 16-row
    # layers it also picks are the Falcon-180B-shaped ones of the workload
    # tests)
    G = 128
    plan = awq.linear_plan(M, K, N, G)
    log(f"slab automatic M={M} K={K} N={N}: {plan}")
    assert plan["x_stage"] == 3, plan
    q, z, s = synth.layer(K, N, G, seed=M)
    x = synth.activations(M, K, seed=M)
    qw, zw, sd = upload_layer(q, z, s)
    y = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G))
    cols = np.random.default_rng(M).choice(N, size=min(N, 256), replace=False)
    y64 = oracle.linear64(x, q[:, cols], z[:, cols], s[:, cols], G)
    D = oracle.l1_scale(x, q[:, cols], z[:, cols], s[:, cols], G)
    check_close(y[:, cols], y64, D, what=f"automatic {plan}")
