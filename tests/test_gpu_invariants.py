"""GPU invariants of the linear layer that hold bit for bit whatever the
summation order, in every plan:

* column independence: permuting the columns of (q, z, s) permutes y;
* group locality: scaling the scales of group g by a power of two gives the
  same bits as scaling the activations of group g's input channels by it, and
  zeroing group g's scales gives the same values as zeroing those activations
  (a kernel that applied some group's scale to another group's rows, or let one
  column's metadata reach another column, fails these);
* row independence: rows of a large prefill call agree with the oracle and with
  the same rows computed alone by the decode path.

The weight matrix is W[k, n] = (q[k, n] - z[k/G, n]) * s[k/G, n] (the group-wise
asymmetric INT4 weights of the AWQ paper's W4A16 setting)."""
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


def run(awq, x, q, z, s, G, plan=None):
    qw, zw, sd = upload_layer(q, z, s)
    return to_np16(awq.linear(x_dev(x), qw, sd, zw, q.shape[1], G, plan=plan))


PLANS = [
    # (M, plan)
    (1, {"path": 1}), (1, {"path": 1, "waves": 4, "x_stage": 2}), (3, {"path": 1, "waves": 16, "x_stage": 1, "tpw": 2}),
    (8, {"path": 1, "waves": 4, "x_stage": 2, "tpw": 4}), (16, {"path": 1}), (33, {"path": 1}),
    (16, {"path": 1, "waves": 8, "x_stage": 2, "tpw": 2}),
    (16, {"path": 1, "waves": 4, "x_stage": 2, "tpw": 2, "split_k": 3}),
    (32, {"path": 1, "waves": 8, "x_stage": 2, "tpw": 4, "split_k": 2}),
    (80, {"path": 2, "tile": 1}), (130, {"path": 2, "tile": 3, "split_k": 3}), (70, {"path": 2, "tile": 2, "split_k": 2}),
]
SHAPES = [(1024, 264, 128), (768, 136, 64), (640, 72, 32)]


def _cases():
    for M, plan in PLANS:
        for K, N, G in SHAPES:
            yield pytest.param(M, K, N, G, plan, id=f"M{M}-K{K}-N{N}-G{G}-{'-'.join(f'{k}{v}' for k, v in plan.items())}")


@pytest.mark.parametrize("M,K,N,G,plan", list(_cases()))
def test_column_permutation_bitwise(awq, M, K, N, G, plan):
    log(f"permutation M={M} K={K} N={N} G={G} plan={plan}")
    q, z, s = synth.layer(K, N, G, seed=K + N)
    x = synth.activations(M, K, seed=M)
    perm = np.random.default_rng(N).permutation(N)
    y = run(awq, x, q, z, s, G, plan)
    yp = run(awq, x, q[:, perm], z[:, perm], s[:, perm], G, plan)
    assert np.array_equal(yp.view(np.uint16), y[:, perm].view(np.uint16))
    check_close(y, oracle.linear64(x, q, z, s, G), oracle.l1_scale(x, q, z, s, G), what=f"{plan}")


@pytest.mark.parametrize("M,K,N,G,plan", list(_cases()))
def test_group_locality_bitwise(awq, M, K, N, G, plan):
    log(f"group locality M={M} K={K} N={N} G={G} plan={plan}")
    q, z, s = synth.layer(K, N, G, seed=K + 3 * N)
    x = synth.activations(M, K, seed=M + 1)
    ng = K // G
    for g in sorted({0, ng // 2, ng - 1}):
        rows = slice(g * G, (g + 1) * G)
        # power-of-two scale on group g: through the scales, or through x
        s2 = s.copy()
        s2[g] = (s2[g].astype(np.float32) * 4).astype(np.float16)
        x2 = x.copy()
        x2[:, rows] = (x2[:, rows].astype(np.float32) * 4).astype(np.float16)
        a = run(awq, x, q, z, s2, G, plan)
        b = run(awq, x2, q, z, s, G, plan)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"group {g}: scale x4"
        # zero group g: through the scales, or through x (signs of zeros aside)
        s0 = s.copy()
        s0[g] = 0
        x0 = x.copy()
        x0[:, rows] = 0
        a = run(awq, x, q, z, s0, G, plan).astype(np.float64)
        b = run(awq, x0, q, z, s, G, plan).astype(np.float64)
        assert np.array_equal(a, b), f"group {g}: zeroed"
        check_close(a.astype(np.float16), oracle.linear64(x0, q, z, s, G), oracle.l1_scale(x0, q, z, s, G),
                    what=f"group {g} zeroed")


def test_column_metadata_stays_in_its_column(awq):
    # Changing one column's scales and zero points changes that column only.
    M, K, N, G = 4, 1024, 136, 128
    q, z, s = synth.layer(K, N, G, seed=11)
    x = synth.activations(M, K, seed=11)
    for plan in ({"path": 1}, {"path": 1, "waves": 4, "x_stage": 2, "tpw": 2}, {"path": 2, "tile": 1},
                 {"path": 2, "tile": 3, "split_k": 2}):
        log(f"column metadata plan={plan}")
        y = run(awq, x, q, z, s, G, plan)
        for c in (0, 7, 8, 71, N - 1):
            z2, s2 = z.copy(), s.copy()
            z2[:, c] = 15 - z2[:, c]
            s2[:, c] = -s2[:, c]
            y2 = run(awq, x, q, z2, s2, G, plan)
            other = np.arange(N) != c
            assert np.array_equal(y2[:, other].view(np.uint16), y[:, other].view(np.uint16)), f"column {c}"
            check_close(y2, oracle.linear64(x, q, z2, s2, G), oracle.l1_scale(x, q, z2, s2, G), what=f"col {c}")


def test_rows_of_large_prefill_match_decode(awq):
    # M = 2048 prefill (the MFMA-bound size) against the oracle on sampled rows,
    # and each sampled row computed alone by the decode path.
    M, K, N, G = 2048, 4096, 1024, 128
    log(f"row independence M={M} K={K} N={N}")
    q, z, s = synth.layer(K, N, G, seed=5)
    x = synth.activations(M, K, seed=5)
    qw, zw, sd = upload_layer(q, z, s)
    assert awq.linear_plan(M, K, N, G)["path"] == 2
    y = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G))
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 1], np.random.default_rng(5).choice(M, 27, replace=False)]))
    y64 = oracle.linear64(x[rows], q, z, s, G)
    D = oracle.l1_scale(x[rows], q, z, s, G)
    check_close(y[rows], y64, D, what="prefill rows")
    for i, r in enumerate(rows[:8]):
        yr = to_np16(awq.linear(x_dev(x[r:r + 1]), qw, sd, zw, N, G))
        check_close(yr, y64[i:i + 1], D[i:i + 1], what=f"decode row {r}")
        check_close(yr, y[r:r + 1].astype(np.float64), D[i:i + 1], tol=4e-3, what=f"decode vs prefill row {r}")


@pytest.mark.parametrize("M,K,N,G,plan", [(1, 1024, 288, 128, None), (16, 768, 160, 64, None),
                                          (16, 1024, 512, 128, {"path": 1, "x_stage": 2, "tpw": 4}),
                                          (130, 640, 160, 32, {"path": 2, "split_k": 2})])
def test_gated_column_permutation_bitwise(awq, M, K, N, G, plan):
    # The same permutation applied to the gate half and to the up half of the
    # fused layer permutes silu(gate) * up.
    log(f"gated permutation M={M} K={K} N={N} G={G} plan={plan}")
    q, z, s = synth.layer(K, N, G, seed=K + N)
    x = synth.activations(M, K, seed=M)
    n2 = N // 2
    perm = np.random.default_rng(N).permutation(n2)
    both = np.concatenate([perm, perm + n2])

    def gated(q, z, s):
        qw, zw, sd = upload_layer(q, z, s)
        return to_np16(awq.linear_silu_mul(x_dev(x), qw, sd, zw, N, G, plan=plan))

    y = gated(q, z, s)
    yp = gated(q[:, both], z[:, both], s[:, both])
    assert np.array_equal(yp.view(np.uint16), y[:, perm].view(np.uint16))
