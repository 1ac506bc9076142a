"""Parity at the full workload sizes, with the automatic plan (the launch
configuration the bench times), on sampled output columns that the oracle
computes one by one."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_close, log, to_np16, upload_layer, x_dev

pytestmark = pytest.mark.gpu

CASES = []
for w in synth.WORKLOADS:
    for si, shape in enumerate(w.shapes):
        CASES.append(pytest.param(w, si, id=f"{w.name}-{shape.name}"))


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


@pytest.mark.parametrize("w,si", CASES)
def test_workload_shape(awq, w, si):
    import torch
    shape = w.shapes[si]
    K, N, G = shape.K, shape.N, w.G
    log(f"{w.name} {shape.name} K={K} N={N} G={G}: generating")
    q, z, s = synth.layer(K, N, G, seed=0, layer_id=si, scales=w.scales, lo=w.lo, hi=w.hi)
    qw, zw, sd = upload_layer(q, z, s)
    rng = np.random.default_rng(si)
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, size=min(N, 254), replace=False)]))
    for M in w.Ms:
        x = synth.activations(M, K, seed=0, stream=si, outlier_frac=w.outlier_frac)
        plan = awq.linear_plan(M, K, N, G)
        log(f"  M={M} plan={plan}")
        y = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G))
        torch.cuda.synchronize()
        # Oracle on the sampled columns only (the layer is column-separable);
        # large M: also sample rows.
        rows = np.arange(M) if M <= 64 else np.unique(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
        xs = x[rows]
        y64 = oracle.linear64(xs, q[:, cols], z[:, cols], s[:, cols], G)
        D = oracle.l1_scale(xs, q[:, cols], z[:, cols], s[:, cols], G)
        check_close(y[np.ix_(rows, cols)], y64, D, what=f"{w.name}/{shape.name}/M={M}")
        assert np.all(np.isfinite(y.astype(np.float32)))
    del qw, zw, sd
    torch.cuda.empty_cache()
