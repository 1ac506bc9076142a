"""GPU parity of the gated epilogue awq_linear_silu_mul (y = silu(gate) * up
on a fused gate+up layer) against the fp64 oracle, on the fused decode
kernel (staged, streamed and slab variants) and on the prefill path (split
and unsplit), with the derived error scale 1.1 |u| D_gate + |silu(g)| D_up
+ |y| and the same 2e-3 budget."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, log, to_np16, upload_layer, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def check_gated(yhat, x, q, z, s, G, what):
    y = oracle.linear_silu_mul64(x, q, z, s, G)
    E = oracle.silu_mul_scale(x, q, z, s, G)
    yh = yhat.astype(np.float64)
    assert np.all(np.isfinite(yh)), what
    diff = np.abs(yh - y)
    assert np.all(diff[E == 0] == 0), what
    err = float(np.max(diff[E > 0] / E[E > 0])) if np.any(E > 0) else 0.0
    assert err <= TOL, f"{what}: normalised error {err:.3e}"
    return err


def sampled(q, z, s, cols):
    """Columns `cols` of the gate half and the matching up columns."""
    n2 = q.shape[1] // 2
    idx = np.concatenate([cols, cols + n2])
    return q[:, idx], z[:, idx], s[:, idx]


@pytest.mark.parametrize("M,K,N,G,plan", [
    (1, 256, 64, 64, None), (4, 1216, 96, 64, None), (16, 512, 160, 32, None), (1, 2048, 2048, 128, None),
    (2, 1024, 256, 128, None), (8, 4544, 192, 64, None), (32, 1024, 544, 128, None), (20, 640, 96, 32, None),
    (4, 768, 64, 128, {"path": 1, "x_stage": 2, "waves": 8}), (3, 640, 64, 128, {"path": 1, "x_stage": 1}),
    (16, 1024, 2048, 128, {"path": 1, "x_stage": 2, "tpw": 4}), (24, 1216, 128, 64, {"path": 1, "tpw": 4}),
    (9, 512, 256, 32, {"path": 1, "x_stage": 2, "tpw": 4, "waves": 8}),
    (3, 768, 64, 128, {"path": 1, "waves": 4}), (1, 14336, 256, 128, None),
    (20, 512, 96, 128, None), (300, 1024, 544, 64, None), (130, 2304, 160, 256, {"path": 2, "split_k": 3}),
    (8, 640, 64, 128, {"path": 2}), (513, 640, 96, 128, {"path": 2, "tile": 3}),
    (257, 640, 288, 64, {"path": 2, "tile": 1}), (600, 1024, 544, 128, {"path": 2, "tile": 2}),
    (300, 4160, 96, 32, {"path": 2, "tile": 3, "split_k": 2}),
    # the streamed decode kernel with K split over workgroups
    (16, 4096, 2048, 128, {"path": 1, "x_stage": 2, "tpw": 4, "split_k": 4}),
    (32, 1216, 128, 64, {"path": 1, "tpw": 2, "waves": 8, "split_k": 3}),
    (5, 3200, 96, 32, {"path": 1, "x_stage": 2, "tpw": 2, "split_k": 16}),
    # the slab variant: gate and up tiles of each wave, with and without a K split
    (16, 1024, 2048, 128, {"path": 1, "x_stage": 3}), (32, 1280, 544, 128, {"path": 1, "x_stage": 3, "split_k": 3}),
    (5, 512, 96, 256, {"path": 1, "x_stage": 3, "tpw": 4}),
    (17, 2048, 4128, 128, {"path": 1, "x_stage": 3, "tpw": 4, "split_k": 2}),
    (24, 640, 160, 128, {"path": 1, "x_stage": 3, "split_k": 5})])
def test_gated_matches_oracle(awq, M, K, N, G, plan):
    log(f"gated M={M} K={K} N={N} G={G} plan={plan}")
    q, z, s = synth.layer(K, N, G, seed=M + K + N)
    x = synth.activations(M, K, seed=K + 3)
    qw, zw, sd = upload_layer(q, z, s)
    used = awq.linear_silu_mul_plan(M, K, N, G, plan)
    log(f"  resolved {used}")
    y = to_np16(awq.linear_silu_mul(x_dev(x), qw, sd, zw, N, G, plan=plan))
    assert y.shape == (M, N // 2)
    check_gated(y, x, q, z, s, G, f"gated {M}x{K}x{N} {used}")


def test_gated_llama_gate_up_m1(awq):
    # the LLaMA-2-7B fused gate+up layer (K=4096, N=2 x 11008) at M=1, sampled columns
    M, K, N, G = 1, 4096, 22016, 128
    log("gated llama2-7b gate_up M=1")
    q, z, s = synth.layer(K, N, G, seed=7)
    x = synth.activations(M, K, seed=7)
    qw, zw, sd = upload_layer(q, z, s)
    assert awq.linear_silu_mul_plan(M, K, N, G)["path"] == 1
    y = to_np16(awq.linear_silu_mul(x_dev(x), qw, sd, zw, N, G))
    rng = np.random.default_rng(0)
    cols = np.unique(np.concatenate([[0, N // 2 - 1], rng.choice(N // 2, 254, replace=False)]))
    qs, zs, ss = sampled(q, z, s, cols)
    check_gated(y[:, cols], x, qs, zs, ss, G, "llama gate_up sampled")


def test_gated_equals_unfused_composition(awq):
    # same weights through awq_linear (fp16 h) and silu*mul on the host: equal
    # up to the fp16 rounding of h that the fused form avoids
    M, K, N, G = 2, 1024, 256, 64
    log("gated vs unfused")
    q, z, s = synth.layer(K, N, G, seed=11)
    x = synth.activations(M, K, seed=11)
    qw, zw, sd = upload_layer(q, z, s)
    yg = to_np16(awq.linear_silu_mul(x_dev(x), qw, sd, zw, N, G)).astype(np.float64)
    h = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G)).astype(np.float64)
    yu = oracle.silu64(h[:, : N // 2]) * h[:, N // 2:]
    assert np.max(np.abs(yg - yu) / (np.abs(yu) + 1e-3)) < 5e-3


def test_gated_errors(awq):
    import torch
    log("gated errors")
    q, z, s = synth.layer(128, 48, 64, seed=1)
    qw, zw, sd = upload_layer(q, z, s)
    x = x_dev(synth.activations(1, 128, seed=1))
    with pytest.raises(awq.AWQError):
        awq.linear_silu_mul(x, qw, sd, zw, 48, 64)                 # N % 32 != 0
    with pytest.raises(awq.AWQError):
        awq.linear_silu_mul_plan(40, 128, 64, 64, {"path": 1})     # no fused decode kernel above M = 32
    assert awq.linear_silu_mul_plan(40, 128, 64, 64)["path"] == 2
    assert awq.linear_silu_mul_workspace_bytes(1, 128, 64, 64) == 0
    assert awq.linear_silu_mul_workspace_bytes(40, 128, 64, 64) == 0      # epilogue in registers
    assert awq.linear_silu_mul_workspace_bytes(130, 2304, 160, 256, {"path": 2, "split_k": 3}) == 3 * 130 * 160 * 4
