"""GPU parity of the W4A8-FP8 path against the oracle.

* awq_quantize_act_fp8: codes and token scales bit for bit (the oracle
  decides each code in the same float32 steps), over rows that reach every
  E4M3 binade, subnormal codes, zero rows, negative zeros and fp16 subnormal
  inputs;
* awq_linear_w4a8: within 2e-3 of the oracle's fp64 value of the layer on
  the quantised activations, normalised by sum_k |x8 sx| |w|, on ragged
  shapes for both tiles, several K splits and groups of 32, 64, 128 and
  256; exactly zero for q == z."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import log, to_np16, upload_layer, x_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def unpermute(codes):
    """Kernel layout -> plain [M, K]: position 4h + j of a 128-column block
    holds the 8-column chunk 4j + h."""
    M, K = codes.shape
    return np.ascontiguousarray(codes.reshape(M, K // 128, 4, 4, 8).transpose(0, 1, 3, 2, 4).reshape(M, K))


def _rows(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-12, 4, (M, 1)))
    x[0] = 0.0                                           # zero row
    if M > 2:
        x[1] = np.exp2(rng.integers(-24, 15, K)) * rng.choice([-1, 1], K)  # every binade incl. fp16 subnormals
        x[2, :K // 2] = rng.uniform(-1e-4, 1e-4, K // 2)  # fp16 subnormals; subnormal E4M3 codes after scaling
        x[2, K // 2] = 3.0
    x = x.astype(np.float16)
    if M > 3:
        x[3, ::7] = np.float16(-0.0)
    return x


@pytest.mark.parametrize("M,K", [(1, 128), (5, 256), (33, 4096), (257, 1024), (16, 14848)])
def test_activation_codes_bitwise(awq, M, K):
    import torch
    log(f"act quant fp8 M={M} K={K}")
    x = _rows(M, K, seed=M + K)
    x8, sx = awq.quantize_act_fp8(x_dev(x))
    torch.cuda.synchronize()
    codes, s_ref = oracle.quantize_act_fp8(x)
    got = unpermute(x8.cpu().numpy())
    bad = np.argwhere(got != codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:3].tolist()}: " \
                          f"{[(int(got[tuple(b)]), int(codes[tuple(b)])) for b in bad[:3]]}"
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


SHAPES = [
    # (M, K, N, G, plan)
    (1, 128, 16, 128, None), (17, 512, 136, 128, None), (130, 1024, 264, 128, None),
    (64, 768, 72, 256, {"tile": 2}), (300, 1024, 520, 128, {"tile": 3}), (513, 640, 264, 128, {"tile": 3}),
    (130, 2048, 40, 128, {"tile": 2, "split_k": 3}), (260, 4096, 136, 256, {"tile": 3, "split_k": 5}),
    (96, 1280, 24, 128, {"tile": 3, "split_k": 2}), (2048, 1024, 256, 128, None),
    # groups of 64 and 32 (16x16x32 FP8 MFMA per 32-row block)
    (130, 1024, 264, 64, None), (300, 640, 136, 64, {"tile": 3}), (64, 768, 72, 64, {"tile": 2, "split_k": 2}),
    (96, 512, 40, 32, None), (257, 1024, 264, 32, {"tile": 3}), (130, 1280, 24, 32, {"tile": 2, "split_k": 3}),
    (512, 4608, 512, 64, None),
]


@pytest.mark.parametrize("M,K,N,G,plan", SHAPES)
def test_linear_w4a8_matches_oracle(awq, M, K, N, G, plan):
    log(f"w4a8 M={M} K={K} N={N} G={G} plan={plan} -> {awq.linear_w4a8_plan(M, K, N, G, plan)}")
    q, z, s = synth.layer(K, N, G, seed=M + K + N)
    x = synth.activations(M, K, seed=N, outlier_frac=0.01)
    qw, zw, sd = upload_layer(q, z, s)
    y = to_np16(awq.linear_w4a8(x_dev(x), qw, sd, zw, N, G, plan=plan))
    codes, sx = oracle.quantize_act_fp8(x)
    y64 = oracle.linear_w4a8_64(codes, sx, q, z, s, G)
    D = oracle.w4a8_l1_scale(codes, sx, q, z, s, G)
    yh = y.astype(np.float64)
    assert np.all(np.isfinite(yh))
    err = float(np.max(np.abs(yh - y64) / np.where(D > 0, D, 1.0)))
    assert np.all(yh[D == 0] == 0)
    assert err <= TOL, f"normalised error {err:.3e}"


def test_q_equals_z_and_zero_rows(awq):
    M, K, N, G = 40, 512, 64, 128
    log("w4a8 q == z, zero rows")
    rng = np.random.default_rng(0)
    z = rng.integers(0, 16, (K // G, N)).astype(np.uint8)
    q = np.repeat(z, G, axis=0)
    s = rng.uniform(0.001, 0.02, (K // G, N)).astype(np.float16)
    x = synth.activations(M, K, seed=1)
    qw, zw, sd = upload_layer(q, z, s)
    y = to_np16(awq.linear_w4a8(x_dev(x), qw, sd, zw, N, G)).astype(np.float64)
    assert np.all(y == 0)
    q2, z2, s2 = synth.layer(K, N, G, seed=2)
    x[5] = 0
    qw, zw, sd = upload_layer(q2, z2, s2)
    y = to_np16(awq.linear_w4a8(x_dev(x), qw, sd, zw, N, G)).astype(np.float64)
    assert np.all(y[5] == 0)


def test_w4a8_close_to_w4a16(awq):
    # The two forms of the layer on the same weights differ by the
    # activations' FP8 rounding only (2^-4 of the L1 scale at most).
    M, K, N, G = 256, 2048, 512, 128
    log("w4a8 vs w4a16")
    q, z, s = synth.layer(K, N, G, seed=9)
    x = synth.activations(M, K, seed=9)
    qw, zw, sd = upload_layer(q, z, s)
    y8 = to_np16(awq.linear_w4a8(x_dev(x), qw, sd, zw, N, G)).astype(np.float64)
    y16 = to_np16(awq.linear(x_dev(x), qw, sd, zw, N, G)).astype(np.float64)
    D = oracle.l1_scale(x, q, z, s, G)
    assert np.max(np.abs(y8 - y16) / D) <= 2.0 ** -4 + 4e-3


def test_w4a8_errors(awq):
    import torch
    log("w4a8 errors")
    q, z, s = synth.layer(320, 16, 64)
    qw, zw, sd = upload_layer(q, z, s)
    with pytest.raises(awq.AWQError):  # K must be whole 128-row steps
        awq.linear_w4a8(torch.zeros((4, 320), dtype=torch.float16, device="cuda"), qw, sd, zw, 16, 64)
    xx = torch.zeros((4, 256), dtype=torch.float16, device="cuda")
    q, z, s = synth.layer(256, 16, 128)
    qw, zw, sd = upload_layer(q, z, s)
    with pytest.raises(awq.AWQError):  # tile 1 does not exist here
        awq.linear_w4a8(xx, qw, sd, zw, 16, 128, plan={"tile": 1})
    with pytest.raises(awq.AWQError):  # more splits than 128-row steps
        awq.linear_w4a8(xx, qw, sd, zw, 16, 128, plan={"split_k": 3})


@pytest.mark.parametrize("si", range(4))
def test_w4a8_prefill_workload_sampled(awq, si):
    # The LLaMA-2-13B prefill shapes at M = 2048 (1% outlier input channels),
    # with the automatic plan the bench times; the oracle checks sampled
    # rows and columns.
    w = synth.LLAMA2_13B_PREFILL
    sh = w.shapes[si]
    M, K, N, G = 2048, sh.K, sh.N, w.G
    log(f"w4a8 workload {sh.name} M={M} K={K} N={N} plan={awq.linear_w4a8_plan(M, K, N, G)}")
    q, z, s = synth.layer(K, N, G, seed=0, layer_id=si)
    x = synth.activations(M, K, seed=0, stream=si, outlier_frac=w.outlier_frac)
    qw, zw, sd = upload_layer(q, z, s)
    y = to_np16(awq.linear_w4a8(x_dev(x), qw, sd, zw, N, G))
    rng = np.random.default_rng(si)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 126, replace=False)]))
    codes, sx = oracle.quantize_act_fp8(x[rows])
    y64 = oracle.linear_w4a8_64(codes, sx, q[:, cols], z[:, cols], s[:, cols], G)
    D = oracle.w4a8_l1_scale(codes, sx, q[:, cols], z[:, cols], s[:, cols], G)
    err = float(np.max(np.abs(y[np.ix_(rows, cols)].astype(np.float64) - y64) / D))
    assert err <= TOL, f"{sh.name}: normalised error {err:.3e}"
