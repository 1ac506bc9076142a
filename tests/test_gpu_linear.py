"""GPU linear-layer parity against the fp64 oracle.

Small shapes spanning several tiles with ragged tails, both paths and several
split-K / wave plans; the exactly representable case bit for bit; q == z;
invariants (power-of-two scaling, row consistency across the path switch)."""
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


def run(awq, x, q, z, s, G, plan=None):
    qw, zw, sd = upload_layer(q, z, s)
    N = q.shape[1]
    y = awq.linear(x_dev(x), qw, sd, zw, N, G, plan=plan)
    return to_np16(y)


SHAPES = [
    # (M, K, N, G)
    (1, 128, 16, 128), (1, 4096, 4096, 128), (3, 384, 40, 64), (16, 256, 24, 32), (5, 96, 8, 32),
    (17, 512, 136, 128), (33, 1024, 64, 64), (64, 640, 48, 128), (8, 11008, 128, 128), (2, 1024, 4104, 256),
    # ragged last band (K not a multiple of 128)
    (1, 4544, 72, 64), (4, 160, 24, 32), (9, 1216, 56, 64), (1, 32, 8, 32), (20, 1184, 40, 32),
    # five 128-row bands per wave with eight waves (all in flight at once)
    (1, 5120, 256, 128), (2, 4544, 64, 32),
]


@pytest.mark.parametrize("M,K,N,G", SHAPES)
def test_decode_path(awq, M, K, N, G):
    log(f"decode M={M} K={K} N={N} G={G}")
    q, z, s = synth.layer(K, N, G, seed=M + K)
    x = synth.activations(M, K, seed=N)
    y64 = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    plans = [{"path": 1}]
    for waves in (1, 2, 4, 8, 16):
        plans.append({"path": 1, "waves": waves, "x_stage": 2})
        if waves in (4, 8):
            for tpw in (2, 4):
                plans.append({"path": 1, "waves": waves, "x_stage": 2, "tpw": tpw})
        for tpw in (1, 2):
            plans.append({"path": 1, "waves": waves, "x_stage": 1, "tpw": tpw})
    ran = 0
    for plan in plans:
        try:
            awq.linear_plan(M, K, N, G, plan)
        except awq.AWQError:
            continue  # e.g. activations too large for the LDS-staged variant
        log(f"  plan {plan}")
        check_close(run(awq, x, q, z, s, G, plan), y64, D, what=f"{plan}")
        ran += 1
    assert ran >= 6


@pytest.mark.parametrize("M,K,N,G", [(1, 128, 16, 128), (65, 256, 136, 128), (130, 384, 40, 64),
                                     (200, 96, 264, 32), (128, 1024, 128, 128), (257, 640, 72, 128),
                                     (300, 1024, 520, 256), (513, 640, 264, 128), (96, 160, 24, 32),
                                     (150, 192, 264, 64), (260, 4160, 48, 64)])
def test_prefill_path(awq, M, K, N, G):
    log(f"prefill M={M} K={K} N={N} G={G}")
    q, z, s = synth.layer(K, N, G, seed=M + K + 1)
    x = synth.activations(M, K, seed=N + 1)
    y64 = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    for tile in (0, 1, 2, 3):
        log(f"  tile {tile}")
        check_close(run(awq, x, q, z, s, G, {"path": 2, "tile": tile}), y64, D, what=f"prefill tile {tile}")


@pytest.mark.parametrize("M,K,N,G", [(130, 1024, 40, 128), (300, 2560, 264, 64), (96, 4160, 24, 32),
                                     (513, 2304, 136, 256)])
def test_prefill_split_k(awq, M, K, N, G):
    log(f"prefill split-K M={M} K={K} N={N} G={G}")
    q, z, s = synth.layer(K, N, G, seed=M + K + 2)
    x = synth.activations(M, K, seed=N + 2)
    y64 = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    for tile in (1, 2, 3):
        for split in (2, 3, 5):
            plan = {"path": 2, "tile": tile, "split_k": split}
            log(f"  plan {plan} -> {awq.linear_plan(M, K, N, G, plan)}")
            check_close(run(awq, x, q, z, s, G, plan), y64, D, what=f"{plan}")


@pytest.mark.parametrize("M,K,N,G", [(1, 4096, 256, 128), (16, 1216, 136, 64), (32, 3200, 64, 32),
                                     (5, 14336, 48, 128), (64, 1024, 96, 128), (9, 4608, 264, 256),
                                     (2, 384, 40, 128)])
def test_decode_split_k(awq, M, K, N, G):
    # the streamed decode kernel with K split over workgroups: fp32 partials
    # in the workspace, added in a fixed order by the reduction kernel
    log(f"decode split-K M={M} K={K} N={N} G={G}")
    q, z, s = synth.layer(K, N, G, seed=M + K + 3)
    x = synth.activations(M, K, seed=N + 3)
    y64 = oracle.linear64(x, q, z, s, G)
    D = oracle.l1_scale(x, q, z, s, G)
    ran = 0
    for waves in (4, 8):
        for tpw in (1, 2, 4):
            for split in (2, 3, 7, 16):
                plan = {"path": 1, "x_stage": 2, "waves": waves, "tpw": tpw, "split_k": split}
                try:
                    used = awq.linear_plan(M, K, N, G, plan)
                except awq.AWQError:
                    continue  # four tiles per workgroup need M <= 32
                log(f"  plan {plan} -> {used}")
                assert used["split_k"] == min(split, -(-K // 128)) or used["split_k"] < split
                check_close(run(awq, x, q, z, s, G, plan), y64, D, what=f"{plan}")
                ran += 1
    assert ran >= 8


def _exact_case(M, K, N, G, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    s = np.full((K // G, N), 2.0 ** -6, np.float16)
    x = np.zeros((M, K), np.float16)
    for m in range(M):
        cols = rng.choice(K, size=min(8, K), replace=False)
        x[m, cols] = rng.choice([-1.0, 1.0], size=cols.size)
    return x, q, z, s


@pytest.mark.parametrize("plan", [{"path": 1}, {"path": 1, "waves": 16, "x_stage": 1, "tpw": 2},
                                  {"path": 1, "waves": 2, "x_stage": 1, "tpw": 1},
                                  {"path": 1, "waves": 1, "x_stage": 2}, {"path": 1, "waves": 4, "x_stage": 2},
                                  {"path": 2, "tile": 1}, {"path": 2, "tile": 2}, {"path": 2, "tile": 3},
                                  {"path": 2, "tile": 2, "split_k": 3}, {"path": 2, "tile": 3, "split_k": 5},
                                  {"path": 1, "x_stage": 2, "waves": 4, "tpw": 2, "split_k": 3},
                                  {"path": 1, "x_stage": 2, "waves": 8, "tpw": 4, "split_k": 6},
                                  {"path": 1, "x_stage": 3, "tpw": 2, "split_k": 1},
                                  {"path": 1, "x_stage": 3, "tpw": 4, "split_k": 2}])
def test_exact_case_bitwise(awq, plan):
    M, K, N, G = 9, 768, 72, 128
    log(f"exact M={M} K={K} N={N} plan={plan}")
    x, q, z, s = _exact_case(M, K, N, G)
    ref = oracle.round_output16(x.astype(np.float64) @ oracle.dequant16(q, z, s, G).astype(np.float64))
    y = run(awq, x, q, z, s, G, plan)
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


def test_q_equals_z_is_zero(awq):
    M, K, N, G = 4, 512, 32, 128
    log("q == z")
    rng = np.random.default_rng(0)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    q = np.repeat(z, G, axis=0)
    s = rng.uniform(-0.02, 0.02, size=(K // G, N)).astype(np.float16)
    x = synth.activations(M, K)
    for plan in ({"path": 1}, {"path": 2}):
        y = run(awq, x, q, z, s, G, plan)
        assert np.all(y.astype(np.float64) == 0)


def test_power_of_two_scaling_bitwise(awq):
    M, K, N, G = 5, 1024, 64, 128
    log("scaling")
    q, z, s = synth.layer(K, N, G, seed=9)
    x = synth.activations(M, K, seed=9)
    x4 = (x.astype(np.float64) * 4).astype(np.float16)
    for plan in ({"path": 1}, {"path": 2}):
        y1 = run(awq, x, q, z, s, G, plan).astype(np.float64)
        y4 = run(awq, x4, q, z, s, G, plan).astype(np.float64)
        assert np.array_equal(y4, 4 * y1)


def test_rows_consistent_across_path_switch(awq):
    # M sweep 1..33 (decode path) and 65..70 (prefill path): each row must be
    # within tolerance of the oracle, and the same row computed alone by the
    # decode path agrees with the prefill path to tolerance.
    K, N, G = 512, 48, 128
    q, z, s = synth.layer(K, N, G, seed=4)
    xall = synth.activations(70, K, seed=4)
    y64 = oracle.linear64(xall, q, z, s, G)
    D = oracle.l1_scale(xall, q, z, s, G)
    for M in list(range(1, 34)) + [64, 65, 70]:
        log(f"sweep M={M}")
        y = run(awq, xall[:M], q, z, s, G)
        check_close(y, y64[:M], D[:M], what=f"M={M}")


def test_k_zero_and_errors(awq):
    import torch
    log("linear K=0 / errors")
    x = torch.zeros((3, 0), dtype=torch.float16, device="cuda")
    qw = torch.zeros(1, dtype=torch.int32, device="cuda")
    sc = torch.zeros((0, 16), dtype=torch.float16, device="cuda")
    zr = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    y = torch.full((3, 16), 7.0, dtype=torch.float16, device="cuda")
    awq.linear(x, qw, sc, zr, 16, 128, out=y)
    assert torch.all(y == 0)
    q, z, s = synth.layer(256, 16, 128)
    qw, zw, sd = upload_layer(q, z, s)
    xx = torch.zeros((1, 256), dtype=torch.float16, device="cuda")
    with pytest.raises(awq.AWQError):  # a K split needs the streamed decode variant
        awq.linear(xx, qw, sd, zw, 16, 128, plan={"path": 1, "x_stage": 1, "split_k": 2})
    with pytest.raises(awq.AWQError):  # split plan, workspace too small
        awq.linear(torch.zeros((80, 256), dtype=torch.float16, device="cuda"), qw, sd, zw, 16, 128,
                   workspace=torch.zeros(64, dtype=torch.uint8, device="cuda"), plan={"path": 2, "split_k": 2})
    with pytest.raises(awq.AWQError):
        awq.linear(xx, qw, sd, zw, 16, 128, plan={"path": 1, "waves": 32})
