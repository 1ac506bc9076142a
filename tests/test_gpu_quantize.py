"""GPU parity of the round-to-nearest group quantiser: awq_quantize must give
the oracle's codes (as device-layout words), fp16 scale bits and packed zero
points exactly, padding included, on random weights and on the method's
special cases (constant groups, groups that do not contain 0, tiny ranges,
quotients exactly half-way between two codes)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_close, log, to_dev, to_np16, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def with_special_groups(w, G, seed):
    """Overwrite a few (group, column) blocks with the quantiser's special
    cases; the rest stays N(0, 0.02)."""
    w = w.copy()
    K, N = w.shape
    rng = np.random.default_rng(seed)
    cols = rng.permutation(N)
    groups = K // G
    cases = []
    for i, c in enumerate(cols[: min(N, 7)]):
        g = int(rng.integers(groups))
        rows = slice(g * G, (g + 1) * G)
        kind = i % 7
        if kind == 0:
            w[rows, c] = 0.0                                    # all zero: range 0
        elif kind == 1:
            w[rows, c] = np.float16(0.75)                       # constant, positive
        elif kind == 2:
            w[rows, c] = np.abs(w[rows, c]) + np.float16(0.01)  # all positive: zero point clamps at 0
        elif kind == 3:
            w[rows, c] = -np.abs(w[rows, c]) - np.float16(0.01)  # all negative: zero point clamps at 15
        elif kind == 4:
            w[rows, c] = np.float16(2.0 ** -20) * rng.integers(-3, 4, size=G)  # range ~ subnormal scale
        elif kind == 5:
            # exact grid with s = 2^-7 and z = 6, with half-way values
            codes = rng.integers(0, 16, size=G).astype(np.float64)
            codes[0], codes[1] = 0, 15
            halves = rng.permutation(np.arange(2, G))[: G // 4]
            codes[halves] = rng.integers(0, 15, size=halves.size) + 0.5
            w[rows, c] = ((codes - 6) * 2.0 ** -7).astype(np.float16)
        else:
            w[rows, c] = rng.normal(0, 3.0, size=G).astype(np.float16)  # wide range
        cases.append((kind, g, int(c)))
    return w, cases


def quantize_and_compare(awq, w, G):
    import torch
    K, N = w.shape
    wd = to_dev(w.view(np.uint16)).view(torch.float16)
    qw, s, zw = awq.quantize(wd, G)
    q_o, z_o, s_o = oracle.quantize_rtn(w, G)
    qw_h = qw.cpu().numpy().view(np.uint32)
    ref = oracle.pack_device(q_o)
    assert qw_h.size == ref.size
    bad = np.nonzero(qw_h != ref)[0]
    assert bad.size == 0, f"{bad.size} device words differ, first at {bad[:5]}"
    assert np.array_equal(to_np16(s).view(np.uint16), s_o.view(np.uint16))
    assert np.array_equal(zw.cpu().numpy().view(np.uint32), oracle.pack_zeros(z_o))
    return qw, s, zw, (q_o, z_o, s_o)


@pytest.mark.parametrize("K,N,G", [(128, 16, 32), (192, 24, 64), (256, 40, 128), (512, 64, 256), (384, 8, 128),
                                   (1024, 200, 64), (4096, 4096, 128), (4544, 4672, 64)])
def test_quantize_matches_oracle(awq, K, N, G):
    log(f"quantize K={K} N={N} G={G}")
    w, cases = with_special_groups(synth.dense_weights(K, N, seed=K + N + G), G, seed=G + N)
    quantize_and_compare(awq, w, G)


def test_quantize_ties_everywhere(awq):
    # every weight half-way between two codes: the exact-quotient branch
    log("quantize ties")
    G, K, N = 64, 256, 64
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 15, size=(K, N)) + 0.5
    for g in range(K // G):
        codes[g * G, :] = 0
        codes[g * G + 1, :] = 15
    z = rng.integers(0, 16, size=(K // G, N))
    e = rng.integers(5, 12, size=(K // G, N))
    w = ((codes - np.repeat(z, G, 0)) * np.ldexp(1.0, -np.repeat(e, G, 0))).astype(np.float16)
    quantize_and_compare(awq, w, G)


def test_quantize_then_linear(awq):
    # the quantiser's output drives awq_linear directly
    import torch
    log("quantize then linear")
    K, N, G, M = 1024, 512, 128, 4
    w = synth.dense_weights(K, N, seed=9)
    qw, s, zw, (q_o, z_o, s_o) = quantize_and_compare(awq, w, G)
    x = synth.activations(M, K, seed=9)
    y = awq.linear(x_dev(x), qw, s, zw, N, G)
    torch.cuda.synchronize()
    check_close(to_np16(y), oracle.linear64(x, q_o, z_o, s_o, G), oracle.l1_scale(x, q_o, z_o, s_o, G),
                what="quantize->linear")


def test_quantize_errors(awq):
    import torch
    log("quantize errors")
    with pytest.raises(awq.AWQError):
        awq.quantize(torch.zeros((100, 16), dtype=torch.float16, device="cuda"), 64)  # K % G
    with pytest.raises(awq.AWQError):
        awq.quantize(torch.zeros((128, 12), dtype=torch.float16, device="cuda"), 128)  # N % 8
    qw, s, zw = awq.quantize(torch.zeros((0, 16), dtype=torch.float16, device="cuda"), 128)
    assert s.numel() == 0
