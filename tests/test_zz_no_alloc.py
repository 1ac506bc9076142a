"""awq_linear_noalloc (no workspace argument; split-K partials in the
library's own 64 MiB device array) against awq_linear_ex with a caller
workspace, through the C ABI: bit for bit with the same plan (the partials
are added in a fixed order either way), within the oracle's tolerance with
its automatic plan; two calls in a row, the second smaller, so the second
reads an array the first left full of its partials; a plan whose partials
exceed the array is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_close, log, to_np16, upload_layer, x_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20
AWQ_ERR_WORKSPACE = -5


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def _call_noalloc(awq, x, qw, sd, zw, N, G, out, plan):
    import torch
    lib = awq.library()
    M, K = x.shape
    p = awq._plan(plan)
    st = lib.awq_linear_noalloc(x.data_ptr(), qw.data_ptr(), sd.data_ptr(), zw.data_ptr(), M, K, N, G,
                                out.data_ptr(), ctypes.byref(p) if p else None,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _layer(M, K, N, G, seed):
    q, z, s = synth.layer(K, N, G, seed=seed)
    x = synth.activations(M, K, seed=seed)
    return x, q, z, s


def test_noalloc_matches_linear_two_calls(awq):
    import torch
    # (M, K, N, G, plan): the first call's partials fill 62.9 MB of the
    # array; each later one is smaller and runs on what the others left behind.
    cases = [(512, 5120, 5120, 128, {"path": 2, "tile": 3, "split_k": 6}),
             (300, 1024, 1000, 128, {"path": 2, "tile": 2, "split_k": 2}),
             # the decode path's slab variant with a K split, on what the
             # prefill calls left in the array
             (24, 4096, 2056, 128, {"path": 1, "x_stage": 3, "split_k": 3})]
    for (M, K, N, G, plan) in cases:
        need = awq.linear_workspace_bytes(M, K, N, G, plan)
        assert 0 < need <= SCRATCH_BYTES
        log(f"noalloc M={M} K={K} N={N} G={G} plan={plan} partials={need}")
        x, q, z, s = _layer(M, K, N, G, seed=M + N)
        qw, zw, sd = upload_layer(q, z, s)
        xd = x_dev(x)
        y_ref = awq.linear(xd, qw, sd, zw, N, G, plan=plan)
        y_na = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        assert _call_noalloc(awq, xd, qw, sd, zw, N, G, y_na, plan) == 0
        torch.cuda.synchronize()
        a, b = to_np16(y_ref), to_np16(y_na)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "differs from awq_linear_ex with the same plan"
        check_close(b, oracle.linear64(x, q, z, s, G), oracle.l1_scale(x, q, z, s, G), what=f"noalloc M={M}")


def test_noalloc_automatic_plan_fits_the_array(awq):
    import torch
    # awq_linear's automatic plan for this layer (the LLaMA-2-13B down
    # projection at 2048 rows) splits K three ways (126 MB of partials); the
    # no-alloc call lowers the split until they fit.
    M, K, N, G = 2048, 13824, 5120, 128
    auto = awq.linear_plan(M, K, N, G)
    assert awq.linear_workspace_bytes(M, K, N, G) > SCRATCH_BYTES
    log(f"noalloc automatic M={M} K={K} N={N} awq_linear plan={auto}")
    x, q, z, s = _layer(M, K, N, G, seed=5)
    qw, zw, sd = upload_layer(q, z, s)
    xd = x_dev(x)
    y_ref = awq.linear(xd, qw, sd, zw, N, G)
    y_na = torch.empty((M, N), dtype=torch.float16, device="cuda")
    assert _call_noalloc(awq, xd, qw, sd, zw, N, G, y_na, None) == 0
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 64, replace=False)
    yr, yn = to_np16(y_ref)[rows], to_np16(y_na)[rows]
    y64 = oracle.linear64(x[rows], q, z, s, G)
    D = oracle.l1_scale(x[rows], q, z, s, G)
    check_close(yr, y64, D, what="awq_linear")
    check_close(yn, y64, D, what="awq_linear_noalloc")
    # an explicit split whose partials exceed the array is refused
    big = {"path": 2, "tile": 3, "split_k": 6}
    assert awq.linear_workspace_bytes(M, K, N, G, big) > SCRATCH_BYTES
    assert _call_noalloc(awq, xd, qw, sd, zw, N, G, y_na, big) == AWQ_ERR_WORKSPACE


def test_noalloc_decode_plan(awq):
    import torch
    # decode plans use no partials: the same kernel and bits as awq_linear
    M, K, N, G = 4, 4096, 4096, 128
    log("noalloc decode M=4")
    x, q, z, s = _layer(M, K, N, G, seed=9)
    qw, zw, sd = upload_layer(q, z, s)
    xd = x_dev(x)
    y_ref = awq.linear(xd, qw, sd, zw, N, G)
    y_na = torch.empty((M, N), dtype=torch.float16, device="cuda")
    assert _call_noalloc(awq, xd, qw, sd, zw, N, G, y_na, None) == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_np16(y_ref).view(np.uint16), to_np16(y_na).view(np.uint16))
