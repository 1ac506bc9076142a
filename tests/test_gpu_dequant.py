"""GPU dequantisation parity: awq_dequant must reproduce the oracle's fp16
weights bit for bit (NaN compared as a class), over the whole input domain."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import log, to_dev, to_np16, upload_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def _bits_equal(got16, ref16):
    g = got16.view(np.uint16)
    r = ref16.view(np.uint16)
    nan_g = np.isnan(got16)
    nan_r = np.isnan(ref16)
    assert np.array_equal(nan_g, nan_r)
    assert np.array_equal(g[~nan_g], r[~nan_r])


def test_exhaustive_domain(awq):
    # All 16 codes x 16 zero points x 65536 scale bit patterns: column n has
    # scale bits n in every group, group g has zero point g, row k code k % 16.
    K, N, G = 512, 65536, 32
    log(f"dequant exhaustive K={K} N={N} G={G}")
    q = (np.arange(K) % 16).astype(np.uint8)[:, None].repeat(N, 1)
    z = np.arange(K // G, dtype=np.uint8)[:, None].repeat(N, 1)
    s = np.arange(N, dtype=np.uint16)[None, :].repeat(K // G, 0).view(np.float16)
    qw, zw, sd = upload_layer(q, z, s)
    w = to_np16(awq.dequant(qw, sd, zw, K, N, G))
    ref = oracle.dequant16(q, z, s, G)
    _bits_equal(w, ref)


@pytest.mark.parametrize("K,N,G", [(4096, 4096, 128), (384, 40, 64), (96, 24, 32), (512, 136, 256),
                                   (11008, 128, 128)])
def test_random_layers(awq, K, N, G):
    log(f"dequant K={K} N={N} G={G}")
    q, z, s = synth.layer(K, N, G, seed=3)
    qw, zw, sd = upload_layer(q, z, s)
    w = to_np16(awq.dequant(qw, sd, zw, K, N, G))
    _bits_equal(w, oracle.dequant16(q, z, s, G))
