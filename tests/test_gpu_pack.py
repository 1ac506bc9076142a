"""GPU packing parity: awq_pack / awq_unpack / awq_pack_zeros must be
byte-identical to the oracle's layouts."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


@pytest.mark.parametrize("K,N", [(128, 16), (4096, 4096), (384, 40), (96, 24), (8, 8), (136, 8), (11008, 64),
                                 (256, 4104)])
def test_pack_matches_oracle(awq, K, N):
    log(f"pack K={K} N={N}")
    rng = np.random.default_rng(K * 7 + N)
    q = rng.integers(0, 256, size=(K, N), dtype=np.uint8)  # high nibble must be ignored
    qw = awq.pack(to_dev(q)).cpu().numpy().view(np.uint32)
    ref = oracle.pack_device(q)
    assert qw.size == ref.size == awq.qweight_words(K, N)
    assert np.array_equal(qw, ref)
    back = awq.unpack(to_dev(ref.view(np.int32)), K, N).cpu().numpy()
    assert np.array_equal(back, q & 0xF)


@pytest.mark.parametrize("G,N", [(1, 8), (32, 4096), (7, 136), (464, 14848)])
def test_pack_zeros_matches_oracle(awq, G, N):
    log(f"pack_zeros groups={G} N={N}")
    rng = np.random.default_rng(G + N)
    z = rng.integers(0, 256, size=(G, N), dtype=np.uint8)
    zw = awq.pack_zeros(to_dev(z)).cpu().numpy().view(np.uint32)
    assert np.array_equal(zw, oracle.pack_zeros(z))


def test_empty_and_errors(awq):
    import torch
    log("pack empty/errors")
    out = awq.pack(torch.zeros((0, 16), dtype=torch.uint8, device="cuda"))
    assert out.numel() == 1
    with pytest.raises(awq.AWQError):
        awq.pack(torch.zeros((12, 16), dtype=torch.uint8, device="cuda"))
