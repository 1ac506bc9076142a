"""The seeded input generators: shapes, ranges, reproducibility."""
import numpy as np

import synth


def test_layer_shapes_ranges_repro():
    q, z, s = synth.layer(512, 64, 128, seed=0)
    assert q.shape == (512, 64) and q.dtype == np.uint8 and q.max() <= 15
    assert z.shape == (4, 64) and z.dtype == np.uint8 and z.max() <= 15
    assert s.dtype == np.float16 and s.min() >= np.float16(0.001) and s.max() <= np.float16(0.02)
    q2, z2, s2 = synth.layer(512, 64, 128, seed=0)
    assert np.array_equal(q, q2) and np.array_equal(z, z2) and np.array_equal(s, s2)
    q3, _, _ = synth.layer(512, 64, 128, seed=1)
    assert not np.array_equal(q, q3)
    _, _, sl = synth.layer(512, 64, 128, scales="loguniform", lo=1e-3, hi=3e-2)
    assert sl.min() >= np.float16(1e-3) and sl.max() <= np.float16(3e-2)
    assert set(np.unique(q)) == set(range(16))


def test_activations_and_outliers():
    x = synth.activations(4, 5120, seed=0)
    assert x.shape == (4, 5120) and x.dtype == np.float16
    assert abs(float(x.astype(np.float64).std()) - 1.0) < 0.05
    xo = synth.activations(4, 5120, seed=0, outlier_frac=0.01)
    cols = synth.outlier_channels(5120, seed=0, M=4)
    assert cols.size == 51
    assert synth.outlier_channels(13824, M=2).size == 138
    mask = np.zeros(5120, bool)
    mask[cols] = True
    assert np.array_equal(xo[:, ~mask], x[:, ~mask])
    ratio = xo[:, mask].astype(np.float64) / np.where(x[:, mask] == 0, 1, x[:, mask]).astype(np.float64)
    assert np.allclose(ratio[x[:, mask] != 0], 20, rtol=2e-3)


def test_workloads():
    assert synth.LLAMA2_7B_DECODE.layers == 32
    assert [s.N for s in synth.LLAMA2_7B_DECODE.shapes] == [12288, 4096, 22016, 4096]
    assert synth.LLAMA2_13B_PREFILL.Ms == (512, 2048)
    for w in synth.WORKLOADS:
        for s in w.shapes:
            assert s.K % w.G == 0 and s.N % 8 == 0
