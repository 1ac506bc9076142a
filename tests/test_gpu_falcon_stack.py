"""The resident Falcon-180B-shaped stack (80 layers x 4 linears, 92 GB of int4
weights) built the way the bench builds it (its own builder and seed, weights
generated on the device), checked against the oracle on its own bytes: every
layer's weights are read back with awq_unpack, its scales and packed zero
points copied to the host, and the layer's output (the automatic plan the
bench times, M = 1 and M = 16) compared with the fp64 oracle on all columns of
the first layer and 256 sampled columns of every other layer.

"Simplifying ..." / TensorRT-LLM news page: Falcon-180B with INT4 AWQ runs on
one GPU; here the whole int4 weight set is resident in one MI355X's HBM."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_close, log, to_np16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _chunked_oracle(x, q, z, s, G, max_bytes=1 << 30):
    """oracle.linear64 over contiguous K chunks of whole groups (bounded
    host memory for the fp64 dequantisation)."""
    K, N = q.shape
    rows = max(G, (max_bytes // (8 * N)) // G * G)
    y = np.zeros((x.shape[0], N))
    for k0 in range(0, K, rows):
        k1 = min(K, k0 + rows)
        y += oracle.linear64(x[:, k0:k1], q[k0:k1], z[k0 // G:k1 // G], s[k0 // G:k1 // G], G)
    return y


def test_resident_falcon180b_stack():
    import torch

    import bench
    import weight_only_bit_awq_amd as awq
    awq.library()
    wf = synth.FALCON_180B_STACK
    dev = torch.device("cuda")
    log(f"falcon stack: building {wf.layers} layers x {len(wf.shapes)} shapes as the bench does")
    layers, ws = bench.build_stack(awq, torch, wf, 1, dev, seed=4)
    total = sum(bench.weight_set_bytes(L.K, L.N, L.G) for _, L in layers)
    log(f"falcon stack: {total / 1e9:.2f} GB resident")
    assert total > 90e9
    G = wf.G
    Ms = tuple(wf.Ms)
    # one activation matrix per K with max(Ms) rows; the M-row calls use its first M rows
    xs = {K: synth.activations(max(Ms), K, seed=5, stream=K % 97) for K in {sh.K for sh in wf.shapes}}
    xd = {K: torch.from_numpy(x.view(np.uint16)).to(dev).view(torch.float16) for K, x in xs.items()}
    rng = np.random.default_rng(7)
    for li, (name, L) in enumerate(layers):
        first = li < len(wf.shapes)
        ys = {}
        for M in Ms:
            y = torch.empty((M, L.N), dtype=torch.float16, device=dev)
            Lm = L.rebound(awq, xd[L.K][:M].contiguous(), y, ws)
            Lm.launch(awq.library(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            ys[M] = y
        cols = np.arange(L.N) if first else np.unique(np.concatenate([[0, L.N - 1],
                                                                      rng.choice(L.N, 254, replace=False)]))
        ct = torch.from_numpy(cols).to(dev)
        q = awq.unpack(L.qw, L.K, L.N).index_select(1, ct).cpu().numpy()
        z = oracle.unpack_zeros(L.zw.cpu().numpy().view(np.uint32))[:, cols]
        s = L.s.cpu().numpy().view(np.float16)[:, cols]
        torch.cuda.synchronize()
        x = xs[L.K]
        y64 = _chunked_oracle(x, q, z, s, G)
        D = _l1_chunked(x, q, z, s, G)
        for M in Ms:
            yh = to_np16(ys[M])[:, cols]
            err = check_close(yh, y64[:M], D[:M], what=f"layer {li // len(wf.shapes)} {name} M={M}")
            if first or li % 40 == 0:
                log(f"  layer {li // len(wf.shapes)} {name} M={M} cols={len(cols)} plan="
                    f"{awq.linear_plan(M, L.K, L.N, G)} err={err:.2e}")
        del ys
    del layers, ws
    torch.cuda.empty_cache()


def _l1_chunked(x, q, z, s, G, max_bytes=1 << 30):
    K, N = q.shape
    rows = max(G, (max_bytes // (8 * N)) // G * G)
    D = np.zeros((x.shape[0], N))
    for k0 in range(0, K, rows):
        k1 = min(K, k0 + rows)
        D += oracle.l1_scale(x[:, k0:k1], q[k0:k1], z[k0 // G:k1 // G], s[k0 // G:k1 // G], G)
    return D
