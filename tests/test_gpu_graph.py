"""The layer's calls captured in a HIP graph (as the bench replays them):
every replay, with fresh inputs written between replays by eager work, must
equal the eager calls on the same inputs bit for bit (same plans, same
kernels, fixed summation order)."""
import numpy as np
import pytest

import synth
from tests.gpu_util import log, upload_layer, x_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def test_graph_replays_match_eager(awq):
    import torch
    log("graph capture / replay")
    cases = [  # (M, K, N, G, plan, gated)
        (1, 4096, 512, 128, None, False),
        (4, 1216, 96, 64, None, False),
        (130, 2304, 160, 256, {"path": 2, "split_k": 3}, False),
        (300, 1024, 256, 128, None, False),
        (1, 1024, 256, 64, None, True),
        (130, 2304, 160, 256, {"path": 2, "split_k": 3}, True),
    ]
    layers = []
    for i, (M, K, N, G, plan, gated) in enumerate(cases):
        q, z, s = synth.layer(K, N, G, seed=50 + i)
        qw, zw, sd = upload_layer(q, z, s)
        x = x_dev(synth.activations(M, K, seed=60 + i))
        nout = N // 2 if gated else N
        y = torch.empty((M, nout), dtype=torch.float16, device="cuda")
        nbytes = (awq.linear_silu_mul_workspace_bytes if gated else awq.linear_workspace_bytes)(M, K, N, G, plan)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        layers.append((x, qw, sd, zw, N, G, plan, gated, y, ws))

    def run_all():
        for x, qw, sd, zw, N, G, plan, gated, y, ws in layers:
            f = awq.linear_silu_mul if gated else awq.linear
            f(x, qw, sd, zw, N, G, out=y, workspace=ws, plan=plan)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    for rep in range(5):
        gen.manual_seed(rep)
        for x, *_ in layers:  # eager work between replays: new activations
            x.copy_(torch.randn(x.shape, device="cuda", generator=gen).half())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [l[8].clone() for l in layers]
        run_all()
        torch.cuda.synchronize()
        for i, (l, a) in enumerate(zip(layers, got)):
            assert torch.equal(a.view(torch.int16), l[8].view(torch.int16)), f"replay {rep}, case {i}"
            assert torch.isfinite(a.float()).all()
