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
        # the decode path's slab variant, split (reduction kernel) and not, plain and gated
        (24, 2048, 1024, 128, {"path": 1, "x_stage": 3, "split_k": 3}, False),
        (16, 1024, 512, 128, {"path": 1, "x_stage": 3, "tpw": 1}, False),
        (32, 1280, 544, 128, {"path": 1, "x_stage": 3, "split_k": 2}, True),
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


def test_graph_replays_attention_and_w4a8(awq):
    # A generation step captured once and replayed as a serving loop would:
    # between replays eager work writes new q/k/v rows and advances the
    # sequence lengths on the device. Each replay must equal an eager call
    # from the same cache state bit for bit (outputs and appended slots), the
    # attention workspace's counters must be back at zero after every
    # replay, and a captured W4A8 call (split-K plan) must equal its eager call.
    import torch
    log("graph capture / replay: attention + w4a8")
    B, Hq, Hkv, D, S = 2, 32, 8, 128, 512
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    kc, vc = awq.kv_cache(B, Hkv, S, D, "cuda")
    kc.copy_(torch.randn(kc.shape, device="cuda", generator=gen).half())
    vc.copy_(torch.randn(vc.shape, device="cuda", generator=gen).half())
    qkv = torch.empty((B, (Hq + 2 * Hkv) * D), dtype=torch.float16, device="cuda")
    lengths = torch.tensor([100, 300], dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq * D), dtype=torch.float16, device="cuda")
    ws = awq.AttentionWorkspace(torch.device("cuda"))
    M, K, N, G = 300, 2048, 256, 128
    q, z, s = synth.layer(K, N, G, seed=70)
    qw, zw, sd = upload_layer(q, z, s)
    x8in = torch.empty((M, K), dtype=torch.float16, device="cuda")
    y8 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    plan8 = {"tile": 3, "split_k": 3}
    w8ws = torch.empty(awq.linear_w4a8_workspace_bytes(M, K, N, G, plan8), dtype=torch.uint8, device="cuda")

    def step():
        awq.attention(qkv, kc, vc, lengths, Hq, Hkv, max_cached=S - 1, rope="half", theta=500000.0, out=out,
                      workspace=ws, steps=1)
        awq.linear_w4a8(x8in, qw, sd, zw, N, G, out=y8, workspace=w8ws, plan=plan8)

    qkv.copy_(torch.randn(qkv.shape, device="cuda", generator=gen).half())
    x8in.copy_(torch.randn(x8in.shape, device="cuda", generator=gen).half())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(6):
        qkv.copy_(torch.randn(qkv.shape, device="cuda", generator=gen).half())
        x8in.copy_(torch.randn(x8in.shape, device="cuda", generator=gen).half())
        lengths += 1
        k0, v0 = kc.clone(), vc.clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), kc.clone(), vc.clone(), y8.clone())
        assert int(torch.count_nonzero(ws.buf[:256])) == 0, f"replay {rep}: counters not reset"
        kc.copy_(k0)
        vc.copy_(v0)
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "k cache", "v cache", "w4a8"), got, (out, kc, vc, y8)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: {name}"
        assert torch.isfinite(got[0].float()).all() and torch.isfinite(got[3].float()).all()
