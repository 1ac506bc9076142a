"""A decoder layer's generation step wired from the library's calls: QKV
projection -> fused attention (rotary embedding, cache append) -> O
projection -> gated gate+up (silu(gate) * up) -> down projection, the output
feeding the next layer, as the generation stage of "TinyChat: Efficient and
Lightweight Chatbot with AWQ" (section "Speed Benchmarks") runs W4A16 layers
and fused attention per token. Each stage is checked against the oracle on
the input that stage actually received (so errors do not compound), which
tests the wiring: the QKV rows as the attention's input, the attention's
[B, Hq*D] output as the O projection's activations, the gated half-width
output as the down projection's input."""
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


def test_two_layer_chain(awq):
    import torch
    B, Hq, Hkv, D, L, S = 2, 8, 2, 64, 37, 64
    H = Hq * D                    # hidden size 512
    F = 768                       # MLP width
    G = 128
    nqkv = (Hq + 2 * Hkv) * D
    rng = np.random.default_rng(3)
    layers = []
    for li in range(2):
        mats = {}
        for name, K, N in (("qkv", H, nqkv), ("o", H, H), ("gate_up", H, 2 * F), ("down", F, H)):
            q, z, s = synth.layer(K, N, G, seed=100 + 10 * li + len(mats))
            mats[name] = (q, z, s, upload_layer(q, z, s))
        kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
        vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
        kd = torch.from_numpy(kc.view(np.uint16)).cuda().view(torch.float16)
        vt = np.ascontiguousarray(vc.reshape(B, Hkv, S // 32, 32, D).transpose(0, 1, 2, 4, 3))
        vd = torch.from_numpy(vt.view(np.uint16)).cuda().view(torch.float16)
        layers.append((mats, kc, vc, kd, vd))
    lengths = np.array([L, L - 20], np.int32)
    ld = torch.from_numpy(lengths).cuda()
    x = synth.activations(B, H, seed=5)
    xd = x_dev(x)
    for li, (mats, kc, vc, kd, vd) in enumerate(layers):
        log(f"chain layer {li}")

        def lin(name, inp, gated=False):
            q, z, s, (qw, zw, sd) = mats[name]
            f = awq.linear_silu_mul if gated else awq.linear
            return f(inp, qw, sd, zw, q.shape[1], G)

        def check_lin(name, inp_dev, out_dev, gated=False):
            q, z, s, _ = mats[name]
            xin = to_np16(inp_dev)
            y = to_np16(out_dev)
            if gated:
                ref = oracle.linear_silu_mul64(xin, q, z, s, G)
                E = oracle.silu_mul_scale(xin, q, z, s, G)
                assert np.max(np.abs(y.astype(np.float64) - ref) / E) <= TOL, f"layer {li} {name}"
            else:
                check_close(y, oracle.linear64(xin, q, z, s, G), oracle.l1_scale(xin, q, z, s, G),
                            what=f"layer {li} {name}")

        qkv = lin("qkv", xd)
        check_lin("qkv", xd, qkv)
        att = awq.attention(qkv, kd, vd, ld, Hq, Hkv, max_cached=S - 1, rope="half", theta=10000.0)
        qkv_np = to_np16(qkv)
        o64, _, _ = oracle.decode_step64(qkv_np, kc, vc, lengths, Hq, Hkv, D, 10000.0, "half")
        E = oracle.decode_error_scale(qkv_np, kc, vc, lengths, Hq, Hkv, D, 10000.0, "half")
        a = to_np16(att).astype(np.float64).reshape(B, Hq, D)
        assert np.max(np.abs(a - o64) / E) <= TOL, f"layer {li} attention"
        o = lin("o", att)
        check_lin("o", att, o)
        hmid = lin("gate_up", o, gated=True)
        check_lin("gate_up", o, hmid, gated=True)
        xd = lin("down", hmid)
        check_lin("down", hmid, xd)
        assert xd.shape == (B, H)
    torch.cuda.synchronize()
    assert torch.isfinite(xd.float()).all()
