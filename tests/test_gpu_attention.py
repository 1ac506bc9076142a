"""GPU parity of the fused decode-step attention (awq_attention_decode)
against the fp64 oracle: MHA, GQA and MQA head groupings, D = 64 and 128,
every rotary pairing, several work splits (one or many workgroups per unit,
one or several 32-position blocks per wave), ragged and empty caches, the
largest position a cache holds.

Checked per call: the output within the oracle's error scale (tol 2e-3); the
appended value bit for bit and the appended key within one fp16 step of the
oracle's rounding of the rotated key (the kernel rotates in fp32, the oracle
in fp64, so a key lying next to a rounding boundary may round the other way);
every other cache slot unchanged bit for bit."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import log, to_np16

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def awq():
    import weight_only_bit_awq_amd as m
    m.library()
    return m


def _inputs(B, Hq, Hkv, D, S, seed, qscale=1.0, nan_tail=False):
    rng = np.random.default_rng(seed)
    qkv = rng.standard_normal((B, (Hq + 2 * Hkv) * D))
    qkv[:, :Hq * D] *= qscale
    kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    if nan_tail:
        kc[:, :, S // 2:] = np.float16(np.nan)
        vc[:, :, S // 2:] = np.float16(np.inf)
    return qkv.astype(np.float16), kc, vc


def _dev16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint16)).view(torch.float16).cuda()


def v_to_tiles(v):
    """Logical values [B, Hkv, S, D] -> the cache layout [B, Hkv, S/32, D, 32]."""
    B, H, S, D = v.shape
    return np.ascontiguousarray(v.reshape(B, H, S // 32, 32, D).transpose(0, 1, 2, 4, 3))


def v_from_tiles(t):
    B, H, T, D, _ = t.shape
    return np.ascontiguousarray(t.transpose(0, 1, 2, 4, 3).reshape(B, H, T * 32, D))


def run_step(awq, qkv, kc, vc, lengths, Hq, Hkv, max_cached, rope, theta, steps=0, workspace=None, scale=0.0):
    """One call on device copies; returns (out [B, Hq, D], k cache, v cache
    in the logical [B, Hkv, S, D] layout) as numpy fp16."""
    import torch
    B, _, S, D = kc.shape
    kd = _dev16(kc)
    vd = _dev16(v_to_tiles(vc))
    ld = torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    out = awq.attention(_dev16(qkv), kd, vd, ld, Hq, Hkv, max_cached=max_cached, rope=rope, theta=theta,
                        scale=scale, steps=steps, workspace=workspace)
    torch.cuda.synchronize()
    return (to_np16(out).reshape(B, Hq, D), to_np16(kd), v_from_tiles(to_np16(vd)))


def check_step(qkv, kc, vc, lengths, Hq, Hkv, rope, theta, got, what, scale=None):
    out, k_after, v_after = got
    B, _, S, D = kc.shape
    y64, k_new, v_new = oracle.decode_step64(qkv, kc, vc, lengths, Hq, Hkv, D, theta, rope, scale)
    E = oracle.decode_error_scale(qkv, kc, vc, lengths, Hq, Hkv, D, theta, rope, scale)
    o = out.astype(np.float64)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = float(np.max(np.abs(o - y64) / E))
    assert err <= TOL, f"{what}: normalised error {err:.3e}"
    for b in range(B):
        L = int(lengths[b])
        keep = np.ones(S, bool)
        keep[L] = False
        assert np.array_equal(k_after[b][:, keep].view(np.uint16), kc[b][:, keep].view(np.uint16)), what
        assert np.array_equal(v_after[b][:, keep].view(np.uint16), vc[b][:, keep].view(np.uint16)), what
        assert np.array_equal(v_after[b][:, L].view(np.uint16), v_new[b].view(np.uint16)), f"{what}: value slot"
        ulp = np.abs(k_after[b][:, L].view(np.int16).astype(np.int32) - k_new[b].view(np.int16).astype(np.int32))
        assert np.all(ulp <= 1), f"{what}: key slot differs by {ulp.max()} fp16 steps"
    return err


CASES = [
    # (B, Hq, Hkv, D, lengths, S, rope, theta, steps)
    (1, 4, 4, 128, [37], 64, "half", 1e4, 0),
    (2, 8, 8, 128, [0, 100], 128, "half", 1e4, 0),
    (2, 32, 8, 128, [300, 511], 512, "half", 5e5, 0),
    (3, 12, 4, 64, [1, 31, 32], 64, "interleaved", 1e4, 0),
    (1, 71, 1, 64, [700], 1024, "half", 1e4, 0),
    (2, 20, 1, 128, [33, 65], 96, "none", 1e4, 0),
    (2, 16, 2, 64, [95, 0], 96, "half", 1e4, 1),
    (1, 32, 32, 128, [1023], 1024, "half", 1e4, 3),
    (4, 8, 2, 128, [200, 1, 129, 64], 256, "interleaved", 5e5, 2),
    (1, 40, 8, 128, [4000], 4096, "half", 5e5, 0),
    (2, 17, 1, 64, [250, 3], 256, "half", 1e4, 1),
    (1, 8, 8, 64, [31], 32, "half", 1e4, 0),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,lengths,S,rope,theta,steps", CASES)
def test_decode_step_matches_oracle(awq, B, Hq, Hkv, D, lengths, S, rope, theta, steps):
    desc = awq.attention_desc(B, Hq, Hkv, D, S, max(lengths), rope=rope, theta=theta, steps=steps)
    log(f"attention B={B} Hq={Hq} Hkv={Hkv} D={D} L={lengths} S={S} {rope} steps={steps} "
        f"plan={awq.attention_plan(desc)}")
    qkv, kc, vc = _inputs(B, Hq, Hkv, D, S, seed=B * 100 + Hq + D + S)
    got = run_step(awq, qkv, kc, vc, lengths, Hq, Hkv, max(lengths), rope, theta, steps)
    check_step(qkv, kc, vc, lengths, Hq, Hkv, rope, theta, got, f"B{B} Hq{Hq} Hkv{Hkv} D{D} {rope}")


@pytest.mark.parametrize("qscale", [4.0, 12.0])
def test_peaked_scores(awq, qscale):
    # Large scores (softmax close to one-hot) exercise the running maximum.
    B, Hq, Hkv, D, S = 2, 16, 4, 128, 256
    lengths = [255, 130]
    log(f"attention peaked qscale={qscale}")
    qkv, kc, vc = _inputs(B, Hq, Hkv, D, S, seed=7, qscale=qscale)
    got = run_step(awq, qkv, kc, vc, lengths, Hq, Hkv, 255, "half", 1e4, 1)
    check_step(qkv, kc, vc, lengths, Hq, Hkv, "half", 1e4, got, f"peaked x{qscale}")


def test_explicit_scale(awq):
    B, Hq, Hkv, D, S = 1, 8, 2, 64, 128
    log("attention explicit scale")
    qkv, kc, vc = _inputs(B, Hq, Hkv, D, S, seed=8)
    got = run_step(awq, qkv, kc, vc, [77], Hq, Hkv, 100, "half", 1e4, scale=0.05)
    check_step(qkv, kc, vc, [77], Hq, Hkv, "half", 1e4, got, "scale 0.05", scale=0.05)


def test_stale_nan_slots_do_not_leak(awq):
    # Slots at and past the cached length hold NaN keys and inf values; the
    # masked positions must not reach the output.
    B, Hq, Hkv, D, S = 2, 8, 2, 128, 128
    lengths = [40, 64]
    log("attention stale NaN/inf slots")
    qkv, kc, vc = _inputs(B, Hq, Hkv, D, S, seed=9, nan_tail=True)
    got = run_step(awq, qkv, kc, vc, lengths, Hq, Hkv, 127, "half", 1e4)
    check_step(qkv, kc, vc, lengths, Hq, Hkv, "half", 1e4, got, "NaN tail")


def test_invalid_lengths_give_nan_rows_and_keep_the_cache(awq):
    B, Hq, Hkv, D, S = 4, 8, 2, 64, 64
    lengths = [10, 50, -1, 63]  # 50 > max_cached = 40, -1 negative, 63 > max_cached
    log("attention invalid lengths")
    qkv, kc, vc = _inputs(B, Hq, Hkv, D, S, seed=10)
    out, k_after, v_after = run_step(awq, qkv, kc, vc, lengths, Hq, Hkv, 40, "half", 1e4)
    assert np.all(np.isnan(out[1:].astype(np.float32)))
    assert np.array_equal(k_after[1:].view(np.uint16), kc[1:].view(np.uint16))
    assert np.array_equal(v_after[1:].view(np.uint16), vc[1:].view(np.uint16))
    check_step(qkv[:1], kc[:1], vc[:1], lengths[:1], Hq, Hkv, "half", 1e4,
               (out[:1], k_after[:1], v_after[:1]), "valid row")


def test_generation_loop_reuses_cache_and_workspace(awq):
    # Twelve steps of generation on one cache and one workspace: each step's
    # appended key and value are read by the next steps, and the workspace's
    # counters return to zero between calls.
    import torch
    B, Hq, Hkv, D, S = 2, 16, 4, 128, 64
    log("attention generation loop")
    rng = np.random.default_rng(11)
    kc = np.zeros((B, Hkv, S, D), np.float16)
    vc = np.zeros((B, Hkv, S, D), np.float16)
    start = np.array([5, 30], np.int32)
    kc[:, :, :30] = rng.standard_normal((B, Hkv, 30, D)).astype(np.float16)
    vc[:, :, :30] = rng.standard_normal((B, Hkv, 30, D)).astype(np.float16)
    kd = _dev16(kc)
    vd = _dev16(v_to_tiles(vc))
    ws = awq.AttentionWorkspace(torch.device("cuda"))
    k_ref, v_ref = kc.copy(), vc.copy()
    for step in range(12):
        lengths = start + step
        qkv = rng.standard_normal((B, (Hq + 2 * Hkv) * D)).astype(np.float16)
        ld = torch.from_numpy(lengths).cuda()
        out = awq.attention(_dev16(qkv), kd, vd, ld, Hq, Hkv, max_cached=S - 1, rope="half", theta=1e4,
                            steps=1, workspace=ws)
        y64, k_new, v_new = oracle.decode_step64(qkv, k_ref, v_ref, lengths, Hq, Hkv, D, 1e4, "half")
        E = oracle.decode_error_scale(qkv, k_ref, v_ref, lengths, Hq, Hkv, D, 1e4, "half")
        o = to_np16(out).reshape(B, Hq, D).astype(np.float64)
        assert float(np.max(np.abs(o - y64) / E)) <= TOL, f"step {step}"
        # the device cache is the reference for the next step (its key slot
        # may differ from the oracle's rounding by one fp16 step)
        k_dev = to_np16(kd)
        for b in range(B):
            L = int(lengths[b])
            d = np.abs(k_dev[b][:, L].view(np.int16).astype(np.int32) - k_new[b].view(np.int16).astype(np.int32))
            assert np.all(d <= 1)
            k_ref[b][:, L] = k_dev[b][:, L]
            v_ref[b][:, L] = v_new[b]
    assert int(torch.count_nonzero(ws.buf[:256])) == 0  # counters back at zero


def test_errors(awq):
    import torch
    log("attention errors")
    kd, vd = awq.kv_cache(1, 2, 64, 64, "cuda")
    qkv = torch.zeros((1, 8 * 64), dtype=torch.float16, device="cuda")
    ld = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(awq.AWQError):  # max_cached must be below capacity
        awq.attention(qkv, kd, vd, ld, 4, 2, max_cached=64)
    with pytest.raises(awq.AWQError):  # Hq not a multiple of Hkv
        awq.attention(torch.zeros((1, 7 * 64), dtype=torch.float16, device="cuda"), kd, vd, ld, 3, 2)
    with pytest.raises(awq.AWQError):  # theta must be positive
        awq.attention(qkv, kd, vd, ld, 4, 2, theta=-1.0)
    k3 = torch.zeros((1, 2, 64, 96), dtype=torch.float16, device="cuda")
    with pytest.raises(awq.AWQError):  # head_dim 96 is not supported
        awq.attention(torch.zeros((1, 8 * 96), dtype=torch.float16, device="cuda"), k3,
                      torch.zeros((1, 2, 2, 96, 32), dtype=torch.float16, device="cuda"), ld, 4, 2)


@pytest.mark.parametrize("w", __import__("synth").ATTENTION_WORKLOADS, ids=lambda w: w.name)
def test_bench_workloads_sampled(awq, w):
    # The bench's workloads at full size, with the automatic work split it
    # times; the oracle checks three sequences (first, middle, last).
    import synth
    log(f"attention workload {w.name}")
    qkv, kc, vc, lengths = synth.attention_inputs(w, seed=1)
    out, k_after, v_after = run_step(awq, qkv, kc, vc, lengths, w.Hq, w.Hkv, w.L, w.rope, w.theta)
    bs = sorted({0, w.B // 2, w.B - 1})
    check_step(qkv[bs], kc[bs], vc[bs], lengths[bs], w.Hq, w.Hkv, w.rope, w.theta,
               (out[bs], k_after[bs], v_after[bs]), w.name)
    assert np.all(np.isfinite(out.astype(np.float32)))


# The bench's attention workloads (L a power of two) with L - 1 cached
# positions, so that L - 1 + 1 is a power of two; the automatic work split is
# the same as at L (the same 32-position blocks).
EXACT_WORKLOADS = [(w, w.L - 1) for w in __import__("synth").ATTENTION_WORKLOADS]


@pytest.mark.parametrize("w,L", EXACT_WORKLOADS, ids=lambda a: getattr(a, "name", str(a)))
def test_exact_case_bit_for_bit(awq, w, L):
    # Every query 0 (every probability 1/(L+1)) and odd-integer values: the
    # output is sum_j v_j / (L + 1), an fp16 number, and must equal the
    # oracle's bit for bit. A dropped, repeated or misplaced cached position,
    # a lost new token or a wrong kv head changes the bits (pinned on the CPU).
    import synth
    assert (L + 1) & L == 0
    desc = awq.attention_desc(w.B, w.Hq, w.Hkv, w.D, (L + 1 + 31) // 32 * 32, L, rope=w.rope, theta=w.theta)
    bench_desc = awq.attention_desc(w.B, w.Hq, w.Hkv, w.D, w.capacity, w.L, rope=w.rope, theta=w.theta)
    plan = awq.attention_plan(desc)
    assert plan == awq.attention_plan(bench_desc)
    log(f"attention exact {w.name} L={L} plan={plan}")
    qkv, kc, vc, lengths = synth.attention_exact_inputs(w, L, seed=2)
    out, k_after, v_after = run_step(awq, qkv, kc, vc, lengths, w.Hq, w.Hkv, L, w.rope, w.theta)
    y64, k_new, v_new = oracle.decode_step64(qkv, kc, vc, lengths, w.Hq, w.Hkv, w.D, w.theta, w.rope)
    want = y64.astype(np.float16).view(np.uint16)
    got = out.view(np.uint16)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at (b, head, d) = {tuple(bad[0])}"
    for b in (0, w.B - 1):
        assert np.array_equal(v_after[b][:, L].view(np.uint16), v_new[b].view(np.uint16))
        assert np.array_equal(v_after[b][:, :L].view(np.uint16), vc[b][:, :L].view(np.uint16))
        assert np.array_equal(k_after[b][:, :L].view(np.uint16), kc[b][:, :L].view(np.uint16))


def test_workspace_shared_across_shapes(awq):
    # One buffer for two calls: B = 1 with 4095 cached positions (32 units,
    # 16 workgroups each: the larger buffer), then B = 8 with at most 31
    # (256 units, whose counters lie where the first call's states were).
    # Both outputs against the oracle; the buffer all zero after each call.
    import torch
    ws = awq.AttentionWorkspace(torch.device("cuda"))
    for (B, lengths, S, seed) in ((1, [4095], 4096, 21), (8, [31, 0, 5, 30, 31, 17, 1, 29], 32, 22)):
        desc = awq.attention_desc(B, 32, 32, 128, S, max(lengths))
        log(f"attention shared workspace B={B} L={lengths} plan={awq.attention_plan(desc)} "
            f"ws={awq.attention_workspace_bytes(desc)} buffer={None if ws.buf is None else ws.buf.numel()}")
        qkv, kc, vc = _inputs(B, 32, 32, 128, S, seed=seed)
        got = run_step(awq, qkv, kc, vc, lengths, 32, 32, max(lengths), "half", 1e4, workspace=ws)
        check_step(qkv, kc, vc, lengths, 32, 32, "half", 1e4, got, f"shared workspace B={B}")
        assert int(torch.count_nonzero(ws.buf)) == 0, "workspace not all zero after the call"
