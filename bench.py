#!/usr/bin/env python3
"""Benchmark of the W4A16 group-quantised linear layer on one MI355X.

Headline (one JSON line on stdout): weight GB/s of the decode path at M=1 over
a LLaMA-2-7B-shaped decode stack -- 32 layers of fused QKV (4096x12288), O
(4096x4096), fused gate+up (4096x22016) and down (11008x4096), group 128,
random-init int4 weights resident in HBM, one fixed activation row per K --
streamed back to back. One step = the 128 linear calls of one pass over the
stack, replayed from a HIP graph; the weight set (3.36 GB) is far larger than
the 256 MB last-level cache, so every step reads cold weights.

Also reported: the prefill GEMM in TFLOP/s at M=2048 (and 512) on
LLaMA-2-13B-shaped layers, per-kernel durations from HIP events recorded at the
kernels' own start and end, a roofline entry for the dominant kernel, and the
plain fp64 CPU oracle timed on a bounded sample of the same workload.

The decode-generation context for this layer is "TinyChat: Efficient and
Lightweight Chatbot with AWQ", section "Speed Benchmarks" (per-token latency of
the generation stage with a W4A16 kernel); the byte accounting follows
"Applied LLM Quantisation Sagemaker", section "How does it help?".
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, vendor figure
FP8_DENSE_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, vendor figure
KERNEL_SOURCES = {
    "quantize": os.path.join(ROOT, "weight_only_bit_awq_amd", "csrc", "awq_quant.hip"),
    "decode": os.path.join(ROOT, "weight_only_bit_awq_amd", "csrc", "awq_decode.hip"),
    "prefill": os.path.join(ROOT, "weight_only_bit_awq_amd", "csrc", "awq_prefill.hip"),
    "attention": os.path.join(ROOT, "weight_only_bit_awq_amd", "csrc", "awq_attention.hip"),
    "w4a8": os.path.join(ROOT, "weight_only_bit_awq_amd", "csrc", "awq_w4a8.hip"),
}


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_set_bytes(K, N, G):
    """4-bit codes + fp16 scales + 4-bit zero points (0.5195 B/weight at G=128)."""
    return K * N // 2 + 2 * N * (K // G) + N * (K // G) // 2


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


class HipEvents:
    """hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            evs.append(e)
        return evs

    def elapsed_ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


class Layer:
    """One quantised linear layer resident on the GPU, with pre-bound C-ABI
    arguments (raw pointers) so launch overhead stays out of the way."""

    def __init__(self, awq, torch, K, N, G, gen, x, y, ws, dev, plan=None, scales=(0.001, 0.02)):
        q = torch.randint(0, 16, (K, N), dtype=torch.uint8, device=dev, generator=gen)
        self.qw = awq.pack(q)
        del q
        z = torch.randint(0, 16, (K // G, N), dtype=torch.uint8, device=dev, generator=gen)
        self.zw = awq.pack_zeros(z)
        del z
        self.s = torch.empty((K // G, N), dtype=torch.float32, device=dev).uniform_(*scales, generator=gen).half()
        self.K, self.N, self.G = K, N, G
        self.M = x.shape[0]
        self.x, self.y = x, y
        self.plan = awq._plan(plan) if plan is not None else None
        nbytes = awq.linear_workspace_bytes(self.M, K, N, G, self.plan)
        buf = ws.get(nbytes) if nbytes else None
        self.ws_ptr = buf.data_ptr() if buf is not None else None
        self.ws_len = buf.numel() if buf is not None else 0
        self.args = (x.data_ptr(), self.qw.data_ptr(), self.s.data_ptr(), self.zw.data_ptr(), self.M, K, N, G,
                     y.data_ptr(), self.ws_ptr, self.ws_len)

    def rebound(self, awq, x, y, ws):
        """The same weights with other activation / output buffers (M rows)."""
        other = object.__new__(Layer)
        other.__dict__.update(self.__dict__)
        other.M = x.shape[0]
        other.x, other.y = x, y
        nbytes = awq.linear_workspace_bytes(other.M, self.K, self.N, self.G, self.plan)
        buf = ws.get(nbytes) if nbytes else None
        other.ws_ptr = buf.data_ptr() if buf is not None else None
        other.ws_len = buf.numel() if buf is not None else 0
        other.args = (x.data_ptr(), self.qw.data_ptr(), self.s.data_ptr(), self.zw.data_ptr(), other.M, self.K,
                      self.N, self.G, y.data_ptr(), other.ws_ptr, other.ws_len)
        return other

    def launch(self, lib, stream):
        st = lib.awq_linear_ex(*self.args, ctypes.byref(self.plan) if self.plan else None, stream)
        if st:
            raise RuntimeError(f"awq_linear failed: {lib.awq_status_string(st).decode()}")

    def launch_timed(self, lib, stream, e0, e1):
        st = lib.awq_linear_timed(*self.args, ctypes.byref(self.plan) if self.plan else None, stream, e0, e1)
        if st:
            raise RuntimeError(f"awq_linear_timed failed: {lib.awq_status_string(st).decode()}")


def build_stack(awq, torch, workload, M, dev, seed, plan=None, layers=None):
    import synth  # noqa: F401
    G = workload.G
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    ws = awq.Workspace(dev)
    xs, ys = {}, {}
    for sh in workload.shapes:
        if sh.K not in xs:
            xs[sh.K] = torch.randn((M, sh.K), dtype=torch.float32, device=dev, generator=gen).half()
        ys[sh.name] = torch.empty((M, sh.N), dtype=torch.float16, device=dev)
    # the workspace is sized for the largest need before any pointer is taken
    need = max(awq.linear_workspace_bytes(M, sh.K, sh.N, G, plan) for sh in workload.shapes)
    ws.get(need)
    lay = []
    for li in range(layers or workload.layers):
        for sh in workload.shapes:
            lay.append((sh.name, Layer(awq, torch, sh.K, sh.N, G, gen, xs[sh.K], ys[sh.name], ws, dev, plan,
                                       (workload.lo, workload.hi))))
    torch.cuda.synchronize()
    return lay, ws


def per_kernel_times(lib, torch, hip, layers, reps):
    """Eager pass: every call launched through hipExtLaunchKernelGGL with
    events at the kernel's own start and end; returns {shape: [ms, ...]}."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # one untimed pass first: a kernel's first launch in the process loads
    # its code, which must not land in a timed call
    for _, L in layers:
        L.launch(lib, stream)
    torch.cuda.synchronize()
    n = len(layers) * reps
    evs = hip.create(2 * n)
    i = 0
    for _ in range(reps):
        for name, L in layers:
            L.launch_timed(lib, stream, evs[2 * i], evs[2 * i + 1])
            i += 1
    torch.cuda.synchronize()
    out = {}
    i = 0
    for _ in range(reps):
        for name, L in layers:
            out.setdefault(name, []).append(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]))
            i += 1
    return out


def time_stack_graph(lib, torch, layers, steps, warmup):
    """Capture one pass over the stack (every launch, in order, on one
    stream) in a HIP graph and replay it: wall-clock and event ms per step,
    K steps between two synchronisations."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        s = ctypes.c_void_p(side.cuda_stream)
        for _, L in layers:
            L.launch(lib, s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for _, L in layers:
            L.launch(lib, s)
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del graph
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def per_shape_stats(awq, lib, torch, hip, wl, layers, M, reps):
    """Per layer shape: kernel durations from events at the kernels' own
    start and end (eager pass), weight and algorithmic GB/s, the plan."""
    times = per_kernel_times(lib, torch, hip, layers, reps)
    per_shape = {}
    for sh in wl.shapes:
        ts = sorted(times[sh.name])
        avg = sum(ts) / len(ts)
        wb = weight_set_bytes(sh.K, sh.N, wl.G)
        alg = wb + 2 * M * sh.K + 2 * M * sh.N
        per_shape[sh.name] = {
            "K": sh.K, "N": sh.N, "launches": len(ts), "avg_us": round(avg * 1e3, 3),
            "p10_us": round(ts[len(ts) // 10] * 1e3, 3), "p90_us": round(ts[(9 * len(ts)) // 10] * 1e3, 3),
            "weight_GBps": round(wb / (avg / 1e3) / 1e9, 1), "alg_GBps": round(alg / (avg / 1e3) / 1e9, 1),
            "plan": awq.linear_plan(M, sh.K, sh.N, wl.G),
        }
    return per_shape


def stream_read_times(lib, torch, hip, layers, reps):
    """Plain streaming read (awq_stream_read) of each layer's qweight buffer,
    cycling through the stack so every read is cold: the achievable HBM read
    rate at that size. Returns {shape: (bytes, [ms, ...])}."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.empty(16, dtype=torch.uint8, device=layers[0][1].qw.device)
    n = len(layers) * reps
    evs = hip.create(2 * n)
    i = 0
    for _ in range(reps):
        for name, L in layers:
            nb = L.qw.numel() * L.qw.element_size()
            st = lib.awq_stream_read(L.qw.data_ptr(), nb, sink.data_ptr(), stream, evs[2 * i], evs[2 * i + 1])
            if st:
                raise RuntimeError(f"awq_stream_read failed: {lib.awq_status_string(st).decode()}")
            i += 1
    torch.cuda.synchronize()
    out = {}
    i = 0
    for _ in range(reps):
        for name, L in layers:
            nb = L.qw.numel() * L.qw.element_size()
            out.setdefault(name, (nb, []))[1].append(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]))
            i += 1
    return out


def fp16_dense_times(torch, shapes, M, dev, reps=20, copies=4):
    """The same layer shapes as a plain fp16 linear layer (torch's
    F.linear on a dense fp16 weight in its [N, K] layout, i.e. the vendor
    BLAS): the W16A16 counterpart of the W4A16 layer. Weights rotate over
    `copies` copies. Returns {shape: median ms}."""
    import torch.nn.functional as F
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    out = {}
    for name, K, N in shapes:
        x = torch.randn((M, K), device=dev, generator=gen).half()
        ws = [torch.randn((N, K), device=dev, generator=gen).half() for _ in range(copies)]
        for w in ws:
            F.linear(x, w)
        torch.cuda.synchronize()
        ts = []
        for r in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            F.linear(x, ws[r % copies])
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        out[name] = ts[len(ts) // 2]
        del ws
        torch.cuda.empty_cache()
    return out


def gated_times(awq, lib, torch, hip, K, N, G, M, dev, copies, reps):
    """Fused gate+up with the silu(gate) * up epilogue (awq_linear_silu_mul,
    events at its kernels' own start and end) against the unfused sequence:
    awq_linear writing [M, N] fp16, then torch's silu and multiply on the two
    halves (a graph of 20 repetitions of those two, per repetition). Weights
    rotate over `copies` layers. Returns medians in microseconds."""
    import torch.nn.functional as F
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    x = torch.randn((M, K), device=dev, generator=gen).half()
    h = torch.empty((M, N), dtype=torch.float16, device=dev)
    yg = torch.empty((M, N // 2), dtype=torch.float16, device=dev)
    ws = awq.Workspace(dev)
    layers = [Layer(awq, torch, K, N, G, gen, x, h, ws, dev) for _ in range(copies)]
    nb = awq.linear_silu_mul_workspace_bytes(M, K, N, G)
    buf = ws.get(max(nb, awq.linear_workspace_bytes(M, K, N, G)))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # The fused and the plain call alternate, layer by layer, so that both
    # run in the same thermal and power state of the chip (timed one after
    # the other, the same kernels differed by up to 8%); the first pass is
    # untimed (it loads the kernels' code).
    evs = hip.create(4 * reps * copies)
    fused, lin, elt = [], [], []
    for r in range(reps + 1):
        for i, L in enumerate(layers):
            e = 4 * ((r % reps) * copies + i)
            st = lib.awq_linear_silu_mul_ex(x.data_ptr(), L.qw.data_ptr(), L.s.data_ptr(), L.zw.data_ptr(), M, K, N,
                                            G, yg.data_ptr(), buf.data_ptr() if buf is not None else None,
                                            buf.numel() if buf is not None else 0, None, stream, evs[e], evs[e + 1])
            if st:
                raise RuntimeError(lib.awq_status_string(st).decode())
            L.launch_timed(lib, stream, evs[e + 2], evs[e + 3])
        torch.cuda.synchronize()
        if r:
            for i in range(copies):
                e = 4 * ((r % reps) * copies + i)
                fused.append(hip.elapsed_ms(evs[e], evs[e + 1]))
                lin.append(hip.elapsed_ms(evs[e + 2], evs[e + 3]))
    # torch's silu and multiply captured in a graph and replayed, so that the
    # host's launch latency stays out of the per-call time
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.mul(F.silu(h[:, : N // 2]), h[:, N // 2:], out=yg)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(20):
            torch.mul(F.silu(h[:, : N // 2]), h[:, N // 2:], out=yg)
    torch.cuda.synchronize()
    for r in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        elt.append(e0.elapsed_time(e1) / 20)
    del g
    med = lambda t: sorted(t)[len(t) // 2] * 1e3
    out = {"K": K, "N": N, "M": M, "fused_us": round(med(fused), 2), "linear_us": round(med(lin), 2),
           "torch_silu_mul_us": round(med(elt), 2)}
    out["unfused_us"] = round(out["linear_us"] + out["torch_silu_mul_us"], 2)
    out["plan"] = awq.linear_silu_mul_plan(M, K, N, G)
    del layers
    torch.cuda.empty_cache()
    return out


def decode_sweep(awq, lib, torch, hip, wl, dev, seed, layers=8, reps=3):
    """Batched decode on the LLaMA-3-8B-shaped layers: for each M, the four
    shapes' kernels (events at their own start and end) over `layers` copies
    of each, cold weights; weight GB/s and TFLOP/s of one layer's four calls.
    Also the same `layers` layers captured in one HIP graph and replayed
    (graph_*): a plan of two launches (K split, then the reduction) costs
    less between its kernels there than eagerly."""
    out = {}
    for M in wl.Ms:
        stack, _ = build_stack(awq, torch, wl, M, dev, seed, layers=layers)
        t = per_kernel_times(lib, torch, hip, stack, reps)
        _, graph_ms = time_stack_graph(lib, torch, stack, 20, 3)
        layer_ms = sum(sum(v) / len(v) for v in t.values())
        wb = sum(weight_set_bytes(sh.K, sh.N, wl.G) for sh in wl.shapes)
        fl = sum(2.0 * M * sh.K * sh.N for sh in wl.shapes)
        per_shape = {}
        for sh in wl.shapes:
            us = sum(t[sh.name]) / len(t[sh.name]) * 1e3
            per_shape[sh.name] = {"avg_us": round(us, 2),
                                  "weight_GBps": round(weight_set_bytes(sh.K, sh.N, wl.G) / us / 1e3, 1),
                                  "plan": awq.linear_plan(M, sh.K, sh.N, wl.G),
                                  "traffic": traffic_set_entry(f"{wl.name}/{sh.name}@M={M}")}
        glayer_ms = graph_ms / layers
        out[f"M={M}"] = {"layer_us": round(layer_ms * 1e3, 2), "weight_GBps": round(wb / (layer_ms / 1e3) / 1e9, 1),
                         "TFLOPs": round(fl / (layer_ms / 1e3) / 1e12, 2),
                         "graph_layer_us": round(glayer_ms * 1e3, 2),
                         "graph_weight_GBps": round(wb / (glayer_ms / 1e3) / 1e9, 1), "per_shape": per_shape}
        del stack
        torch.cuda.empty_cache()
    return out


def quantize_times(awq, torch, shapes, G, dev, reps=10):
    """awq_quantize (fp16 W -> device qweight, scales, zeros) on each shape,
    per call from a graph of `reps` calls; HBM bytes per call = 2 B per
    weight read + the quantised weight set written. Returns {shape: {...}}."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    out = {}
    for name, K, N in shapes:
        ws = [(torch.randn((K, N), device=dev, generator=gen) * 0.02).half() for _ in range(2)]
        for w in ws:
            awq.quantize(w, G)
        torch.cuda.synchronize()
        # `reps` calls captured in a graph and replayed between two events:
        # per-call time without the host's launch latency
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            awq.quantize(ws[0], G)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(reps):
                awq.quantize(ws[r % 2], G)
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps)
        del g
        ts.sort()
        med = ts[len(ts) // 2]
        nbytes = 2 * K * N + weight_set_bytes(K, N, G)
        out[name] = {"K": K, "N": N, "median_us": round(med * 1e3, 2), "hbm_bytes": nbytes,
                     "GBps": round(nbytes / (med / 1e3) / 1e9, 1)}
        del ws
        torch.cuda.empty_cache()
    return out


def attention_bytes(w):
    """Algorithmic HBM bytes of one decode-step attention call: every cached
    key and value read once (2 x 2 x D bytes per cached token and kv head),
    the qkv rows read, the output written, the new key and value written."""
    return (4 * w.D * w.Hkv * w.B * w.L + 2 * w.B * (w.Hq + 2 * w.Hkv) * w.D + 2 * w.B * w.Hq * w.D
            + 4 * w.B * w.Hkv * w.D)


def attention_copies(w):
    """Cache copies cycled through so that the calls read cold HBM: enough to
    span 512 MiB (twice the last-level cache), at most 1024."""
    n = w.B * w.Hkv * w.capacity * w.D
    return max(1, min(1024, -(-(512 << 20) // (4 * n))))


def attention_times(awq, lib, torch, hip, workloads, dev, reps=5):
    """awq_attention_decode on each workload, from events at the kernel's own
    start and end, cycling over enough copies of the caches (each copy one
    buffer) that every call reads cold HBM; beside
    it a plain streaming read of the same number of bytes from the same
    buffers (keys, then values in tiles of 32 positions). Returns {name: {...}}."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    out = {}
    for w in workloads:
        S = w.capacity
        n = w.B * w.Hkv * S * w.D
        nbytes = attention_bytes(w)
        R = attention_copies(w)
        bufs = [torch.randn(2 * n, device=dev, generator=gen).half() for _ in range(R)]
        kv = [(b[:n].view(w.B, w.Hkv, S, w.D), b[n:].view(w.B, w.Hkv, S // 32, w.D, 32)) for b in bufs]
        qkv = torch.randn((w.B, (w.Hq + 2 * w.Hkv) * w.D), device=dev, generator=gen).half()
        lengths = torch.full((w.B,), w.L, dtype=torch.int32, device=dev)
        y = torch.empty((w.B, w.Hq * w.D), dtype=torch.float16, device=dev)
        desc = awq.attention_desc(w.B, w.Hq, w.Hkv, w.D, S, w.L, rope=w.rope, theta=w.theta)
        wsb = awq.AttentionWorkspace(dev).get(awq.attention_workspace_bytes(desc))
        sink = torch.empty(16, dtype=torch.uint8, device=dev)
        sr_bytes = min(nbytes, 4 * n) // 16 * 16

        def call(i, e0=None, e1=None):
            k, v = kv[i % R]
            st = lib.awq_attention_decode_timed(ctypes.byref(desc), qkv.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                lengths.data_ptr(), y.data_ptr(), wsb.data_ptr(), wsb.numel(),
                                                stream, e0, e1)
            if st:
                raise RuntimeError(f"awq_attention_decode failed: {lib.awq_status_string(st).decode()}")

        for i in range(R):
            call(i)
        torch.cuda.synchronize()
        evs = hip.create(2 * R * reps)
        for i in range(R * reps):
            call(i, evs[2 * i], evs[2 * i + 1])
        sevs = hip.create(2 * R * reps)
        for i in range(R * reps):
            st = lib.awq_stream_read(bufs[i % R].data_ptr(), sr_bytes, sink.data_ptr(), stream, sevs[2 * i],
                                     sevs[2 * i + 1])
            if st:
                raise RuntimeError("awq_stream_read failed")
        torch.cuda.synchronize()
        ts = sorted(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(R * reps))
        ss = sorted(hip.elapsed_ms(sevs[2 * i], sevs[2 * i + 1]) for i in range(R * reps))
        med, smed = ts[len(ts) // 2], ss[len(ss) // 2]
        gbps = nbytes / (med / 1e3) / 1e9
        sr_gbps = sr_bytes / (smed / 1e3) / 1e9
        out[w.name] = {
            "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "cached": w.L, "rope": w.rope, "theta": w.theta,
            "launches": len(ts), "cache_copies": R, "median_us": round(med * 1e3, 3),
            "p10_us": round(ts[len(ts) // 10] * 1e3, 3), "p90_us": round(ts[(9 * len(ts)) // 10] * 1e3, 3),
            "alg_bytes": nbytes, "GBps": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBS, 2),
            "stream_read_GBps_same_size": round(sr_gbps, 1), "pct_of_stream_read": round(100 * gbps / sr_gbps, 1),
            "plan": awq.attention_plan(desc),
        }
        del bufs, kv, wsb
        torch.cuda.empty_cache()
    return out


def decode_chain(awq, lib, torch, hip, dev, steps, warmup, n_layers=32, B=1, L=1024, seed=11):
    """One generation step of a LLaMA-2-7B-shaped decoder (hidden 4096, 32
    heads of 128, MLP 11008, group 128) through the library's calls, each
    output feeding the next call: QKV projection -> fused attention (rotary
    embedding, append to the layer's cache, L tokens cached) -> O projection
    -> gated gate+up (silu(gate) * up) -> down projection -> next layer.
    RMSNorm, residual adds, embedding and LM head are not part of it. The
    step is captured in a HIP graph and replayed (per-token latency); an
    eager pass with kernel events splits it into linears and attention."""
    Hq = Hkv = 32
    D, Hd, F, G = 128, 4096, 11008, 128
    S = (L + 1 + 31) // 32 * 32
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = awq.Workspace(dev)
    xs = [torch.randn((B, Hd), device=dev, generator=gen).half() for _ in range(2)]
    qkv = torch.empty((B, (Hq + 2 * Hkv) * D), dtype=torch.float16, device=dev)
    att = torch.empty((B, Hq * D), dtype=torch.float16, device=dev)
    oo = torch.empty((B, Hd), dtype=torch.float16, device=dev)
    hh = torch.empty((B, F), dtype=torch.float16, device=dev)
    lengths = torch.full((B,), L, dtype=torch.int32, device=dev)
    desc = awq.attention_desc(B, Hq, Hkv, D, S, L, rope="half", theta=10000.0)
    aws = awq.AttentionWorkspace(dev).get(awq.attention_workspace_bytes(desc))
    gu_bytes = awq.linear_silu_mul_workspace_bytes(B, Hd, 2 * F, G)
    gws = torch.empty(max(gu_bytes, 256), dtype=torch.uint8, device=dev)
    layers = []
    for li in range(n_layers):
        x_in, x_out = xs[li % 2], xs[(li + 1) % 2]
        lq = Layer(awq, torch, Hd, (Hq + 2 * Hkv) * D, G, gen, x_in, qkv, ws, dev)
        lo = Layer(awq, torch, Hd, Hd, G, gen, att, oo, ws, dev)
        lg = Layer(awq, torch, Hd, 2 * F, G, gen, oo, hh, ws, dev)
        ld = Layer(awq, torch, F, Hd, G, gen, hh, x_out, ws, dev)
        kc, vc = awq.kv_cache(B, Hkv, S, D, dev)
        kc.normal_(generator=gen)
        vc.normal_(generator=gen)
        layers.append((lq, lo, lg, ld, kc, vc))
    gargs = lambda lg: (lg.x.data_ptr(), lg.qw.data_ptr(), lg.s.data_ptr(), lg.zw.data_ptr(), B, Hd, 2 * F, G,
                        hh.data_ptr(), gws.data_ptr(), gws.numel(), None)

    def run(events=None):
        i = 0
        for lq, lo, lg, ld, kc, vc in layers:
            calls = [("linear", lq), ("attention", (kc, vc)), ("linear", lo), ("gated", lg), ("linear", ld)]
            for kind, obj in calls:
                e0, e1 = (events[2 * i], events[2 * i + 1]) if events else (None, None)
                if kind == "linear":
                    st = lib.awq_linear_timed(*obj.args, None, stream, e0, e1)
                elif kind == "gated":
                    st = lib.awq_linear_silu_mul_ex(*gargs(obj), stream, e0, e1)
                else:
                    st = lib.awq_attention_decode_timed(ctypes.byref(desc), qkv.data_ptr(), obj[0].data_ptr(),
                                                        obj[1].data_ptr(), lengths.data_ptr(), att.data_ptr(),
                                                        aws.data_ptr(), aws.numel(), stream, e0, e1)
                if st:
                    raise RuntimeError(f"chain call failed: {lib.awq_status_string(st).decode()}")
                i += 1
        return i

    n_calls = run()
    torch.cuda.synchronize()
    evs = hip.create(2 * n_calls)
    run(evs)
    torch.cuda.synchronize()
    kinds = (["linear", "attention", "linear", "linear", "linear"] * n_layers)
    split = {"linear": 0.0, "attention": 0.0}
    for i, k in enumerate(kinds):
        split[k] += hip.elapsed_ms(evs[2 * i], evs[2 * i + 1])
    # graph of one step, replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stream = ctypes.c_void_p(side.cuda_stream)
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        run()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    wbytes = n_layers * sum(weight_set_bytes(K, N, G) for K, N in ((Hd, (Hq + 2 * Hkv) * D), (Hd, Hd), (Hd, 2 * F),
                                                                   (F, Hd)))
    kvbytes = n_layers * 4 * D * Hkv * B * L
    del g, layers
    torch.cuda.empty_cache()
    return {"workload": f"llama2-7b-shaped decoder step: {n_layers} layers x (QKV, attention, O, gated gate+up, "
                        f"down), B={B}, {L} tokens cached, G={G}",
            "excluded": "RMSNorm, residual adds, embedding, LM head",
            "ms_per_token": round(ms, 4), "tokens_per_s": round(1e3 / ms * B, 1),
            "eager_linear_ms": round(split["linear"], 4), "eager_attention_ms": round(split["attention"], 4),
            "weight_bytes": wbytes, "kv_bytes": kvbytes,
            "GBps": round((wbytes + kvbytes) / (ms / 1e3) / 1e9, 1)}


def cpu_baseline(workload, seconds):
    """The fp64 oracle on host cores, on one layer of the stack (M=1),
    repeated until about `seconds` of CPU work; weight GB/s. Run with the
    BLAS library's default threads, then again on one thread for a third of
    the time."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threadpool_limits = None
        threads = 1
    data = []
    for si, sh in enumerate(workload.shapes):
        q, z, s = synth.layer(sh.K, sh.N, workload.G, seed=0, layer_id=si, lo=workload.lo, hi=workload.hi)
        x = synth.activations(1, sh.K, seed=0, stream=si)
        data.append((x, q, z, s))

    def run(budget):
        total_bytes, passes = 0, 0
        t0 = time.perf_counter()
        while True:
            for (x, q, z, s), sh in zip(data, workload.shapes):
                oracle.linear64(x, q, z, s, workload.G)
                total_bytes += weight_set_bytes(sh.K, sh.N, workload.G)
            passes += 1
            if time.perf_counter() - t0 >= budget:
                return total_bytes / (time.perf_counter() - t0) / 1e9, passes, time.perf_counter() - t0

    gbps, passes, dt = run(seconds)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            g1, p1, d1 = run(seconds / 3)
        single = {"value": round(g1, 4), "unit": "GB/s", "cores": 1,
                  "sample": f"{p1} pass(es) of the same layer on one BLAS thread, {d1:.1f} s"}
    return {
        "value": round(gbps, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{passes} pass(es) over one layer of the stack ({len(workload.shapes)} linears, M=1, "
                   f"{sum(weight_set_bytes(s.K, s.N, workload.G) for s in workload.shapes) / 1e6:.1f} MB of "
                   f"weights), numpy fp64 dequantise + BLAS matmul, {dt:.1f} s; BLAS threads={threads}, "
                   f"elementwise steps single-threaded"),
        "single_core": single,
    }


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1]))
    except Exception:
        return 1


def _oracle_linear_chunked(x, q, z, s, G, max_bytes=2 << 30):
    """The oracle's layer over contiguous K chunks of whole groups, each
    dequantised to at most `max_bytes` of fp64 (same arithmetic as
    oracle.linear64: fp64 dequantisation, fp64 product, summed over chunks)."""
    import numpy as np

    import oracle
    K, N = q.shape
    rows = max(G, (max_bytes // (8 * N)) // G * G)
    y = np.zeros((x.shape[0], N))
    for k0 in range(0, K, rows):
        k1 = min(K, k0 + rows)
        y += oracle.linear64(x[:, k0:k1], q[k0:k1], z[k0 // G:k1 // G], s[k0 // G:k1 // G], G)
    return y


def cpu_baseline_configs(seconds_small=3.0):
    """The fp64 oracle on the host cores for the other workloads, in the GPU
    metric's units, each leg bounded to a few seconds of CPU work:
    the single 4096 x 4096 layer (M = 1, full shape, repeated); the
    LLaMA-3-8B layer at every M of its sweep (one full pass each); the
    LLaMA-2-13B prefill layer at M = 512 and 2048 on a column slice of every
    shape (1/8 of N), scaled to the full width (extrapolated); one
    Falcon-180B-shaped layer (four linears, full shapes) with the
    dequantisation taken in K chunks of at most 2 GB, times 80 layers
    (extrapolated)."""
    import numpy as np

    import oracle
    import synth
    threads = _blas_threads()
    out = {"kind": "oracle", "cores": threads,
           "what": "numpy fp64 dequantise + BLAS matmul on the host cores (BLAS threads = cores; elementwise "
                   "steps single-threaded); same generated bytes as the parity tests (seeded numpy)"}
    # config: single layer 4096 x 4096, M = 1
    w0 = synth.SINGLE_4096
    sh = w0.shapes[0]
    q, z, s = synth.layer(sh.K, sh.N, w0.G, seed=0)
    x = synth.activations(1, sh.K, seed=0)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds_small:
        oracle.linear64(x, q, z, s, w0.G)
        n += 1
    dt = time.perf_counter() - t0
    out[w0.name] = {"value": round(n * weight_set_bytes(sh.K, sh.N, w0.G) / dt / 1e9, 4), "unit": "GB/s",
                    "sample": f"{n} call(s) of the full 4096 x 4096 layer at M=1, {dt:.1f} s"}
    # config: LLaMA-3-8B layer, M = 1 .. 32, one full pass per M
    w2 = synth.LLAMA3_8B_SWEEP
    lay = [synth.layer(sh.K, sh.N, w2.G, seed=0, layer_id=i, scales=w2.scales, lo=w2.lo, hi=w2.hi)
           for i, sh in enumerate(w2.shapes)]
    per_m = {}
    for M in w2.Ms:
        t0 = time.perf_counter()
        for i, (sh, (q, z, s)) in enumerate(zip(w2.shapes, lay)):
            oracle.linear64(synth.activations(M, sh.K, seed=0, stream=i), q, z, s, w2.G)
        dt = time.perf_counter() - t0
        wb = sum(weight_set_bytes(sh.K, sh.N, w2.G) for sh in w2.shapes)
        per_m[f"M={M}"] = {"value": round(wb / dt / 1e9, 4), "unit": "GB/s", "seconds": round(dt, 2)}
    out[w2.name] = {"per_M": per_m, "sample": "one pass over the four full-shape linears per M"}
    del lay
    # config: LLaMA-2-13B prefill, column slice of 1/8 of N per shape
    w3 = synth.LLAMA2_13B_PREFILL
    per_m = {}
    for M in w3.Ms:
        flop, dt = 0.0, 0.0
        for i, sh in enumerate(w3.shapes):
            n8 = sh.N // 8
            q, z, s = synth.layer(sh.K, n8, w3.G, seed=0, layer_id=i)
            x = synth.activations(M, sh.K, seed=0, stream=i, outlier_frac=w3.outlier_frac)
            t0 = time.perf_counter()
            oracle.linear64(x, q, z, s, w3.G)
            dt += time.perf_counter() - t0
            flop += 2.0 * M * sh.K * sh.N
        per_m[f"M={M}"] = {"value": round(flop / (8 * dt) / 1e9, 3), "unit": "GFLOP/s", "extrapolated": True,
                           "seconds_measured": round(dt, 2)}
    out[w3.name] = {"per_M": per_m, "sample": "each shape on 1/8 of its columns (full K, full M), time x 8"}
    # config: Falcon-180B, one layer, K-chunked, x 80
    w4 = synth.FALCON_180B_STACK
    dt, wb = 0.0, 0
    for i, sh in enumerate(w4.shapes):
        q, z, s = synth.layer(sh.K, sh.N, w4.G, seed=0, layer_id=i)
        x = synth.activations(1, sh.K, seed=0, stream=i)
        t0 = time.perf_counter()
        _oracle_linear_chunked(x, q, z, s, w4.G)
        dt += time.perf_counter() - t0
        wb += weight_set_bytes(sh.K, sh.N, w4.G)
        del q, z, s
    out[w4.name] = {"value": round(wb / dt / 1e9, 4), "unit": "GB/s", "extrapolated": True,
                    "ms_per_step": round(dt * w4.layers * 1e3, 1),
                    "sample": f"one full layer (four linears, {wb / 1e9:.2f} GB of weights) at M=1 with K-chunked "
                              f"fp64 dequantisation (<= 2 GB per chunk), {dt:.1f} s, x {w4.layers} layers"}
    return out


def _short(name):
    return name.split("(")[0].replace("void ", "")


def summarize_profiles(trace_dir, fetch_dir, write_dir, commands):
    """Turn the CSV output of three rocprofv3 runs of this script (kernel
    trace; --pmc FETCH_SIZE; --pmc WRITE_SIZE, the last two with
    --copy-calibration) into profiles/linear_quantize_attention_llama_falcon.md and the
    per-shape traffic files read by traffic_entry().

    Dispatches are matched to layer shapes by their order, which main()
    fixes: decode calls cycle through the decode workload's shapes; prefill
    calls come in two equal blocks (M = 512, then 2048), each cycling through
    the prefill workload's shapes; a split-K reduce kernel belongs to the
    prefill call it follows."""
    import csv
    import statistics
    import synth

    def rows(d, name):
        with open(os.path.join(d, name)) as f:
            return sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))

    def label(seq):
        """[(kernel, key, record)] of awq dispatches -> {(path, shape): [[records of one call], ...]}"""
        dec = [r for r in seq if "decode_" in r[0] and "attn_" not in r[0]]
        out = {}
        dshapes = [sh.name for sh in synth.LLAMA2_7B_DECODE.shapes]
        for i, r in enumerate(dec):
            out.setdefault(("decode", dshapes[i % len(dshapes)]), []).append([r])
        # prefill and W4A8 calls in dispatch order: a W4A8 call is the
        # activation quantiser and its GEMM; a split-K reduction belongs to
        # the call it follows
        calls = {"prefill": [], "w4a8": []}
        last = None
        for r in seq:
            if "prefill_reduce" in r[0] and last:
                last.append(r)
            elif "prefill_kernel" in r[0]:
                last = [r]
                calls["prefill"].append(last)
            elif "act_quant_fp8" in r[0]:
                last = [r]
                calls["w4a8"].append(last)
            elif "w4a8_gemm" in r[0] and last:
                last.append(r)
        # Each half (M = 512, then 2048) of the prefill calls cycles through the
        # shapes; the W4A8 calls of a half come shape by shape in equal blocks.
        pw = synth.LLAMA2_13B_PREFILL
        ns = len(pw.shapes)
        for path, cl in calls.items():
            half = len(cl) // 2
            for i, c in enumerate(cl):
                Mp = pw.Ms[0] if i < half else pw.Ms[1]
                j = i if i < half else i - half
                sh = pw.shapes[j % ns if path == "prefill" else (j * ns) // half]
                out.setdefault((path, f"{sh.name}@M={Mp}"), []).append(c)
        # quantiser calls on the decode stack's shapes, told apart by their
        # grid (one 256-thread workgroup per 128-row band and 128 columns)
        qgrid = {((sh.N + 127) // 128) * ((sh.K + 127) // 128) * 256: sh.name for sh in synth.LLAMA2_7B_DECODE.shapes}
        for r in seq:
            if "quantize_" in r[0]:
                name = qgrid.get(int(r[2].get("Grid_Size_X") or r[2].get("Grid_Size") or -1))
                if name:
                    out.setdefault(("quantize", name), []).append([r])
        # attention calls: per workload, in order, attention_copies(w) warm-up
        # calls and the same number per timed repetition
        att = [r for r in seq if "attn_" in r[0]]
        if att:
            copies = [attention_copies(w) for w in synth.ATTENTION_WORKLOADS]
            per_rep = sum(copies)
            if len(att) % per_rep:
                raise RuntimeError(f"{len(att)} attention dispatches do not split into the workloads' calls")
            i = 0
            for w, c in zip(synth.ATTENTION_WORKLOADS, copies):
                n = c * (len(att) // per_rep)
                out[("attention", w.name)] = [[r] for r in att[i:i + n]]
                i += n
        return out

    trace = [(_short(r["Kernel_Name"]), None, r) for r in rows(trace_dir, "bench_kernel_trace.csv")
             if "awq::" in r["Kernel_Name"]]
    dur = label(trace)

    def counter_calls(d):
        rs = rows(d, "bench_counter_collection.csv")
        copy = [float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"]]
        return label([(_short(r["Kernel_Name"]), None, r) for r in rs if "awq::" in r["Kernel_Name"]]), copy[-1]

    fe, copy_f = counter_calls(fetch_dir)
    wr, copy_w = counter_calls(write_dir)
    ff, fw = (1 << 30) / (copy_f * 1024), (1 << 30) / (copy_w * 1024)
    dshape = {sh.name: sh for sh in synth.LLAMA2_7B_DECODE.shapes}
    pshape = {sh.name: sh for sh in synth.LLAMA2_13B_PREFILL.shapes}

    awl = {w.name: w for w in synth.ATTENTION_WORKLOADS}

    def alg_bytes(path, shape):
        if path == "attention":
            return attention_bytes(awl[shape])
        if path == "quantize":
            sh = dshape[shape]
            return 2 * sh.K * sh.N + weight_set_bytes(sh.K, sh.N, 128)
        if path == "decode":
            sh = dshape[shape]
            return weight_set_bytes(sh.K, sh.N, 128) + 2 * sh.K + 2 * sh.N
        name, m = shape.split("@M=")
        sh, Mp = pshape[name], int(m)
        if path == "w4a8":  # fp16 x read, FP8 x written and read back, token scales, y written
            return weight_set_bytes(sh.K, sh.N, 128) + 4 * Mp * sh.K + 8 * Mp + 2 * Mp * sh.N
        return weight_set_bytes(sh.K, sh.N, 128) + 2 * Mp * sh.K + 2 * Mp * sh.N

    lines = ["# rocprofv3 summary: W4A16 linear, quantiser and decode-attention kernels of bench.py on one MI355X", "",
             "Workloads: LLaMA-2-7B-shaped decode stack (M=1, 32 layers x QKV 4096x12288, O 4096x4096, "
             "gate+up 4096x22016, down 11008x4096) and LLaMA-2-13B-shaped prefill GEMMs (M=512 and 2048; "
             "QKV 5120x15360, O 5120x5120, gate+up 5120x27648, down 13824x5120), group 128; the quantiser on "
             "the decode stack's shapes; the fused decode-step attention on the workloads named in the table "
             "(LLaMA-2-7B MHA 32x128, LLaMA-3-8B GQA 32/8x128, Falcon-7B MQA 71/1x64; B sequences with L "
             "tokens cached).", "",
             "Commands (each run from /tmp with TMPDIR=/tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "The table below comes from `python bench.py --summarize-profiles TRACE FETCH WRITE` on "
              "their output directories.", "",
              "Calibration: a plain 1 GiB device copy (`__amd_rocclr_copyBuffer`) reads "
              f"FETCH_SIZE = {copy_f:.1f} KiB and WRITE_SIZE = {copy_w:.1f} KiB, so the per-dispatch counters "
              f"below are scaled by {ff:.4f} (fetch) and {fw:.4f} (write).", "",
              "| path | shape | kernels of one call | calls | kernel-trace us (median / min / max) | "
              "FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    traffic = {"decode": {}, "prefill": {}, "quantize": {}, "attention": {}, "w4a8": {}}
    for (path, shape), calls in sorted(dur.items()):
        per_call = [sum((int(r[2]["End_Timestamp"]) - int(r[2]["Start_Timestamp"])) / 1e3 for r in c)
                    for c in calls]
        names = " + ".join(f"{r[0]} (grid {r[2].get('Grid_Size_X') or r[2].get('Grid_Size')})" for r in calls[0])
        f_calls = fe.get((path, shape), [])
        w_calls = wr.get((path, shape), [])
        alg = alg_bytes(path, shape)
        trace_cell = f"{statistics.median(per_call):.2f} / {min(per_call):.2f} / {max(per_call):.2f}"
        if not f_calls or not w_calls:
            # not in the counter runs: traffic unmeasured
            lines.append(f"| {path} | {shape} | {names} | {len(per_call)} | {trace_cell} | — | — | — | "
                         f"{alg / 1e6:.2f} MB | — |")
            continue
        f_kib = statistics.mean(sum(float(r[2]["Counter_Value"]) for r in c) for c in f_calls)
        w_kib = statistics.mean(sum(float(r[2]["Counter_Value"]) for r in c) for c in w_calls)
        hbm = f_kib * 1024 * ff + w_kib * 1024 * fw
        lines.append(f"| {path} | {shape} | {names} | {len(per_call)} | {trace_cell} | {f_kib:.0f} | {w_kib:.0f} | "
                     f"{hbm / 1e6:.2f} MB | {alg / 1e6:.2f} MB | {hbm / alg:.3f} |")
        traffic[path][shape] = {"kernels": names, "read_bytes_per_launch": f_kib * 1024 * ff,
                                "write_bytes_per_launch": w_kib * 1024 * fw, "hbm_bytes_per_launch": hbm,
                                "alg_bytes_per_launch": alg, "median_us": statistics.median(per_call)}
    if any(path == "attention" for path, _ in dur) and not traffic["attention"]:
        lines += ["", "The attention kernel appears in the kernel trace only: the counter runs leave it out "
                      "(`--no-attention`), because a FETCH_SIZE run that included it ended with a host-side "
                      "segmentation fault inside the launch call of its first dispatch (not a GPU fault; the "
                      "kernel-trace run of the same kernel completes). Its traffic is unmeasured."]
    md = os.path.join(ROOT, "profiles", "linear_quantize_attention_llama_falcon.md")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    for path in ("decode", "prefill", "quantize", "attention", "w4a8"):
        if not traffic[path]:
            continue
        with open(os.path.join(ROOT, "profiles", f"{path}_traffic.json"), "w") as f:
            json.dump({"kernel_source_sha": source_sha(KERNEL_SOURCES[path]), "fetch_scale": ff,
                       "write_scale": fw, "shapes": traffic[path], "source": os.path.basename(md)}, f, indent=1)
    print("\n".join(lines))


def traffic_set_cases():
    """The decode-path layers profiled by --traffic-set, in launch order:
    the LLaMA-3-8B layer at every M of its sweep, one Falcon-180B-shaped
    layer at M = 1 and 16, the Falcon-7B layer at group 64, M = 1 and 8.
    Each: (label, K, N, G, M, scales, lo, hi)."""
    import synth
    cases = []
    for wl in (synth.LLAMA3_8B_SWEEP, synth.FALCON_180B_STACK, synth.FALCON_7B_DECODE_G64):
        for sh in wl.shapes:
            for M in wl.Ms:
                cases.append((f"{wl.name}/{sh.name}@M={M}", sh.K, sh.N, wl.G, M, wl.scales, wl.lo, wl.hi))
    return cases


TRAFFIC_SET_REPS = 3


def run_traffic_set(awq, lib, torch, dev, seed):
    """Launch every case of traffic_set_cases() TRAFFIC_SET_REPS times (automatic
    plan), one case after another, for rocprofv3 counter and trace runs."""
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    ws = awq.Workspace(dev)
    built = {}
    for label, K, N, G, M, scales, lo, hi in traffic_set_cases():
        key = (K, N, G, lo, hi)
        if key not in built:
            built.clear()
            torch.cuda.empty_cache()
            x = torch.randn((64, K), device=dev, generator=gen).half()
            y = torch.empty((64, N), dtype=torch.float16, device=dev)
            built[key] = Layer(awq, torch, K, N, G, gen, x[:1], y[:1], ws, dev, scales=(lo, hi))
            built["x"], built["y"] = x, y
        L = built[key].rebound(awq, built["x"][:M], built["y"][:M], ws)
        for _ in range(TRAFFIC_SET_REPS):
            L.launch(lib, stream)
        torch.cuda.synchronize()
        eprint(f"[bench] traffic set: {label} plan {awq.linear_plan(M, K, N, G)}")


def summarize_traffic_set(trace_dir, fetch_dir, write_dir, commands):
    """profiles/decode_sweep_falcon_g64_traffic.md and decode_set_traffic.json
    from the CSV output of three rocprofv3 runs of `bench.py --traffic-set`
    (kernel trace; --pmc FETCH_SIZE; --pmc WRITE_SIZE, the counter runs with
    --copy-calibration). A call is a decode kernel and, for a plan that splits
    K, the reduction kernel after it; calls come case by case in
    traffic_set_cases() order, TRAFFIC_SET_REPS per case."""
    import csv
    import statistics

    def rows(d, name):
        with open(os.path.join(d, name)) as f:
            return sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))

    cases = traffic_set_cases()

    def calls(rs):
        out, last = [], None
        for r in rs:
            name = _short(r["Kernel_Name"])
            if "decode_" in name:
                last = [(name, r)]
                out.append(last)
            elif "prefill_reduce" in name and last is not None:
                last.append((name, r))
        if len(out) != len(cases) * TRAFFIC_SET_REPS:
            raise RuntimeError(f"{len(out)} decode calls for {len(cases)} cases x {TRAFFIC_SET_REPS}")
        return {c[0]: out[i * TRAFFIC_SET_REPS:(i + 1) * TRAFFIC_SET_REPS] for i, c in enumerate(cases)}

    tr = calls(rows(trace_dir, "bench_kernel_trace.csv"))

    def counters(d):
        rs = rows(d, "bench_counter_collection.csv")
        copy = [float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"]]
        return calls([r for r in rs if "awq::" in r["Kernel_Name"]]), copy[-1]

    fe, copy_f = counters(fetch_dir)
    wr, copy_w = counters(write_dir)
    ff, fw = (1 << 30) / (copy_f * 1024), (1 << 30) / (copy_w * 1024)
    lines = ["# rocprofv3 summary: decode-path kernels on the batched LLaMA-3-8B layer, a Falcon-180B-shaped layer "
             "and the Falcon-7B layer at group 64, one MI355X", "",
             "Layers (automatic plans): LLaMA-3-8B QKV 4096x6144, O 4096x4096, gate+up 4096x28672, down 14336x4096 "
             "at M = 1, 2, 4, 8, 16, 32 (G = 128); Falcon-180B-shaped QKV 14848x15872, O 14848x14848, up "
             "14848x59392, down 59392x14848 at M = 1 and 16 (G = 128); Falcon-7B QKV 4544x4672, O 4544x4544, up "
             "4544x18176, down 18176x4544 at M = 1 and 8 (G = 64). Each layer is launched "
             f"{TRAFFIC_SET_REPS} times in a row.", "", "Commands (each run from /tmp with TMPDIR=/tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "The table comes from `python bench.py --summarize-traffic-set TRACE FETCH WRITE` on their output "
              "directories.", "",
              f"Calibration: a plain 1 GiB device copy reads FETCH_SIZE = {copy_f:.1f} KiB and WRITE_SIZE = "
              f"{copy_w:.1f} KiB, so the per-call counters below are scaled by {ff:.4f} (fetch) and {fw:.4f} "
              "(write). Algorithmic bytes = weight set + 2MK (x) + 2MN (y); a K split adds its fp32 partials "
              "(written and read back, 8 split M N) to the traffic but not to the algorithmic bytes.", "",
              "| layer | kernels of one call | kernel-trace us (median) | weight GB/s | FETCH_SIZE KiB | WRITE_SIZE KiB "
              "| HBM bytes (scaled) | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|---|---|---|"]
    out = {}
    for label, K, N, G, M, *_ in cases:
        us = statistics.median(sum((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3 for _, r in c)
                               for c in tr[label])
        names = " + ".join(f"{n} (grid {r.get('Grid_Size_X') or r.get('Grid_Size')})" for n, r in tr[label][0])
        fk = statistics.mean(sum(float(r["Counter_Value"]) for _, r in c) for c in fe[label])
        wk = statistics.mean(sum(float(r["Counter_Value"]) for _, r in c) for c in wr[label])
        hbm = fk * 1024 * ff + wk * 1024 * fw
        wb = weight_set_bytes(K, N, G)
        alg = wb + 2 * M * K + 2 * M * N
        lines.append(f"| {label} | {names} | {us:.2f} | {wb / us / 1e3:.0f} | {fk:.0f} | {wk:.0f} | "
                     f"{hbm / 1e6:.2f} MB | {alg / 1e6:.2f} MB | {hbm / alg:.3f} |")
        out[label] = {"kernels": names, "median_us": round(us, 3), "hbm_bytes_per_launch": hbm,
                      "alg_bytes_per_launch": alg}
    md = os.path.join(ROOT, "profiles", "decode_sweep_falcon_g64_traffic.md")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(ROOT, "profiles", "decode_set_traffic.json"), "w") as f:
        json.dump({"kernel_source_sha": source_sha(KERNEL_SOURCES["decode"]), "fetch_scale": ff,
                   "write_scale": fw, "shapes": out, "source": os.path.basename(md)}, f, indent=1)
    print(md)


def traffic_set_entry(label):
    """HBM bytes per call of a decode-set layer (profiles/decode_set_traffic.json),
    if taken on the current decode kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_set_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != source_sha(KERNEL_SOURCES["decode"]):
        return None
    entry = t.get("shapes", {}).get(label)
    return round(entry["hbm_bytes_per_launch"]) if entry else None


def traffic_entry(kernel, shape):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the counters'
    reading of a plain copy of known size) from the committed rocprofv3
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    entry = t.get("shapes", {}).get(shape)
    return round(entry["hbm_bytes_per_launch"]) if entry else None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-g64", action="store_true", help="skip the group-64 (Falcon-7B) decode stack")
    ap.add_argument("--no-gated", action="store_true", help="skip the gated-epilogue comparison")
    ap.add_argument("--no-sweep", action="store_true", help="skip the batched-decode sweep (M = 1 .. 32)")
    ap.add_argument("--no-falcon180b", action="store_true", help="skip the 92 GB Falcon-180B-shaped stack")
    ap.add_argument("--no-attention", action="store_true", help="skip the decode-step attention kernel")
    ap.add_argument("--no-w4a8", action="store_true", help="skip the W4A8-FP8 prefill comparison")
    ap.add_argument("--no-chain", action="store_true", help="skip the decoder-step chain (linears + attention)")
    ap.add_argument("--kernel-reps", type=int, default=3, help="eager passes with per-kernel events")
    ap.add_argument("--prefill-reps", type=int, default=50)
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV output of this script, then exit")
    ap.add_argument("--profile-commands", nargs="*", default=[],
                    help="the rocprofv3 command lines, quoted in the summary")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--traffic-set", action="store_true",
                    help="only launch the decode-path profiling set (batched LLaMA-3-8B, Falcon-180B and Falcon-7B "
                         "group-64 layers) for rocprofv3, then exit")
    ap.add_argument("--summarize-traffic-set", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries of --traffic-set runs, then exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, args.profile_commands)
        return
    if args.summarize_traffic_set:
        summarize_traffic_set(*args.summarize_traffic_set, args.profile_commands)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the layer's multi-GPU "
              f"sharding is a design note, not a built path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import weight_only_bit_awq_amd as awq

    lib = awq.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.traffic_set:
        run_traffic_set(awq, lib, torch, dev, args.seed + 9)
        if args.copy_calibration:
            a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            eprint("[bench] copy calibration: 1 GiB device copy done")
        return
    hip = HipEvents()
    wl = synth.LLAMA2_7B_DECODE
    M = 1

    eprint(f"[bench] building {wl.name}: {wl.layers} layers x {len(wl.shapes)} shapes, M={M}")
    layers, ws = build_stack(awq, torch, wl, M, dev, args.seed)
    step_bytes = sum(weight_set_bytes(L.K, L.N, L.G) for _, L in layers)
    eprint(f"[bench] weight set {step_bytes / 1e9:.3f} GB resident")

    wall_ms, event_ms = time_stack_graph(lib, torch, layers, args.steps, args.warmup)
    value = step_bytes / (wall_ms / 1e3) / 1e9
    eprint(f"[bench] decode stack: {wall_ms:.4f} ms/step wall, {event_ms:.4f} ms/step events, {value:.1f} GB/s")

    # Per-kernel durations (events at the kernels' own start/end).
    per_shape = per_shape_stats(awq, lib, torch, hip, wl, layers, M, args.kernel_reps)
    # Context for the roofline: the achievable streaming-read rate at each
    # layer's size, and the same shapes as dense fp16 weights (W16A16).
    sr = stream_read_times(lib, torch, hip, layers, args.kernel_reps)
    for name, (nb, ts) in sr.items():
        ts = sorted(ts)
        med = ts[len(ts) // 2]
        p = per_shape[name]
        p["stream_read_GBps"] = round(nb / (med / 1e3) / 1e9, 1)
        p["pct_of_stream_read"] = round(100 * p["weight_GBps"] / p["stream_read_GBps"], 1)
    kern_sum_ms = sum(p["avg_us"] for p in per_shape.values()) * wl.layers / 1e3
    dom = max(per_shape, key=lambda k: per_shape[k]["avg_us"])
    d = per_shape[dom]
    alg_bytes = weight_set_bytes(d["K"], d["N"], wl.G) + 2 * M * d["K"] + 2 * M * d["N"]
    achieved = alg_bytes / (d["avg_us"] / 1e6) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_entry("decode", dom),
        "kernel": f"decode_kernel ({dom}: K={d['K']} N={d['N']} M={M})", "alg_bytes_per_launch": alg_bytes,
        "avg_launch_us": d["avg_us"],
        "stream_read_GBps_same_size": d.get("stream_read_GBps"),
    }
    eprint(f"[bench] per-kernel: " + ", ".join(f"{k} {v['avg_us']}us {v['weight_GBps']}GB/s"
                                               for k, v in per_shape.items()))

    layers = None
    torch.cuda.empty_cache()
    fp16 = fp16_dense_times(torch, [(sh.name, sh.K, sh.N) for sh in wl.shapes], M, dev)
    fp16_layer_ms = sum(fp16.values())
    w4_layer_ms = sum(p["avg_us"] for p in per_shape.values()) / 1e3
    for name, ms in fp16.items():
        per_shape[name]["fp16_dense_us"] = round(ms * 1e3, 3)
        per_shape[name]["speedup_vs_fp16"] = round(ms * 1e3 / per_shape[name]["avg_us"], 3)
    fp16_ref = {"what": "the same M=1 layer shapes as dense fp16 weights through torch F.linear (vendor BLAS), "
                        "median event time per call; the W16A16 counterpart of the W4A16 layer",
                "layer_us": round(fp16_layer_ms * 1e3, 2), "w4a16_layer_us": round(w4_layer_ms * 1e3, 2),
                "speedup_w4a16_over_fp16": round(fp16_layer_ms / w4_layer_ms, 3)}
    eprint(f"[bench] fp16 dense layer {fp16_layer_ms * 1e3:.1f} us vs W4A16 {w4_layer_ms * 1e3:.1f} us")

    # Group size 64 (the Falcon-7B setting): the Falcon-7B-shaped decode stack.
    g64 = None
    if not args.no_g64:
        wg = synth.FALCON_7B_DECODE_G64
        eprint(f"[bench] building {wg.name}: {wg.layers} layers x {len(wg.shapes)} shapes, M={M}, G={wg.G}")
        glayers, _ = build_stack(awq, torch, wg, M, dev, args.seed + 2)
        gbytes = sum(weight_set_bytes(L.K, L.N, L.G) for _, L in glayers)
        gwall, gev = time_stack_graph(lib, torch, glayers, args.steps, args.warmup)
        gps = per_shape_stats(awq, lib, torch, hip, wg, glayers, M, args.kernel_reps)
        g64 = {"workload": wg.name, "group": wg.G, "layers": wg.layers, "M": M,
               "weight_bytes_per_step": gbytes, "ms_per_step": round(gwall, 5),
               "value": round(gbytes / (gwall / 1e3) / 1e9, 1), "unit": "GB/s",
               "pct_hbm_peak": round(100 * gbytes / (gwall / 1e3) / 1e9 / HBM_PEAK_GBS, 2), "per_kernel": gps}
        eprint(f"[bench] G=64 stack: {gwall:.4f} ms/step, {g64['value']} GB/s; " +
               ", ".join(f"{k} {v['avg_us']}us {v['weight_GBps']}GB/s" for k, v in gps.items()))
        glayers = None
        torch.cuda.empty_cache()

    # The Falcon-180B-shaped stack: 80 layers (92 GB of int4 weights) resident
    # in HBM, one pass per step, at M = 1 and M = 16.
    falcon = None
    if not args.no_falcon180b:
        wf = synth.FALCON_180B_STACK
        eprint(f"[bench] building {wf.name}: {wf.layers} layers x {len(wf.shapes)} shapes")
        flayers, fws = build_stack(awq, torch, wf, 1, dev, args.seed + 4)
        fbytes = sum(weight_set_bytes(L.K, L.N, L.G) for _, L in flayers)
        falcon = {"workload": wf.name, "layers": wf.layers, "group": wf.G, "weight_bytes_per_step": fbytes}
        for Mf in wf.Ms:
            if Mf == 1:
                fl = flayers
            else:
                xs = {K: torch.randn((Mf, K), device=dev).half() for K in {L.K for _, L in flayers}}
                ys = {N: torch.empty((Mf, N), dtype=torch.float16, device=dev) for N in {L.N for _, L in flayers}}
                fl = [(n, L.rebound(awq, xs[L.K], ys[L.N], fws)) for n, L in flayers]
            fwall, _ = time_stack_graph(lib, torch, fl, max(3, args.steps // 10), 2)
            fps = per_shape_stats(awq, lib, torch, hip, wf, fl, Mf, 1)
            falcon[f"M={Mf}"] = {"ms_per_step": round(fwall, 4), "weight_GBps": round(fbytes / (fwall / 1e3) / 1e9, 1),
                                 "pct_hbm_peak": round(100 * fbytes / (fwall / 1e3) / 1e9 / HBM_PEAK_GBS, 2),
                                 "per_kernel": fps}
            eprint(f"[bench] {wf.name} M={Mf}: {fwall:.3f} ms/step, {falcon[f'M={Mf}']['weight_GBps']} GB/s; " +
                   ", ".join(f"{k} {v['avg_us']}us {v['weight_GBps']}GB/s" for k, v in fps.items()))
            fl = None
        flayers = None
        torch.cuda.empty_cache()

    # Batched decode: M = 1 .. 32 on the LLaMA-3-8B-shaped layers.
    sweep = None
    if not args.no_sweep:
        ws3 = synth.LLAMA3_8B_SWEEP
        sweep = {"workload": ws3.name, "group": ws3.G, "per_M": decode_sweep(awq, lib, torch, hip, ws3, dev,
                                                                             args.seed + 3)}
        eprint("[bench] decode sweep: " + ", ".join(f"{k} {v['layer_us']}us {v['weight_GBps']}GB/s "
                                                     f"(graph {v['graph_layer_us']}us)"
                                                    for k, v in sweep["per_M"].items()))

    # Gated epilogue (silu(gate) * up) on the fused gate+up layer.
    gated = None
    if not args.no_gated:
        gated = {"what": "awq_linear_silu_mul (silu(gate) * up in the kernel's epilogue) against awq_linear "
                         "followed by torch silu and multiply on the halves",
                 "decode_llama2_7b_gate_up_M1": gated_times(awq, lib, torch, hip, 4096, 22016, 128, 1, dev, 24, 4),
                 "decode_llama3_8b_gate_up_M16": gated_times(awq, lib, torch, hip, 4096, 28672, 128, 16, dev, 8, 4)}
        if not args.no_prefill:
            gated["prefill_llama2_13b_gate_up_M2048"] = gated_times(awq, lib, torch, hip, 5120, 27648, 128, 2048,
                                                                      dev, 2, 10)
        eprint("[bench] gated: " + ", ".join(f"{k}: fused {v['fused_us']}us vs unfused {v['unfused_us']}us"
                                              for k, v in gated.items() if isinstance(v, dict)))

    # Fused decode-step attention (rotary embedding, MHA/GQA/MQA, cache append).
    attention = None
    if not args.no_attention:
        at = attention_times(awq, lib, torch, hip, synth.ATTENTION_WORKLOADS, dev)
        adom = max(at, key=lambda k: at[k]["alg_bytes"])
        attention = {"what": "awq_attention_decode: one generation step of attention (rotary embedding of q and "
                             "the new k, softmax attention over the fp16 cache, append of the new key and value) "
                             "in one kernel; HBM bytes = cached keys and values read once + qkv read + output "
                             "and new key/value written",
                     "cases": at,
                     "roofline": {"bound": "hbm", "achieved": at[adom]["GBps"], "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(at[adom]["GBps"] / HBM_PEAK_GBS, 4),
                                  "traffic": traffic_entry("attention", adom),
                                  "kernel": f"attn_decode_kernel ({adom})",
                                  "alg_bytes_per_launch": at[adom]["alg_bytes"],
                                  "avg_launch_us": at[adom]["median_us"]}}
        eprint("[bench] attention: " + ", ".join(f"{k} {v['median_us']}us {v['GBps']}GB/s"
                                                 for k, v in at.items()))

    chain = None
    if not args.no_chain:
        chain = decode_chain(awq, lib, torch, hip, dev, max(5, args.steps // 2), 3)
        eprint(f"[bench] decoder step chain: {chain['ms_per_token']} ms/token ({chain['tokens_per_s']} tokens/s), "
               f"eager split linear {chain['eager_linear_ms']} ms / attention {chain['eager_attention_ms']} ms")

    qt = quantize_times(awq, torch, [(sh.name, sh.K, sh.N) for sh in wl.shapes], wl.G, dev)
    qdom = max(qt, key=lambda k: qt[k]["median_us"])
    quantize = {"what": "awq_quantize: round-to-nearest group quantiser, fp16 W [K,N] (N(0, 0.02)) -> device "
                        "qweight + fp16 scales + packed zero points, on the decode stack's layer shapes",
                "shapes": qt,
                "roofline": {"bound": "hbm", "achieved": qt[qdom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(qt[qdom]["GBps"] / HBM_PEAK_GBS, 4),
                             "traffic": traffic_entry("quantize", qdom),
                             "kernel": f"quantize_kernel ({qdom})"}}
    eprint("[bench] quantize: " + ", ".join(f"{k} {v['median_us']}us {v['GBps']}GB/s" for k, v in qt.items()))

    prefill = None
    if not args.no_prefill:
        pw = synth.LLAMA2_13B_PREFILL
        prefill = {"metric": "GEMM TFLOP/s at M=2048", "unit": "TFLOP/s", "workload": pw.name, "shapes": {}}
        for Mp in pw.Ms:
            play, _ = build_stack(awq, torch, pw, Mp, dev, args.seed + 1, layers=1)
            # 1% outlier input channels scaled by 20 in each activation matrix
            for K in {L.K for _, L in play}:
                gen = torch.Generator(device=dev)
                gen.manual_seed(K)
                cols = torch.randperm(K, device=dev, generator=gen)[: round(0.01 * K)]
                for _, L in play:
                    if L.K == K:
                        L.x[:, cols] *= 20
                        break
            per_kernel_times(lib, torch, hip, play, 5)  # warm-up: first launches, clocks
            pt = per_kernel_times(lib, torch, hip, play, args.prefill_reps)
            tot_flop, tot_ms = 0.0, 0.0
            for name, L in play:
                ts = sorted(pt[name])
                med = ts[len(ts) // 2]
                fl = 2.0 * Mp * L.K * L.N
                tot_flop += fl
                tot_ms += med
                prefill["shapes"][f"{name}@M={Mp}"] = {
                    "K": L.K, "N": L.N, "median_us": round(med * 1e3, 2),
                    "p10_us": round(ts[len(ts) // 10] * 1e3, 2), "p90_us": round(ts[(9 * len(ts)) // 10] * 1e3, 2),
                    "TFLOPs": round(fl / (med / 1e3) / 1e12, 1),
                    "plan": awq.linear_plan(Mp, L.K, L.N, 128)}
            prefill[f"M={Mp}"] = round(tot_flop / (tot_ms / 1e3) / 1e12, 1)
            del play
            torch.cuda.empty_cache()
        dense = fp16_dense_times(torch, [(sh.name, sh.K, sh.N) for sh in pw.shapes], max(pw.Ms), dev, reps=20,
                                 copies=2)
        dflop = sum(2.0 * max(pw.Ms) * sh.K * sh.N for sh in pw.shapes)
        prefill["dense_fp16_torch"] = {
            "what": "the same M=2048 shapes as a dense fp16 GEMM through torch F.linear (vendor BLAS)",
            "TFLOPs": round(dflop / (sum(dense.values()) / 1e3) / 1e12, 1),
            "shapes": {k: round(2.0 * max(pw.Ms) * sh.K * sh.N / (dense[k] / 1e3) / 1e12, 1)
                       for k, sh in ((s.name, s) for s in pw.shapes)}}
        prefill["value"] = prefill["M=2048"]
        big = max((k for k in prefill["shapes"] if k.endswith("M=2048")),
                  key=lambda k: prefill["shapes"][k]["median_us"])
        pv = prefill["shapes"][big]["TFLOPs"]
        prefill["roofline"] = {"bound": "mfma", "achieved": pv, "peak": FP16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(pv / FP16_DENSE_PEAK_TFLOPS, 4),
                               "traffic": traffic_entry("prefill", big), "kernel": f"prefill_kernel ({big})"}
        eprint(f"[bench] prefill: M=2048 {prefill['M=2048']} TFLOP/s, M=512 {prefill['M=512']} TFLOP/s")

    # W4A8-FP8 form of the same prefill layers: per-token FP8 activations,
    # FP8 matrix cores; one call = the activation quantiser + the GEMM (+ the
    # split-K reduction), timed from the first kernel's start to the last's end.
    w4a8 = None
    if not args.no_prefill and not args.no_w4a8:
        pw = synth.LLAMA2_13B_PREFILL
        w4a8 = {"what": "awq_linear_w4a8: activations quantised per token to FP8 E4M3 inside the call, int4 weights "
                        "decoded to exact FP8 (q - z), FP8 MFMA, group and token scales in fp32; same LLaMA-2-13B "
                        "shapes and activations as the prefill section",
                "unit": "TFLOP/s", "shapes": {}}
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for Mp in pw.Ms:
            play, _ = build_stack(awq, torch, pw, Mp, dev, args.seed + 1, layers=1)
            tot_flop, tot_ms = 0.0, 0.0
            for name, L in play:
                nb = awq.linear_w4a8_workspace_bytes(Mp, L.K, L.N, 128)
                wsb = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
                cargs = (L.x.data_ptr(), L.qw.data_ptr(), L.s.data_ptr(), L.zw.data_ptr(), Mp, L.K, L.N, 128,
                         L.y.data_ptr(), wsb.data_ptr(), wsb.numel(), None, stream)
                for _ in range(5):
                    if lib.awq_linear_w4a8_ex(*cargs, None, None):
                        raise RuntimeError("awq_linear_w4a8 failed")
                evs = hip.create(2 * args.prefill_reps)
                for i in range(args.prefill_reps):
                    lib.awq_linear_w4a8_ex(*cargs, evs[2 * i], evs[2 * i + 1])
                torch.cuda.synchronize()
                ts = sorted(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(args.prefill_reps))
                med = ts[len(ts) // 2]
                fl = 2.0 * Mp * L.K * L.N
                tot_flop += fl
                tot_ms += med
                w4a8["shapes"][f"{name}@M={Mp}"] = {
                    "K": L.K, "N": L.N, "median_us": round(med * 1e3, 2),
                    "p10_us": round(ts[len(ts) // 10] * 1e3, 2), "p90_us": round(ts[(9 * len(ts)) // 10] * 1e3, 2),
                    "TFLOPs": round(fl / (med / 1e3) / 1e12, 1), "plan": awq.linear_w4a8_plan(Mp, L.K, L.N, 128)}
                del wsb
            w4a8[f"M={Mp}"] = round(tot_flop / (tot_ms / 1e3) / 1e12, 1)
            del play
            torch.cuda.empty_cache()
        big = max((k for k in w4a8["shapes"] if k.endswith("M=2048")), key=lambda k: w4a8["shapes"][k]["median_us"])
        wv = w4a8["shapes"][big]["TFLOPs"]
        w4a8["roofline"] = {"bound": "mfma", "achieved": wv, "peak": FP8_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(wv / FP8_DENSE_PEAK_TFLOPS, 4), "traffic": traffic_entry("w4a8", big),
                            "kernel": f"act_quant_fp8_kernel + w4a8_gemm_kernel ({big})"}
        if prefill:
            w4a8["speedup_over_w4a16_M2048"] = round(w4a8["M=2048"] / prefill["M=2048"], 3)
        eprint(f"[bench] w4a8: M=2048 {w4a8['M=2048']} TFLOP/s, M=512 {w4a8['M=512']} TFLOP/s")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        eprint("[bench] copy calibration: 1 GiB device copy done")

    cpu = None
    cpu_configs = None
    if not args.no_cpu_baseline:
        eprint(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        eprint("[bench] timing the CPU oracle on the other workloads")
        cpu_configs = cpu_baseline_configs()
        eprint("[bench] CPU oracle: " + json.dumps({k: v for k, v in cpu_configs.items() if isinstance(v, dict)})[:400])

    out = {
        "metric": "W4A16 GEMV weight GB/s (% HBM peak) at M=1; GEMM TFLOP/s at M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded random-init int4 weights, fp16 N(0,1) activations)",
        "config": {"workload": wl.name, "layers": wl.layers, "M": M, "group": wl.G,
                   "shapes": {sh.name: [sh.K, sh.N] for sh in wl.shapes},
                   "weight_bytes_per_step": step_bytes, "graph": True},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "event_ms_per_step": round(event_ms, 5),
        "kernel_sum_ms_per_step": round(kern_sum_ms, 5),
        "per_kernel": per_shape,
        "roofline": roofline,
        "fp16_dense_reference": fp16_ref,
        "decode_g64": g64,
        "decode_sweep": sweep,
        "decode_falcon180b": falcon,
        "gated": gated,
        "quantize": quantize,
        "attention": attention,
        "decode_layer_chain": chain,
        "prefill": prefill,
        "w4a8": w4a8,
        "cpu_baseline": cpu,
        "cpu_baseline_configs": cpu_configs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
