"""Seeded synthetic inputs for the W4A16 linear layer.

Shared by the tests, the bench and the smoke check. This module only draws
random numbers and describes workload shapes: it holds none of the layer's
arithmetic (no packing, no dequantisation, no products), so the HIP path and
the CPU oracle can both consume its output without sharing method code.

Value distributions follow the workloads the layer is measured on: codes and
zero points uniform over 0..15, fp16 scales uniform in [0.001, 0.02] (or
log-uniform in [1e-3, 3e-2]), fp16 activations N(0, 1), optionally with 1% of
input channels scaled by 20 (outlier channels). Draw order per layer: codes,
zero points, scales; activations come from their own stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _rng(*tags: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(t) for t in tags]))


def layer(K: int, N: int, G: int = 128, seed: int = 0, layer_id: int = 0,
          scales: str = "uniform", lo: float = 0.001, hi: float = 0.02):
    """Codes q uint8 [K, N], zero points z uint8 [K/G, N], scales s fp16 [K/G, N]."""
    if K % G:
        raise ValueError("K must be a multiple of G")
    rng = _rng(seed, 1, layer_id, K, N, G)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    if scales == "uniform":
        s = rng.uniform(lo, hi, size=(K // G, N))
    elif scales == "loguniform":
        s = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(K // G, N)))
    else:
        raise ValueError(scales)
    return q, z, s.astype(np.float16)


def activations(M: int, K: int, seed: int = 0, stream: int = 0,
                outlier_frac: float = 0.0, outlier_gain: float = 20.0):
    """x fp16 [M, K] ~ N(0, 1); round(outlier_frac*K) input channels (chosen
    without replacement) are multiplied by outlier_gain before the fp16 cast."""
    rng = _rng(seed, 2, stream, M, K)
    x = rng.standard_normal(size=(M, K))
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = rng.choice(K, n_out, replace=False)
        x[:, cols] *= outlier_gain
    return x.astype(np.float16)


def outlier_channels(K: int, seed: int = 0, stream: int = 0, M: int = 1,
                     outlier_frac: float = 0.01):
    """The channel indices ``activations`` scales (same draws, same order)."""
    rng = _rng(seed, 2, stream, M, K)
    rng.standard_normal(size=(M, K))
    n_out = int(round(outlier_frac * K))
    return np.sort(rng.choice(K, n_out, replace=False)) if n_out else np.zeros(0, int)


@dataclass(frozen=True)
class Shape:
    name: str
    K: int
    N: int


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple
    Ms: tuple
    G: int = 128
    layers: int = 1
    scales: str = "uniform"
    lo: float = 0.001
    hi: float = 0.02
    outlier_frac: float = 0.0


# Single layer, M=1, K=N=4096, G=128.
SINGLE_4096 = Workload("single-4096x4096", (Shape("proj", 4096, 4096),), (1,))

# LLaMA-2-7B-shaped decode set: 32 layers of fused QKV, O, fused gate+up, down.
LLAMA2_7B_DECODE = Workload(
    "llama2-7b-decode-stack",
    (Shape("qkv", 4096, 12288), Shape("o", 4096, 4096),
     Shape("gate_up", 4096, 22016), Shape("down", 11008, 4096)),
    (1,), layers=32)

# LLaMA-3-8B-shaped batched decode sweep (GQA: 32 q / 8 kv heads of dim 128).
LLAMA3_8B_SWEEP = Workload(
    "llama3-8b-decode-sweep",
    (Shape("qkv", 4096, 6144), Shape("o", 4096, 4096),
     Shape("gate_up", 4096, 28672), Shape("down", 14336, 4096)),
    (1, 2, 4, 8, 16, 32), scales="loguniform", lo=1e-3, hi=3e-2)

# LLaMA-2-13B-shaped prefill with 1% outlier input channels.
LLAMA2_13B_PREFILL = Workload(
    "llama2-13b-prefill",
    (Shape("qkv", 5120, 15360), Shape("o", 5120, 5120),
     Shape("gate_up", 5120, 27648), Shape("down", 13824, 5120)),
    (512, 2048), outlier_frac=0.01)

# Falcon-180B-shaped stack (232 q heads + 2 x 8 kv heads of dim 64), 80 layers.
FALCON_180B_STACK = Workload(
    "falcon-180b-stack",
    (Shape("qkv", 14848, 15872), Shape("o", 14848, 14848),
     Shape("up", 14848, 59392), Shape("down", 59392, 14848)),
    (1, 16), layers=80)

# Falcon-7B-shaped decode stack at group size 64 (the group the TinyChat
# README prescribes for Falcon-7B): 71 query heads + 1 shared key/value head
# of dim 64 (hidden 4544), 4x MLP, 32 layers. K = 4544 is not a multiple of
# 128, so the last 128-row band of every layer is ragged.
FALCON_7B_DECODE_G64 = Workload(
    "falcon-7b-decode-stack-g64",
    (Shape("qkv", 4544, 4672), Shape("o", 4544, 4544),
     Shape("up", 4544, 18176), Shape("down", 18176, 4544)),
    (1, 8), G=64, layers=32)

WORKLOADS = (SINGLE_4096, LLAMA2_7B_DECODE, LLAMA3_8B_SWEEP, LLAMA2_13B_PREFILL,
             FALCON_180B_STACK, FALCON_7B_DECODE_G64)


def dense_weights(K: int, N: int, seed: int = 0, layer_id: int = 0, std: float = 0.02):
    """fp16 weights [K, N] ~ N(0, std^2) (the usual initialisation scale of
    LLM linear layers): input of the round-to-nearest quantiser."""
    rng = _rng(seed, 3, layer_id, K, N)
    return (rng.standard_normal(size=(K, N)) * std).astype(np.float16)


@dataclass(frozen=True)
class AttnWorkload:
    """One generation step of attention: B sequences with L tokens cached
    each, Hq query / Hkv key-value heads of dimension D, rotary base theta."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int
    theta: float = 10000.0
    rope: str = "half"

    @property
    def capacity(self) -> int:
        """Cache slots: room for the new token, rounded up to 32."""
        return (self.L + 1 + 31) // 32 * 32


# Decode-step attention of the models in the TinyChat generation benchmarks
# (LLaMA-2-7B: 32 heads of 128; LLaMA-3-8B: 32 query / 8 key-value heads,
# rotary base 500000; Falcon-7B: 71 query heads sharing one key-value head of
# 64), at the >500-token prompts of the LLaMA-2 figures, at long contexts and
# batched.
ATTENTION_WORKLOADS = (
    AttnWorkload("llama2-7b-mha-B1-L1024", 1, 32, 32, 128, 1024),
    AttnWorkload("llama2-7b-mha-B1-L4096", 1, 32, 32, 128, 4096),
    AttnWorkload("llama3-8b-gqa-B1-L4096", 1, 32, 8, 128, 4096, theta=500000.0),
    AttnWorkload("falcon-7b-mqa-B1-L2048", 1, 71, 1, 64, 2048),
    AttnWorkload("llama2-7b-mha-B16-L2048", 16, 32, 32, 128, 2048),
    AttnWorkload("llama3-8b-gqa-B32-L4096", 32, 32, 8, 128, 4096, theta=500000.0),
)


def attention_inputs(w: AttnWorkload, seed: int = 0):
    """qkv rows [B, (Hq + 2 Hkv) D] fp16 ~ N(0, 1) and caches k, v
    [B, Hkv, capacity, D] fp16 ~ N(0, 1) (logical layout; positions past L are
    filled too), lengths [B] = L."""
    rng = _rng(seed, 4, w.B, w.Hq, w.Hkv, w.D, w.L)
    qkv = rng.standard_normal((w.B, (w.Hq + 2 * w.Hkv) * w.D)).astype(np.float16)
    k = rng.standard_normal((w.B, w.Hkv, w.capacity, w.D)).astype(np.float16)
    v = rng.standard_normal((w.B, w.Hkv, w.capacity, w.D)).astype(np.float16)
    return qkv, k, v, np.full(w.B, w.L, np.int32)


def attention_exact_inputs(w: AttnWorkload, L: int, seed: int = 0):
    """Inputs of an attention step whose result is exact in binary arithmetic:
    the query part of every qkv row is 0 (every score is 0), and every value
    (cached, and the new token's) is an odd integer drawn from {-3, -1, 1, 3}
    independently per sequence, kv head, position and element; keys ~ N(0, 1).
    With L + 1 a power of two the output is a sum of small integers divided by
    a power of two. Returns (qkv, k, v, lengths) like ``attention_inputs``,
    with lengths[b] = L and capacity = L + 1 rounded up to 32."""
    cap = (L + 1 + 31) // 32 * 32
    rng = _rng(seed, 5, w.B, w.Hq, w.Hkv, w.D, L)
    odd = np.array([-3.0, -1.0, 1.0, 3.0], np.float16)
    qkv = rng.standard_normal((w.B, (w.Hq + 2 * w.Hkv) * w.D)).astype(np.float16)
    qkv[:, :w.Hq * w.D] = 0
    qkv[:, (w.Hq + w.Hkv) * w.D:] = odd[rng.integers(0, 4, size=(w.B, w.Hkv * w.D))]
    k = rng.standard_normal((w.B, w.Hkv, cap, w.D)).astype(np.float16)
    v = odd[rng.integers(0, 4, size=(w.B, w.Hkv, cap, w.D))]
    return qkv, k, v, np.full(w.B, L, np.int32)
