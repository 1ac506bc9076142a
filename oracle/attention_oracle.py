"""Plain CPU oracle for the fused decode-step attention (fp64).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library never calls it and the two share no code.

What the pages fix and what is a reading
----------------------------------------
"TinyChat: Efficient and Lightweight Chatbot with AWQ", section *Speed
Benchmarks*: in the generation stage every operation of multi-head,
grouped-query and multi-query attention (MHA / GQA / MQA) runs in one kernel,
the positional-embedding kernels are fused into it, and the key-value caches
are allocated once up front. The pages define neither the attention nor the
embedding; the readings taken here are the textbook ones of the models in
that section's tables (LLaMA-2/3, Vicuna, Falcon):

* one new token per sequence b, at position ``L = lengths[b]`` (the number of
  tokens already cached); its q, k, v come from the QKV projection's output
  row ``qkv[b]`` laid out as [Hq query heads | Hkv key heads | Hkv value
  heads], D values per head;
* rotary position embedding: the pairs of a head vector are rotated by the
  angle ``L * theta**(-2i/D)`` for pair i (i = 0 .. D/2-1), counter-clockwise,
  ``(a, b) -> (a cos t - b sin t, a sin t + b cos t)``; the pairs are either
  (i, i + D/2) ("half", the LLaMA/Falcon form) or (2i, 2i+1) ("interleaved");
  "none" leaves the vectors as they are. q and k are rotated, v is not;
* the cache holds fp16 values: the new key is stored as the rotated key
  rounded once to fp16 (round-to-nearest-even), the new value as given;
  cached keys were rotated when they were stored and are not rotated again;
* query head h reads key/value head ``h // (Hq // Hkv)``;
* scaled dot-product attention over the L cached tokens and the new one:
  ``o = softmax(scale * K q) V`` with ``scale = 1/sqrt(D)`` unless given;
* the output row ``out[b]`` is [Hq, D] flattened, rounded to fp16 by the
  kernel (the oracle returns fp64).

Parity status: every function is pinned by ``-m "not gpu"`` tests against
other formulations (complex rotation, torch's scaled-dot-product attention,
composition and relative-position identities, closed cases).
"""
from __future__ import annotations

import numpy as np

ROPE_STYLES = ("none", "half", "interleaved")


def rope_inv_freq64(D: int, theta: float) -> np.ndarray:
    """Rotation rate of pair i: theta ** (-2i / D), i = 0 .. D/2 - 1."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / D)


def rope_pairs(D: int, style: str):
    """Index arrays (first, second) of the rotated pairs."""
    if style == "half":
        a = np.arange(D // 2)
        return a, a + D // 2
    if style == "interleaved":
        a = np.arange(0, D, 2)
        return a, a + 1
    raise ValueError(f"no pairs for rope style {style!r}")


def rope64(x: np.ndarray, pos, theta: float, style: str) -> np.ndarray:
    """Rotary embedding of x [..., D] at integer position(s) ``pos``
    (a scalar, or an array broadcast against x's leading axes)."""
    x = np.asarray(x, dtype=np.float64)
    if style == "none":
        return x.copy()
    D = x.shape[-1]
    first, second = rope_pairs(D, style)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq64(D, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., first], x[..., second]
    out = np.empty_like(x)
    out[..., first] = a * c - b * s
    out[..., second] = a * s + b * c
    return out


def split_qkv(qkv_row: np.ndarray, Hq: int, Hkv: int, D: int):
    """One row of the QKV output -> q [Hq, D], k [Hkv, D], v [Hkv, D] (fp64)."""
    r = np.asarray(qkv_row, dtype=np.float64)
    q = r[:Hq * D].reshape(Hq, D)
    k = r[Hq * D:(Hq + Hkv) * D].reshape(Hkv, D)
    v = r[(Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(Hkv, D)
    return q, k, v


def softmax64(s: np.ndarray) -> np.ndarray:
    """Softmax along the last axis, shifted by the maximum (same value, no
    overflow)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def decode_step64(qkv, k_cache, v_cache, lengths, Hq, Hkv, D, theta=10000.0, style="half", scale=None):
    """One generation step of attention for B sequences.

    qkv      [B, >= (Hq + 2 Hkv) D] fp16 (the QKV projection's output rows)
    k_cache  [B, Hkv, S, D] fp16, v_cache [B, Hkv, S, D] fp16 (logical layout;
             positions 0 .. lengths[b]-1 are read)
    lengths  [B] tokens already cached (the new token's position)

    Returns (out [B, Hq, D] fp64, k_new [B, Hkv, D] fp16, v_new [B, Hkv, D]
    fp16): the attention output and the key/value the step appends at
    position lengths[b]."""
    qkv = np.asarray(qkv)
    B = qkv.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((B, Hq, D))
    k_new = np.zeros((B, Hkv, D), np.float16)
    v_new = np.zeros((B, Hkv, D), np.float16)
    for b in range(B):
        L = int(lengths[b])
        q, k, v = split_qkv(qkv[b], Hq, Hkv, D)
        q_rot = rope64(q, L, theta, style)
        k_store = rope64(k, L, theta, style).astype(np.float16)
        k_new[b] = k_store
        v_new[b] = np.asarray(qkv[b], np.float16)[(Hq + Hkv) * D:(Hq + 2 * Hkv) * D].reshape(Hkv, D)
        for h in range(Hq):
            j = h // g
            keys = np.concatenate([np.asarray(k_cache[b, j, :L], np.float64), k_store[j:j + 1].astype(np.float64)])
            vals = np.concatenate([np.asarray(v_cache[b, j, :L], np.float64), v[j:j + 1]])
            p = softmax64(scale * (keys @ q_rot[h]))
            out[b, h] = p @ vals
    return out, k_new, v_new


def decode_error_scale(qkv, k_cache, v_cache, lengths, Hq, Hkv, D, theta=10000.0, style="half", scale=None):
    """Per-output error scale E [B, Hq, D] for an fp32 kernel with fp16 inputs.

    With scores s_j = scale q.k_j, probabilities p_j and o = sum_j p_j v_j, a
    perturbation d_j of the scores moves o by sum_j p_j d_j (v_j - o) to first
    order. The kernel's score errors come from rounding the rotated q (and the
    new key) to fp16, at most 2^-11 * sigma with sigma = scale * max_j
    sum_d |q_d k_jd|; rounding the probabilities to fp16 moves o by at most
    2^-11 sum_j p_j |v_j|, and rounding o to fp16 by 2^-11 |o|. Hence
      E = (1 + sigma) * (sum_j p_j |v_jd| + |o_d|)
    and the bar is |o_kernel - o| <= tol * E with the 2^-11-sized terms well
    inside tol = 2e-3."""
    qkv = np.asarray(qkv)
    B = qkv.shape[0]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    E = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lengths[b])
        q, k, v = split_qkv(qkv[b], Hq, Hkv, D)
        q_rot = rope64(q, L, theta, style)
        k_store = rope64(k, L, theta, style).astype(np.float16).astype(np.float64)
        for h in range(Hq):
            j = h // g
            keys = np.concatenate([np.asarray(k_cache[b, j, :L], np.float64), k_store[j:j + 1]])
            vals = np.concatenate([np.asarray(v_cache[b, j, :L], np.float64), v[j:j + 1]])
            p = softmax64(scale * (keys @ q_rot[h]))
            o = p @ vals
            sigma = scale * np.max(np.abs(keys) @ np.abs(q_rot[h]))
            E[b, h] = (1.0 + sigma) * (p @ np.abs(vals) + np.abs(o))
    return E


def decode_bytes(B: int, lengths, Hq: int, Hkv: int, D: int) -> int:
    """Algorithmic HBM bytes of one step: the cached keys and values read
    (2 * 2 * D bytes per cached token and key/value head), the QKV rows read,
    the output written and the new key and value written."""
    cached = int(np.sum(np.asarray(lengths, dtype=np.int64)))
    return 4 * D * Hkv * cached + 2 * B * (Hq + 2 * Hkv) * D + 2 * B * Hq * D + 4 * B * Hkv * D
