"""Plain CPU oracle for the W4A8-FP8 form of the group-quantised linear layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library never calls it and the two share no code.

What the pages fix and what is a reading
----------------------------------------
The TensorRT-LLM news page (Falcon-180B on one H200 with INT4 AWQ) says the
AWQ kernels there compute in FP8: 4-bit weights, 8-bit floating-point
activations. Nothing else is printed. The readings taken here:

* FP8 is the OCP E4M3 ("e4m3fn") format: 1 sign, 4 exponent bits (bias 7),
  3 mantissa bits, no infinities, largest finite value 448, smallest
  subnormal 2^-9; conversion rounds to nearest, ties to even;
* activations are quantised per row (per token), dynamically, with the
  row's largest magnitude mapped to 448. Each step is one IEEE float32
  operation in this order (the same order on both sides, because these
  roundings decide integer codes):
      amax = max_k |x[m, k]|                (exact)
      inv  = fp32(448 / amax)
      code = fp8(fp32(x[m, k] * inv))
      sx   = fp32(amax / 448)
  and a row of zeros gets codes 0 and sx = 0;
* the weight of the layer is unchanged, (q - z) * s with (q - z) an integer
  in [-15, 15] (exact in E4M3) and s the fp16 group scale, so
      y[m, n] = fp16( sx[m] * sum_g s[g, n] * sum_{k in g} x8[m, k] * (q[k, n] - z[g, n]) )
  with the real values of the codes x8; the oracle evaluates it in fp64.

Parity status: pinned by ``-m "not gpu"`` tests against an independent
enumeration of every E4M3 value, closed cases and the W4A16 oracle.
"""
from __future__ import annotations

import numpy as np

from .awq_oracle import dequant64

FP8_MAX = 448.0


def fp8_e4m3_value(code) -> np.ndarray:
    """Real value (fp64) of E4M3 codes (uint8). NaN for the two NaN codes."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(v) -> np.ndarray:
    """Round real values (given as float64, e.g. float32 results) to the
    nearest E4M3 code, ties to even. |v| must not exceed 464 (the midpoint
    above 448; larger values are outside the reading). Signed zeros kept."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) >= 464.0):
        raise ValueError("value outside the E4M3 range of this reading")
    a = np.abs(v)
    sign = np.signbit(v).astype(np.int64) << 7
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # log2 can be off by one next to powers of two: fix so 2^e <= a < 2^(e+1)
    e = np.where(np.exp2(e.astype(np.float64)) > a, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= a, e + 1, e)
    e = np.maximum(e, -6)                       # below 2^-6: subnormal spacing 2^-9
    quantum = np.exp2((e - 3).astype(np.float64))
    r = np.rint(a / quantum).astype(np.int64)   # ties to even (exact division by a power of two)
    carry = r == 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r)
    normal = r >= 8
    field_e = np.where(normal, e + 7, 0)
    field_m = np.where(normal, r - 8, r)
    code = sign | (field_e << 3) | field_m
    code = np.where(a == 0, sign, code)
    return code.astype(np.uint8)


def quantize_act_fp8(x: np.ndarray):
    """Per-row FP8 quantisation of fp16 activations x [M, K] ->
    (codes uint8 [M, K], sx float32 [M]), the float32 steps of the reading."""
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    codes = np.zeros(x32.shape, np.uint8)
    sx = np.zeros(x32.shape[0], np.float32)
    for m in range(x32.shape[0]):
        if amax[m] == 0:
            continue
        inv = np.float32(FP8_MAX) / amax[m]              # float32 division
        prod = (x32[m] * inv).astype(np.float32)        # float32 multiply
        codes[m] = fp8_e4m3_encode(prod.astype(np.float64))
        sx[m] = amax[m] / np.float32(FP8_MAX)
    return codes, sx


def linear_w4a8_64(codes, sx, q, z, s, G):
    """fp64 value of the W4A8 layer from the activation codes and row scales."""
    xv = fp8_e4m3_value(codes) * np.asarray(sx, np.float64)[:, None]
    return xv @ dequant64(q, z, s, G)


def w4a8_l1_scale(codes, sx, q, z, s, G):
    """Error scale sum_k |x8 sx| |w| (the W4A16 scale with the quantised
    activations): the kernel's fp32 sums and fp16 output round within it."""
    xv = np.abs(fp8_e4m3_value(codes) * np.asarray(sx, np.float64)[:, None])
    return xv @ np.abs(dequant64(q, z, s, G))
