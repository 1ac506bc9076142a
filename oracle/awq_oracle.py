"""Plain CPU oracle for the W4A16 group-quantised linear layer (fp64).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
library and its Python binding never call it, and the two share no code: this
file re-states every layout and rule from its written definition with numpy.

What the pages fix and what is a reading
----------------------------------------
* "TinyChat: Efficient and Lightweight Chatbot with AWQ", section *Usage*,
  step 3: weights are quantised to 4 bits (``--w_bit 4``) in groups of 128
  input channels (``--q_group_size 128``), 64 for Falcon-7B; step 4 runs the
  result as ``W4A16`` (4-bit weights, 16-bit activations).
* Section *Speed Benchmarks*: the INT4 path uses a W4A16 GPU kernel in the
  generation stage, compared against an FP16 baseline.
* The pages print neither the dequantisation rule nor a packing order. The
  readings taken here (each listed in the design notes) are:
    - W is [K, N] with K input channels, y[M, N] = x[M, K] . W[K, N];
    - q and z are unsigned 4-bit codes 0..15, s is an fp16 scale, one (z, s)
      pair per (group of G consecutive input channels, output column);
    - w[k, n] = (q[k, n] - z[k // G, n]) * s[k // G, n]   (asymmetric affine);
    - the dequantised fp16 weight is that exact product rounded once to fp16,
      round-to-nearest-even, with IEEE special cases;
    - the layer output is that sum rounded to fp16 (activations are 16-bit,
      so the layer output is too);
    - "canonical" packing: 8 codes per uint32 along K, least-significant
      nibble first; zero points 8 per uint32 along N, least-significant first;
    - the device layout (``pack_device``) is this library's own choice,
      defined in ``device_layout_doc`` below and in ``include/awq.h``.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against something other than itself (closed forms, an independent integer
rounding, exact rational brute force, the pages' printed size figures).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# ----------------------------------------------------------------------------
# Canonical interchange packing (reading: 8 codes per uint32, LSB first)
# ----------------------------------------------------------------------------


def low_nibble(a: np.ndarray) -> np.ndarray:
    """Codes are taken from the low 4 bits of each byte (reading for bytes
    above 15, which the pages never mention)."""
    return (np.asarray(a).astype(np.uint8) & np.uint8(0x0F))


def pack_canonical(q: np.ndarray) -> np.ndarray:
    """q uint8 [K, N] -> uint32 [K/8, N]; nibble i of word (j, n) is q[8j+i, n].

    Follows the 4-bit weight setting of the TinyChat README (*Usage*, step 3)
    with the least-significant-nibble-first reading."""
    q = low_nibble(q)
    K, N = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        out |= q[i::8, :].astype(np.uint32) << np.uint32(4 * i)
    return out


def unpack_canonical(words: np.ndarray) -> np.ndarray:
    """uint32 [K/8, N] -> uint8 [K, N] (inverse of ``pack_canonical``)."""
    words = np.asarray(words, dtype=np.uint32)
    K8, N = words.shape
    q = np.zeros((K8 * 8, N), dtype=np.uint8)
    for i in range(8):
        q[i::8, :] = ((words >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.uint8)
    return q


def pack_zeros(z: np.ndarray) -> np.ndarray:
    """z uint8 [K/G, N] -> uint32 [K/G, N/8]; nibble i of word (g, c) is
    z[g, 8c+i]. One zero point per (group, column), packed along N."""
    z = low_nibble(z)
    Gn, N = z.shape
    if N % 8:
        raise ValueError("N must be a multiple of 8")
    out = np.zeros((Gn, N // 8), dtype=np.uint32)
    for i in range(8):
        out |= z[:, i::8].astype(np.uint32) << np.uint32(4 * i)
    return out


def unpack_zeros(words: np.ndarray) -> np.ndarray:
    """uint32 [K/G, N/8] -> uint8 [K/G, N] (inverse of ``pack_zeros``)."""
    words = np.asarray(words, dtype=np.uint32)
    Gn, N8 = words.shape
    z = np.zeros((Gn, N8 * 8), dtype=np.uint8)
    for i in range(8):
        z[:, i::8] = ((words >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.uint8)
    return z


# ----------------------------------------------------------------------------
# Device layout, written from its definition
# ----------------------------------------------------------------------------

device_layout_doc = """
Tiles of 16 output columns x 128 input channels, 256 uint32 words each.
KT = ceil(K/128) tiles along K, NT = ceil(N/16) tiles along N; tile (t, kt)
begins at word (kt*NT + t)*256 (tiles of one 128-row band are adjacent).
Word w of a tile: lane l = w // 4, slot
j = w % 4; it holds column n = 16t + (l mod 16) and rows k0 .. k0+7 with
k0 = 128kt + 32j + 8(l // 16). Row k0+e sits in nibble position
p(e) = 4(e mod 2) + (e // 2) (bits 4p .. 4p+3). Rows k >= K and columns
n >= N hold code 0.
"""


def device_words(K: int, N: int) -> int:
    """Number of uint32 words of the device layout for a [K, N] code matrix."""
    KT = -(-K // 128)
    NT = -(-N // 16)
    return NT * KT * 256


def _device_coords(K: int, N: int):
    """For every device word: (column n, first row k0), as flat int64 arrays."""
    KT = -(-K // 128)
    NT = -(-N // 16)
    w = np.arange(NT * KT * 256, dtype=np.int64)
    tile = w // 256
    kt = tile // NT
    t = tile % NT
    within = w % 256
    lane = within // 4
    slot = within % 4
    n = 16 * t + (lane % 16)
    k0 = 128 * kt + 32 * slot + 8 * (lane // 16)
    return n, k0


def _nibble_position(e: int) -> int:
    return 4 * (e % 2) + (e // 2)


def pack_device(q: np.ndarray) -> np.ndarray:
    """q uint8 [K, N] -> uint32 device words (flat), per ``device_layout_doc``."""
    q = low_nibble(q)
    K, N = q.shape
    n, k0 = _device_coords(K, N)
    out = np.zeros(n.shape, dtype=np.uint32)
    for e in range(8):
        k = k0 + e
        ok = (k < K) & (n < N)
        vals = np.zeros(n.shape, dtype=np.uint32)
        vals[ok] = q[k[ok], n[ok]]
        out |= vals << np.uint32(4 * _nibble_position(e))
    return out


def unpack_device(words: np.ndarray, K: int, N: int) -> np.ndarray:
    """Device words -> uint8 [K, N] (inverse of ``pack_device`` on the valid
    region)."""
    words = np.asarray(words, dtype=np.uint32).reshape(-1)
    if words.size != device_words(K, N):
        raise ValueError("wrong number of device words")
    n, k0 = _device_coords(K, N)
    q = np.zeros((K, N), dtype=np.uint8)
    for e in range(8):
        k = k0 + e
        ok = (k < K) & (n < N)
        nib = (words >> np.uint32(4 * _nibble_position(e))) & np.uint32(0xF)
        q[k[ok], n[ok]] = nib[ok].astype(np.uint8)
    return q


# ----------------------------------------------------------------------------
# Dequantisation and the linear layer
# ----------------------------------------------------------------------------


def _check_groups(K: int, G: int, z: np.ndarray, s: np.ndarray, N: int):
    if G <= 0 or K % G:
        raise ValueError("K must be a positive multiple of the group size")
    if z.shape != (K // G, N) or s.shape != (K // G, N):
        raise ValueError("zeros/scales must be [K/G, N]")


def dequant64(q: np.ndarray, z: np.ndarray, s: np.ndarray, G: int) -> np.ndarray:
    """w64[k, n] = (q[k, n] - z[k//G, n]) * s[k//G, n] in float64.

    Group-wise 4-bit weights with group size G (TinyChat README, *Usage*,
    step 3: ``--w_bit 4 --q_group_size 128``; 64 for Falcon-7B). The product
    has at most 4 + 11 significant bits, so it is exact in float64."""
    q = low_nibble(q)
    z = low_nibble(z)
    s = np.asarray(s, dtype=np.float16)
    K, N = q.shape
    _check_groups(K, G, z, s, N)
    g = np.arange(K) // G
    diff = q.astype(np.float64) - z[g, :].astype(np.float64)
    return diff * s[g, :].astype(np.float64)


def dequant16(q: np.ndarray, z: np.ndarray, s: np.ndarray, G: int) -> np.ndarray:
    """The exact product rounded once to fp16 (round to nearest, ties to
    even): the value ``awq_dequant`` must reproduce bit for bit."""
    with np.errstate(over="ignore", invalid="ignore"):
        return dequant64(q, z, s, G).astype(np.float16)


def linear64(x: np.ndarray, q: np.ndarray, z: np.ndarray, s: np.ndarray,
             G: int) -> np.ndarray:
    """y64[M, N] = float64(x) @ w64: the W4A16 layer (4-bit weights, 16-bit
    activations; TinyChat README, *Usage*, step 4, ``--precision W4A16``),
    evaluated with the exact dequantised weights in float64."""
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    return x64 @ dequant64(q, z, s, G)


def l1_scale(x, q, z, s, G) -> np.ndarray:
    """D[m, n] = sum_k |x[m, k]| * |w64[k, n]|: the L1 norm of the products
    that make up output (m, n); the error of any summation order is bounded
    by a multiple of it."""
    x64 = np.abs(np.asarray(x, dtype=np.float16).astype(np.float64))
    return x64 @ np.abs(dequant64(q, z, s, G))


def normalised_error(yhat: np.ndarray, y64: np.ndarray, D: np.ndarray) -> float:
    """max |yhat - y64| / D over all outputs; where D == 0, yhat must be 0
    (returns inf otherwise)."""
    yhat = np.asarray(yhat, dtype=np.float64)
    diff = np.abs(yhat - y64)
    zero = D == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(diff[~zero] / D[~zero]))


def linear_bruteforce(x, q, z, s, G) -> list:
    """Exact rational result by triple loop (tiny shapes only):
    y[m][n] = sum_k x[m,k] * (q[k,n] - z[k//G,n]) * s[k//G,n]."""
    x = np.asarray(x, dtype=np.float16)
    q = low_nibble(q)
    z = low_nibble(z)
    s = np.asarray(s, dtype=np.float16)
    M, K = x.shape
    N = q.shape[1]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // G
                w = (int(q[k, n]) - int(z[g, n])) * Fraction(float(s[g, n]))
                acc += Fraction(float(x[m, k])) * w
            row.append(acc)
        out.append(row)
    return out


def round_output16(y64: np.ndarray) -> np.ndarray:
    """Layer output in fp16 (reading: 16-bit activations in, 16-bit out)."""
    with np.errstate(over="ignore"):
        return np.asarray(y64, dtype=np.float64).astype(np.float16)


# ----------------------------------------------------------------------------
# Gated epilogue: y = silu(gate) * up on a fused gate+up layer
# ----------------------------------------------------------------------------


def silu64(h: np.ndarray) -> np.ndarray:
    """silu(h) = h * sigmoid(h) = h / (1 + exp(-h)), in float64 (exp of a
    large positive -h overflows to inf and gives the correct limit 0)."""
    h = np.asarray(h, dtype=np.float64)
    with np.errstate(over="ignore"):
        return h / (1.0 + np.exp(-h))


def linear_silu_mul64(x, q, z, s, G) -> np.ndarray:
    """The fused gate+up projection of a gated MLP followed by its gate:
    h = x . W with W = [W_gate | W_up] (output columns 0 .. N/2-1 are the
    gate, N/2 .. N-1 the up projection), y[m, i] = silu(h[m, i]) * h[m, N/2+i].

    The pages measure LLaMA-family decoders ("TinyChat" README, *Speed
    Benchmarks*), whose MLP takes this form, and TinyChat fuses the small
    operators around its W4A16 kernels; the column order of the fused weight
    is not printed, so gate-then-up halves are the reading taken here."""
    h = linear64(x, q, z, s, G)
    n2 = h.shape[1] // 2
    return silu64(h[:, :n2]) * h[:, n2:]


def silu_mul_scale(x, q, z, s, G) -> np.ndarray:
    """Error scale of the gated output: 1.1 |u| D_gate + |silu(g)| D_up + |y|,
    with D the L1 norms of ``l1_scale`` (1.1 bounds |silu'|, so an error
    e_g in g and e_u in u moves y by at most 1.1 |u| e_g + |silu(g)| e_u);
    the |y| term covers the final fp16 rounding."""
    h = linear64(x, q, z, s, G)
    D = l1_scale(x, q, z, s, G)
    n2 = h.shape[1] // 2
    g, u = h[:, :n2], h[:, n2:]
    return 1.1 * np.abs(u) * D[:, :n2] + np.abs(silu64(g)) * D[:, n2:] + np.abs(silu64(g) * u)


# ----------------------------------------------------------------------------
# Round-to-nearest group quantiser (fp16 W -> q, z, s)
# ----------------------------------------------------------------------------

RTN_QMAX = 15  # 2^4 - 1 levels above code 0


def quantize_rtn(w: np.ndarray, G: int):
    """fp16 W [K, N] -> (q uint8 [K, N], z uint8 [K/G, N], s fp16 [K/G, N]).

    The step that makes the "real" INT4 weights before the W4A16 kernel runs
    (TinyChat README, *Usage*, step 3: ``--w_bit 4 --q_group_size 128``,
    ``--q_backend real``); the Sagemaker page names the plain variant,
    round-to-nearest (RTN), in its *GGUF* section. The pages print no formula;
    the reading taken here is the asymmetric min-max rule, per group of G
    input channels and per output column:

        lo, hi = min and max of the group's weights
        s      = fp16((hi - lo) / 15)           (1 if that rounds to 0)
        z      = clamp(rne(-lo / s), 0, 15)
        q[k]   = clamp(rne(w[k] / s) + z, 0, 15)

    rne = round half to even. Every operation is one IEEE float32 operation
    (difference, quotient, conversion), taken in that order: the pages fix no
    precision, so the integer decisions are made in the kernel's float32 and
    both sides reach the same codes. The dequantised weight (q - z) * s then
    lies within s/2 (plus the fp16 rounding of s) of w wherever lo <= 0 <= hi;
    a group that does not contain 0 has its zero point clamped (z = 0 or 15)
    and loses the end of its range. Inputs must be finite."""
    w = np.asarray(w, dtype=np.float16)
    K, N = w.shape
    if G <= 0 or K % G:
        raise ValueError("K must be a positive multiple of the group size")
    wg = w.reshape(K // G, G, N).astype(np.float32)
    lo = wg.min(axis=1)
    hi = wg.max(axis=1)
    s32 = (hi - lo) / np.float32(RTN_QMAX)
    s16 = s32.astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16).astype(np.float16)
    sf = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / sf), 0, RTN_QMAX)
    q = np.clip(np.rint(wg / sf[:, None, :]) + z[:, None, :], 0, RTN_QMAX)
    return (q.reshape(K, N).astype(np.uint8), z.astype(np.uint8), s16)


# ----------------------------------------------------------------------------
# Byte accounting (the size arithmetic the pages use)
# ----------------------------------------------------------------------------


def weight_set_bytes(K: int, N: int, G: int) -> int:
    """Bytes of the quantised weight set: K*N/2 (4-bit codes) + 2*N*K/G
    (fp16 scales) + N*K/(2G) (4-bit zero points).

    "Applied LLM Quantisation Sagemaker", *How does it help?*: a model's size
    scales with the bits per weight (16 -> 8 -> 4 halves and quarters it)."""
    return K * N // 2 + 2 * N * (K // G) + N * (K // G) // 2


def model_bytes(params: float, bits: float) -> float:
    """Naive size estimate: parameters x bits / 8 (same section)."""
    return params * bits / 8.0
