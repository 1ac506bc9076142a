"""Pins for the oracle's packing functions (CPU only)."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_canonical_worked_examples():
    for parts in _golden_lines("canonical_pack.txt"):
        codes = np.array([int(c) for c in parts[:8]], dtype=np.uint8).reshape(8, 1)
        word = int(parts[8], 16)
        packed = oracle.pack_canonical(codes)
        assert packed.shape == (1, 1)
        assert int(packed[0, 0]) == word
        assert np.array_equal(oracle.unpack_canonical(packed), codes)


def test_canonical_little_endian_bytes():
    # Byte b of a word holds row 8j+2b in its low nibble, 8j+2b+1 in its high.
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(64, 5), dtype=np.uint8)
    words = oracle.pack_canonical(q)
    as_bytes = words.astype("<u4").T.copy().view(np.uint8).reshape(5, -1)  # column-major bytes
    for n in range(5):
        lo = as_bytes[n] & 0xF
        hi = as_bytes[n] >> 4
        assert np.array_equal(lo, q[0::2, n])
        assert np.array_equal(hi, q[1::2, n])


def test_canonical_exhaustive_slots():
    # Every value in every slot, alone: exactly one nibble set, at bits 4i.
    for i in range(8):
        for v in range(16):
            q = np.zeros((8, 1), dtype=np.uint8)
            q[i, 0] = v
            assert int(oracle.pack_canonical(q)[0, 0]) == v << (4 * i)


def test_canonical_roundtrip_and_low_nibble():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 256, size=(256, 40), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_canonical(oracle.pack_canonical(q)), q & 0xF)


def test_zeros_packing_along_n():
    z = np.arange(16, dtype=np.uint8).reshape(1, 16)
    w = oracle.pack_zeros(z)
    assert w.shape == (1, 2)
    assert int(w[0, 0]) == 0x76543210 and int(w[0, 1]) == 0xFEDCBA98
    rng = np.random.default_rng(1)
    z = rng.integers(0, 16, size=(7, 64), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_zeros(oracle.pack_zeros(z)), z)
    with pytest.raises(ValueError):
        oracle.pack_zeros(np.zeros((2, 12), np.uint8))


def test_device_golden_words():
    K, N = 128, 16
    q = (np.arange(K)[:, None] % 16 * np.ones((1, N), int)).astype(np.uint8)
    words = oracle.pack_device(q)
    assert words.size == 256
    for parts in _golden_lines("device_layout_words.txt"):
        if parts[0] == "tile":
            continue
        assert int(words[int(parts[0])]) == int(parts[1], 16), parts


def test_device_tile_order_golden():
    K, N = 256, 32
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    q = (2 * (kk // 128) + nn // 16).astype(np.uint8)
    words = oracle.pack_device(q).reshape(4, 256)
    for parts in _golden_lines("device_layout_words.txt"):
        if parts[0] != "tile":
            continue
        assert np.all(words[int(parts[1])] == int(parts[2], 16)), parts


@pytest.mark.parametrize("K,N", [(128, 16), (256, 48), (96, 24), (384, 8), (32, 40)])
def test_device_bijection_and_padding(K, N):
    # Give every (k, n) a distinct tag split over several packs: each tag must
    # land in exactly one nibble, and padding nibbles must be zero.
    n_words = oracle.device_words(K, N)
    KT, NT = -(-K // 128), -(-N // 16)
    assert n_words == NT * KT * 256
    idx = np.arange(K * N).reshape(K, N)
    digits = []
    for digit in range(8):  # base-16 digits of the position id
        q = ((idx >> (4 * digit)) & 0xF).astype(np.uint8)
        w = oracle.pack_device(q)
        nib = np.stack([(w >> np.uint32(4 * p)) & np.uint32(0xF) for p in range(8)], 1)
        digits.append(nib.astype(np.int64))
    recon = sum(d << (4 * i) for i, d in enumerate(digits))  # [words, 8] position ids
    # Locate each (k, n) id; padding nibbles decode to id 0, which also belongs
    # to (0, 0): count that one separately.
    flat = recon.reshape(-1)
    counts = np.bincount(flat, minlength=K * N)
    pad = NT * KT * 256 * 8 - K * N
    assert counts[0] == 1 + pad
    assert np.all(counts[1:] == 1)
    assert np.array_equal(oracle.unpack_device(oracle.pack_device(idx % 16), K, N), (idx % 16).astype(np.uint8))


def test_device_word_structure():
    # Every word covers 8 consecutive rows of one column, starting at a
    # multiple of 8; the nibble pairs (0,4), (1,5), (2,6), (3,7) -- the pairs a
    # 16-bit-lane decode extracts -- hold rows (k0, k0+1), (k0+2, k0+3), ...
    K, N = 256, 32
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    wk = [oracle.pack_device(((kk >> (4 * d)) & 0xF).astype(np.uint8)) for d in range(2)]
    wn = [oracle.pack_device(((nn >> (4 * d)) & 0xF).astype(np.uint8)) for d in range(2)]

    def nib(ws, p):
        return sum(((w >> np.uint32(4 * p)) & np.uint32(0xF)).astype(np.int64) << (4 * d)
                   for d, w in enumerate(ws))

    order = [0, 4, 1, 5, 2, 6, 3, 7]  # nibble positions of rows k0+0 .. k0+7
    k0 = nib(wk, 0)
    n0 = nib(wn, 0)
    assert np.all(k0 % 8 == 0)
    for e, p in enumerate(order):
        assert np.array_equal(nib(wk, p), k0 + e)
        assert np.array_equal(nib(wn, p), n0)
    # Lane l = w//4 of a tile holds column l mod 16; its four words (a 16-byte
    # chunk) hold rows 32*slot + 8*(l div 16) inside the tile.
    w = np.arange(k0.size)
    lane = (w % 256) // 4
    slot = w % 4
    assert np.array_equal(n0 % 16, lane % 16)
    assert np.array_equal(k0 % 128, 32 * slot + 8 * (lane // 16))
