"""Pins for the oracle of the PQ2_0 and PTQ1_0 containers (oracle/formats.py):
checks against things other than that code -- the sizes the pages state,
the MLX container seen through numpy's byte view, a brute-force enumeration
of every trit byte, decode values written out by hand from the pages'
decode rule, and the (separately pinned) MLX oracle on the same weights.

Each pin takes the formats namespace `f` (the real one, or a copy with a
planted mistake) and raises AssertionError when it is violated.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _ternary(rng, N, K):
    return rng.integers(-1, 2, size=(N, K)).astype(np.int8)


def _scales(rng, N, K):
    return (np.abs(rng.normal(0, 0.02, size=(N, K // 128))) + 1e-3).astype(np.float16)


def _raises(fn, *args):
    try:
        fn(*args)
    except ValueError:
        return True
    return False


# ---------------------------------------------------------------------------
# PQ2_0
# ---------------------------------------------------------------------------
def pin_pq2_size(f):
    """[P2 "packing-format engineering"] 34 bytes per 128 weights, 2.125 bits."""
    rng = _rng(1)
    for N, K in ((1, 128), (5, 1024), (3, 5120)):
        c, s, b = oracle.pack(_ternary(rng, N, K), _scales(rng, N, K))
        pq = f.pq2_from_mlx(c, s, b)
        assert pq.dtype == np.uint8 and pq.size == N * K * 34 // 128
        assert pq.size * 8 == N * K * 2.125


def pin_pq2_bytes_are_the_mlx_words(f):
    """Block g of row n = the fp16 scale's bytes, then the group's eight MLX
    code words as little-endian bytes (numpy byte views, not shifts)."""
    rng = _rng(2)
    N, K = 4, 1024
    c, s, b = oracle.pack(_ternary(rng, N, K), _scales(rng, N, K))
    pq = f.pq2_from_mlx(c, s, b).reshape(N, K // 128, 34)
    for n in range(N):
        for g in range(K // 128):
            assert bytes(pq[n, g, :2]) == s[n, g:g + 1].astype("<f2").tobytes()
            assert bytes(pq[n, g, 2:]) == c[n, 8 * g:8 * g + 8].astype("<u4").tobytes()


def pin_pq2_roundtrip_and_scale_bitcompare(f):
    """Lossless transcode both ways; the group scales compare bit for bit."""
    rng = _rng(3)
    N, K = 7, 2048
    c, s, b = oracle.pack(_ternary(rng, N, K), _scales(rng, N, K))
    c2, s2, b2 = f.pq2_to_mlx(f.pq2_from_mlx(c, s, b), K)
    assert np.array_equal(c2, c)
    assert np.array_equal(np.asarray(s2).view(np.uint16), np.asarray(s).view(np.uint16))
    assert np.array_equal(np.asarray(b2).view(np.uint16), np.asarray(b).view(np.uint16))


def pin_pq2_rejects_what_it_cannot_hold(f):
    rng = _rng(4)
    N, K = 2, 256
    c, s, b = oracle.pack(_ternary(rng, N, K), _scales(rng, N, K))
    b_bad = b.copy()
    b_bad[1, 1] = np.float16(-0.5) if b_bad[1, 1] != np.float16(-0.5) else np.float16(-0.25)
    assert _raises(f.pq2_from_mlx, c, s, b_bad)
    c3 = c.copy()
    c3[0, 3] |= np.uint32(3) << np.uint32(10)   # code 5 of word 3 becomes 3
    assert _raises(f.pq2_from_mlx, c3, s, b)
    pq = f.pq2_from_mlx(c, s, b)
    pq[1, 2 + 34] |= 0xC0                        # a code 3 in block 1 of row 1
    assert _raises(f.pq2_to_mlx, pq, K)


def pin_pq2_hand_decoded_block(f):
    """A block written by hand: scale 0.5 (fp16 0x3800: bytes 00 38), every
    code byte 0x24 = 0b00100100, i.e. codes 0, 1, 2, 0 from the low bits up.
    Codes {0, 1, 2} are -d, 0, +d [P2 "packing-format engineering"], so the
    weights repeat -0.5, 0, 0.5, -0.5."""
    blk = np.array([[0x00, 0x38] + [0x24] * 32], np.uint8)
    w = f.pq2_dequantize_rows(blk, 128, [0])[0]
    assert np.array_equal(w, np.tile([-0.5, 0.0, 0.5, -0.5], 32))


def pin_pq2_decode_and_linear_equal_mlx(f):
    rng = _rng(5)
    N, K = 33, 2048
    t = _ternary(rng, N, K)
    c, s, b = oracle.pack(t, _scales(rng, N, K))
    pq = f.pq2_from_mlx(c, s, b)
    assert np.array_equal(f.pq2_dequantize_rows(pq, K, np.arange(N)), oracle.dequantize(c, s, b, K))
    sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((3, K))
    want = oracle.packed_linear(x, sig, 1024, c, s, b)
    got = f.pq2_packed_linear(x, sig, 1024, pq, K)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


# ---------------------------------------------------------------------------
# PTQ1_0
# ---------------------------------------------------------------------------
def pin_ptq1_size(f):
    """[P2 "packing-format engineering"] 28 bytes per 128 weights, 1.75 bits."""
    rng = _rng(6)
    for N, K in ((1, 128), (4, 1024), (2, 5120)):
        pt = f.ptq1_pack(_ternary(rng, N, K), _scales(rng, N, K))
        assert pt.dtype == np.uint8 and pt.size == N * K * 28 // 128
        assert pt.size * 8 == N * K * 1.75


def pin_ptq1_every_trit_byte_by_enumeration(f):
    """All 243 patterns of five codes: itertools.product counts in base 3
    with its LAST element as the lowest digit, so pattern k (k = 0..242),
    read backwards as codes c0..c4, is exactly the byte k under the reading
    'first code = lowest digit'.  Row k carries pattern k in codes 0..4 of
    its block (the rest t = 0), and byte 2 of its block must be k."""
    pats = list(itertools.product(range(3), repeat=5))
    t = np.zeros((243, 128), np.int8)
    for k, tup in enumerate(pats):
        t[k, :5] = np.array(tup[::-1], np.int8) - 1
    sc = np.full((243, 1), 0.25, np.float16)
    pt = f.ptq1_pack(t, sc)
    assert np.array_equal(pt[:, 2], np.arange(243, dtype=np.uint8))
    # the other full bytes hold five codes 1 (t = 0): 1 + 3 + 9 + 27 + 81
    assert (pt[:, 3:27] == 121).all()
    # the last byte holds codes 125..127 only: 1 + 3 + 9
    assert (pt[:, 27] == 13).all()
    back, s2 = f.ptq1_unpack(pt, 128)
    assert np.array_equal(back, t)


def pin_ptq1_last_byte_by_enumeration(f):
    pats = list(itertools.product(range(3), repeat=3))
    t = np.zeros((27, 128), np.int8)
    for k, tup in enumerate(pats):
        t[k, 125:] = np.array(tup[::-1], np.int8) - 1
    pt = f.ptq1_pack(t, np.full((27, 1), 1.0, np.float16))
    assert np.array_equal(pt[:, 27], np.arange(27, dtype=np.uint8))


def pin_ptq1_roundtrip_and_scale_bitcompare(f):
    rng = _rng(7)
    N, K = 9, 3072
    t = _ternary(rng, N, K)
    sc = _scales(rng, N, K)
    pt = f.ptq1_pack(t, sc)
    t2, s2 = f.ptq1_unpack(pt, K)
    assert np.array_equal(t2, t)
    assert np.array_equal(np.asarray(s2).view(np.uint16), sc.view(np.uint16))
    assert bytes(pt.reshape(N, K // 128, 28)[2, 3, :2]) == sc[2, 3:4].astype("<f2").tobytes()


def pin_ptq1_rejects_invalid_bytes(f):
    rng = _rng(8)
    pt = f.ptq1_pack(_ternary(rng, 2, 256), _scales(rng, 2, 256))
    bad = pt.copy()
    bad[0, 2 + 7] = 243
    assert _raises(f.ptq1_unpack, bad, 256)
    bad = pt.copy()
    bad[1, 28 + 27] = 27                       # last byte of block 1 of row 1
    assert _raises(f.ptq1_unpack, bad, 256)
    t = _ternary(rng, 1, 128)
    t[0, 5] = 2
    assert _raises(f.ptq1_pack, t, _scales(rng, 1, 128))


def pin_ptq1_hand_decoded_block(f):
    """A block written by hand: scale 2.0 (fp16 0x4000: bytes 00 40); byte
    0x0B = 11 = 2 + 0*3 + 1*9 holds codes 2, 0, 1, 0, 0 (lowest digit
    first), i.e. weights +2, -2, 0, -2, -2.  Every other byte is 0 (all codes
    0: weights -2)."""
    blk = np.zeros((1, 28), np.uint8)
    blk[0, 1] = 0x40
    blk[0, 2] = 0x0B
    w = f.ptq1_dequantize_rows(blk, 128, [0])[0]
    want = np.full(128, -2.0)
    want[:5] = [2.0, -2.0, 0.0, -2.0, -2.0]
    assert np.array_equal(w, want)


def pin_ptq1_decode_and_linear_equal_mlx(f):
    rng = _rng(9)
    N, K = 21, 2048
    t = _ternary(rng, N, K)
    sc = _scales(rng, N, K)
    c, s, b = oracle.pack(t, sc)
    pt = f.ptq1_pack(t, sc)
    assert np.array_equal(f.ptq1_dequantize_rows(pt, K, np.arange(N)), oracle.dequantize(c, s, b, K))
    sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((2, K))
    want = oracle.packed_linear(x, sig, 1024, c, s, b)
    got = f.ptq1_packed_linear(x, sig, 1024, pt, K)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


PINS_FORMATS = [
    pin_pq2_size, pin_pq2_bytes_are_the_mlx_words, pin_pq2_roundtrip_and_scale_bitcompare,
    pin_pq2_rejects_what_it_cannot_hold, pin_pq2_hand_decoded_block, pin_pq2_decode_and_linear_equal_mlx,
    pin_ptq1_size, pin_ptq1_every_trit_byte_by_enumeration, pin_ptq1_last_byte_by_enumeration,
    pin_ptq1_roundtrip_and_scale_bitcompare, pin_ptq1_rejects_invalid_bytes, pin_ptq1_hand_decoded_block,
    pin_ptq1_decode_and_linear_equal_mlx,
]
