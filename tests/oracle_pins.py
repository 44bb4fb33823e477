"""Pins for the fp64 oracle: checks against things other than the oracle
itself -- the hand examples in tests/golden, scipy's Sylvester Hadamard
matrix, brute-force dense products, closed forms and invariants.

Each pin takes an oracle namespace `o` (the real oracle, or a copy with a
planted mistake) and raises AssertionError when the oracle violates it.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.linalg

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _ternary(rng, N, K):
    return rng.integers(-1, 2, size=(N, K)).astype(np.int8)


def _scales(rng, N, K):
    return (np.abs(rng.normal(0, 0.02, size=(N, K // 128))) + 1e-3).astype(np.float16)


def _dense_rotation(signs, block):
    """R = blockdiag(H/sqrt(block)) @ diag(signs) built from scipy's Sylvester matrix."""
    K = signs.size
    Hn = scipy.linalg.hadamard(block).astype(np.float64) / math.sqrt(block)
    R = np.zeros((K, K))
    for j in range(K // block):
        R[j * block:(j + 1) * block, j * block:(j + 1) * block] = Hn
    return R @ np.diag(signs.astype(np.float64))


def _w_true(t, scales):
    """Dense weights straight from the ternary draws: s * t (bias = -s means
    code t+1 decodes to s*(t+1) - s = s*t)."""
    g = np.arange(t.shape[1]) // 128
    return scales.astype(np.float64)[:, g] * t.astype(np.float64)


# ---------------------------------------------------------------------------
# transform
# ---------------------------------------------------------------------------
def pin_fwht_matches_scipy(o):
    """I3/I14: butterfly transform == scipy.linalg.hadamard(L)/sqrt(L) @ x blockwise."""
    rng = _rng(11)
    for L in (512, 1024, 2048):
        x = rng.standard_normal((3, 2 * L))
        Hn = scipy.linalg.hadamard(L).astype(np.float64) / math.sqrt(L)
        want = np.concatenate([x[:, :L] @ Hn.T, x[:, L:] @ Hn.T], axis=1)
        got = o.fwht_blocks(x, L)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_fwht_closed_forms(o):
    """I3: H e0 = ones/32, H ones = 32 e0, H e1 = alternating/32 (natural order)."""
    L = 1024
    e0 = np.zeros(L); e0[0] = 1
    e1 = np.zeros(L); e1[1] = 1
    np.testing.assert_array_equal(o.fwht_blocks(e0, L), np.full(L, 1 / 32))
    want = np.zeros(L); want[0] = 32
    np.testing.assert_array_equal(o.fwht_blocks(np.ones(L), L), want)
    alt = np.where(np.arange(L) % 2 == 0, 1.0, -1.0) / 32
    np.testing.assert_array_equal(o.fwht_blocks(e1, L), alt)


def pin_hh_identity(o):
    """I1: the normalized matrix has entries +-1/32 and H H = I exactly in fp64."""
    L = 1024
    H = o.fwht_blocks(np.eye(L), L)       # row i = H e_i = column i (H symmetric)
    assert np.all(np.abs(H) == 1 / 32)
    np.testing.assert_array_equal(H @ H, np.eye(L))
    np.testing.assert_array_equal(H, H.T)


def pin_parseval(o):
    """I5: ||fwht(x)|| = ||x|| for the signed forward transform."""
    rng = _rng(12)
    x = rng.standard_normal((4, 5120))
    s = np.where(rng.random(5120) < 0.5, -1, 1).astype(np.int8)
    y = o.fwht_signed(x, s, 1024)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def pin_inverse_undoes_forward(o):
    """I2: inverse(forward(x)) = x and forward(inverse(x)) = x."""
    rng = _rng(13)
    for L in (512, 1024, 4096):
        K = 2 * L if L < 4096 else L
        x = rng.standard_normal((2, K))
        s = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
        np.testing.assert_allclose(o.fwht_signed(o.fwht_signed(x, s, L), s, L, inverse=True), x, atol=1e-13)
        np.testing.assert_allclose(o.fwht_signed(o.fwht_signed(x, s, L, inverse=True), s, L), x, atol=1e-13)


def pin_sign_handling(o):
    """I4 and the golden rotated example: all signs -1 negate the forward output;
    signs are applied before the transform (forward) and after it (inverse)."""
    rng = _rng(14)
    K = 2048
    x = rng.standard_normal((2, K))
    plus = np.ones(K, np.int8)
    minus = -plus
    np.testing.assert_array_equal(o.fwht_signed(x, minus, 1024), -o.fwht_signed(x, plus, 1024))
    s = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    R = _dense_rotation(s, 1024)
    np.testing.assert_allclose(o.fwht_signed(x, s, 1024), x @ R.T, atol=1e-12)
    np.testing.assert_allclose(o.fwht_signed(x, s, 1024, inverse=True), x @ R, atol=1e-12)


def pin_rejects_bad_signs(o):
    """Contract v1: signs must all be +-1; blocks other than 512..4096 refused."""
    x = np.zeros((1, 1024))
    bad = np.ones(1024, np.int8); bad[7] = 0
    for call in (lambda: o.fwht_signed(x, bad, 1024),
                 lambda: o.fwht_signed(x, np.ones(1024, np.int8), 256)):
        try:
            call()
        except ValueError:
            continue
        raise AssertionError("invalid sign vector / block accepted")


# ---------------------------------------------------------------------------
# container
# ---------------------------------------------------------------------------
def pin_golden_words(o):
    """Hand example: exact uint32 words and outputs of the unrotated case."""
    g = _golden("hand_examples.json")["unrotated"]
    N, K = g["N"], g["K"]
    t = np.zeros((N, K), np.int8)
    t[0, :64] = 1
    t[0, 64:] = -1
    t[1, 5] = 1
    sc = np.array(g["scales"], np.float16).reshape(N, 1)
    codes, s2, b2 = o.pack(t, sc)
    want = np.array([[int(h, 16) for h in row] for row in g["expected_words_hex"]], np.uint32)
    np.testing.assert_array_equal(codes, want)
    np.testing.assert_array_equal(b2, -sc)
    x = np.arange(K, dtype=np.float64)[None, :]
    y = o.packed_linear(x, None, 0, codes, s2, b2)
    np.testing.assert_array_equal(y[0], np.array(g["expected_y"]))


def pin_golden_rotated(o):
    """Hand example: rotated case with one-hot inputs and the embedding rows."""
    g = _golden("hand_examples.json")["rotated"]
    N, K = g["N"], g["K"]
    t = np.ones((N, K), np.int8)
    t[1, 1::2] = -1
    sc = np.full((N, K // 128), g["scale"], np.float16)
    codes, s2, b2 = o.pack(t, sc)
    for case in g["cases"]:
        s = np.full(K, 1 if case["signs"] == "+1" else -1, np.int8)
        x = np.zeros((1, K)); x[0, 0 if case["x"] == "e0" else 1] = 1
        y = o.packed_linear(x, s, g["block"], codes, s2, b2)
        np.testing.assert_array_equal(y[0], np.array(case["expected_y"]))
    e = o.embed_inverse([0, 1], codes, s2, b2, np.ones(K, np.int8), g["block"])
    want = np.zeros((2, K)); want[0, 0] = 32; want[1, 1] = 32
    np.testing.assert_array_equal(e, want)


def pin_pack_bitwise(o):
    """I8: codes equal a bit-by-bit packer (pure Python) and the 4-codes-per-
    byte view of the words (little endian) holds symbol j at bits 2j."""
    rng = _rng(15)
    N, K = 3, 256
    t = _ternary(rng, N, K)
    codes, _, _ = o.pack(t, _scales(rng, N, K))
    for n in range(N):
        for w in range(K // 16):
            v = 0
            for j in range(16):
                v |= (int(t[n, 16 * w + j]) + 1) << (2 * j)
            assert int(codes[n, w]) == v, (n, w)
    by = codes.view(np.uint8)
    for n in range(N):
        for k in range(K):
            assert (int(by[n, k // 4]) >> (2 * (k % 4))) & 3 == int(t[n, k]) + 1


def pin_unpack_roundtrip(o):
    """I8: unpack(pack(t)) == t bit-exactly; code 3 is rejected."""
    rng = _rng(16)
    t = _ternary(rng, 17, 1024)
    codes, _, _ = o.pack(t, _scales(rng, 17, 1024))
    np.testing.assert_array_equal(o.unpack(codes, 1024), t)
    bad = codes.copy()
    bad[3, 5] |= np.uint32(3 << 6)
    try:
        o.unpack(bad, 1024)
    except ValueError:
        return
    raise AssertionError("code 3 accepted by unpack")


def pin_container_size(o):
    """I9: container bytes = N*K*9/32 (2.25 bits/weight), matching the array sizes."""
    g = _golden("hand_examples.json")["container_bytes"]
    for c in g["cases"]:
        assert o.container_bytes(c["N"], c["K"]) == c["bytes"]
    rng = _rng(17)
    t = _ternary(rng, 8, 1024)
    codes, s, b = o.pack(t, _scales(rng, 8, 1024))
    assert codes.nbytes + s.nbytes + b.nbytes == o.container_bytes(8, 1024) == 8 * 1024 * 9 // 32


def pin_decode_values(o):
    """I10: code q decodes to s*q + b with the stored (arbitrary) bias, per group;
    checked element by element in pure Python on a tiny container."""
    rng = _rng(18)
    N, K = 2, 256
    c = rng.integers(0, 4, size=(N, K))
    words = np.zeros((N, K // 16), np.uint32)
    for n in range(N):
        for k in range(K):
            words[n, k // 16] |= np.uint32(int(c[n, k]) << (2 * (k % 16)))
    sc = np.array([[0.5, -0.75], [3.0, 0.125]], np.float16)
    bi = np.array([[0.25, 1.5], [-2.0, 7.0]], np.float16)
    W = o.dequantize(words, sc, bi, K)
    for n in range(N):
        for k in range(K):
            g = k // 128
            assert W[n, k] == float(sc[n, g]) * int(c[n, k]) + float(bi[n, g]), (n, k)


def pin_zero_weights(o):
    """I11: all ternary zeros give W~ = 0 and y = 0 exactly."""
    rng = _rng(19)
    t = np.zeros((5, 2048), np.int8)
    codes, s, b = o.pack(t, _scales(rng, 5, 2048))
    x = rng.standard_normal((2, 2048))
    sig = np.where(rng.random(2048) < 0.5, -1, 1).astype(np.int8)
    np.testing.assert_array_equal(o.packed_linear(x, sig, 1024, codes, s, b), np.zeros((2, 5)))


# ---------------------------------------------------------------------------
# the Packed linear and the embedding
# ---------------------------------------------------------------------------
def pin_folded_rotation_bruteforce(o):
    """I6: W~ (R x) == (W~ R) x with dense fp64 matrices built from the ternary
    draws and scipy's Hadamard matrix, N <= 64, K in {1024, 2048}, distinct
    signs per block."""
    rng = _rng(20)
    for N, K in ((64, 1024), (48, 2048), (7, 2048)):
        t = _ternary(rng, N, K)
        sc = _scales(rng, N, K)
        sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
        x = rng.standard_normal((3, K))
        codes, s2, b2 = o.pack(t, sc)
        got = o.packed_linear(x, sig, 1024, codes, s2, b2)
        W = _w_true(t, sc)
        R = _dense_rotation(sig, 1024)
        want_a = (R @ x.T).T @ W.T
        want_b = x @ (W @ R).T
        scale = np.abs(want_a).max()
        np.testing.assert_allclose(got, want_a, rtol=0, atol=1e-12 * scale)
        np.testing.assert_allclose(got, want_b, rtol=0, atol=1e-12 * scale)
        rows = np.array([N - 1, 0, N // 2])
        np.testing.assert_allclose(o.packed_linear_rows(x, sig, 1024, codes, s2, b2, rows), got[:, rows],
                                   rtol=0, atol=1e-14 * scale)


def pin_fold_bruteforce(o):
    """The offline fold W_s = W R^T against a dense R built from scipy's
    Hadamard matrix, and the identity it exists for: W x == W_s (R x), with a
    dense fp64 W, blocks 512 and 1024, distinct signs per block."""
    rng = _rng(27)
    for N, K, L in ((40, 2048, 1024), (9, 1536, 512)):
        W = rng.standard_normal((N, K))
        sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
        x = rng.standard_normal((2, K))
        Ws = o.fold_rotation(W, sig, L)
        R = _dense_rotation(sig, L)
        np.testing.assert_allclose(Ws, W @ R.T, rtol=0, atol=1e-13 * np.abs(W).max())
        xr = o.fwht_signed(x, sig, L)
        want = x @ W.T
        np.testing.assert_allclose(xr @ Ws.T, want, rtol=0, atol=1e-12 * np.abs(want).max())


def pin_unrotated_is_plain_matmul(o):
    """block = 0: y = x @ (s*t)^T, brute force."""
    rng = _rng(21)
    N, K = 33, 384
    t = _ternary(rng, N, K)
    sc = _scales(rng, N, K)
    x = rng.standard_normal((2, K))
    codes, s2, b2 = o.pack(t, sc)
    want = x @ _w_true(t, sc).T
    np.testing.assert_allclose(o.packed_linear(x, None, 0, codes, s2, b2), want, rtol=0,
                               atol=1e-13 * np.abs(want).max())


def pin_batch_and_linearity(o):
    """I12/I13: each batch row equals the single-row call; y is linear in x."""
    rng = _rng(22)
    N, K = 40, 2048
    t = _ternary(rng, N, K)
    codes, s, b = o.pack(t, _scales(rng, N, K))
    sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((4, K))
    y = o.packed_linear(x, sig, 1024, codes, s, b)
    for i in range(4):
        np.testing.assert_allclose(o.packed_linear(x[i:i + 1], sig, 1024, codes, s, b)[0], y[i], atol=1e-14)
    z = o.packed_linear(2.5 * x[0:1] - 0.5 * x[1:2], sig, 1024, codes, s, b)[0]
    np.testing.assert_allclose(z, 2.5 * y[0] - 0.5 * y[1], atol=1e-12)


def pin_embed_bruteforce(o):
    """Embedding row = sigma * (H W~[r]) blockwise, dense scipy construction;
    out-of-range ids give NaN rows; block 0 gives the dequantized row."""
    rng = _rng(23)
    V, K = 12, 2048
    t = _ternary(rng, V, K)
    sc = _scales(rng, V, K)
    sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    codes, s2, b2 = o.pack(t, sc)
    ids = [3, 0, 11, 3, -1, 12]
    e = o.embed_inverse(ids, codes, s2, b2, sig, 1024)
    W = _w_true(t, sc)
    R = _dense_rotation(sig, 1024)
    for i, r in enumerate(ids[:4]):
        np.testing.assert_allclose(e[i], R.T @ W[r], atol=1e-13)
    assert np.isnan(e[4]).all() and np.isnan(e[5]).all()
    e0 = o.embed_inverse([5], codes, s2, b2, None, 0)
    np.testing.assert_array_equal(e0[0], W[5])


def pin_embed_linear_duality(o):
    """I7: <embed(r), x> == packed_linear(x)[r] for the same pack and signs."""
    rng = _rng(24)
    V, K = 9, 3072
    t = _ternary(rng, V, K)
    codes, s, b = o.pack(t, _scales(rng, V, K))
    sig = np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((1, K))
    y = o.packed_linear(x, sig, 1024, codes, s, b)[0]
    e = o.embed_inverse(np.arange(V), codes, s, b, sig, 1024)
    np.testing.assert_allclose(e @ x[0], y, atol=1e-12)


def pin_bf16_widening(o):
    """bf16 bit patterns widen exactly: 0x3F80 = 1, 0xC000 = -2, 0x3F81 = 1 + 2^-7."""
    got = o.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x3F81, 0x0000], np.uint16))
    np.testing.assert_array_equal(got, np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 0.0]))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
