"""fp64 reference for the two other ternary containers the pages name
(test infrastructure only; nothing in the product path imports it).

[P2] kwkr.cn/news/564617, section "packing-format engineering (MLX 2.25 bits
vs GGUF)": besides the MLX affine container (2 bits per weight plus an fp16
scale and an fp16 bias per 128 weights, 2.25 bits/weight), the same ternary
weights ship as GGUF blocks of 128 weights:

* PQ2_0 -- one 2-bit slot per trit and one fp16 scale per block: 34 bytes
  per 128 weights, 2.125 bits/weight.  The pack's converter transcodes the
  MLX container to it losslessly; its independent unpack() checks the
  result and the group scales were compared bit for bit.  The speed figure
  of the pages' GPU run uses this format.
* PTQ1_0 -- dense trits: 28 bytes per 128 weights, 1.75 bits/weight, which
  need extra arithmetic to decode.

The pages print neither block's byte layout.  Readings used here (the
plainest ones the stated sizes allow; see the design notes):

* both blocks start with the fp16 scale d (little-endian), then the codes;
  no bias is stored -- a ternary code c in {0, 1, 2} (t = c - 1) decodes to
  (c - 1) * d, the MLX decode with bias = -scale;
* PQ2_0: the 32 code bytes hold code k of the block at bits 2 (k % 4) of
  byte k // 4 -- byte for byte the MLX group's eight code words (code j of a
  word at bits 2 j, little-endian words);
* PTQ1_0: the 26 trit bytes hold five codes each, base 3 with the first code
  as the lowest digit: byte i = sum_j c[5 i + j] 3^j (j < 5; at most 242);
  the last byte holds codes 125..127 the same way (at most 26).

Arithmetic is fp64 on exactly widened inputs, as in oracle.reference.
"""
from __future__ import annotations

import numpy as np

from oracle.reference import GROUP, _rotate, codes_of, f16_to_f64, pack

#: bytes of one 128-weight block [P2 "packing-format engineering"]
PQ2_BLOCK_BYTES = 34
PTQ1_BLOCK_BYTES = 28
#: trits per dense byte (3^5 = 243 <= 256) and dense bytes per block
TRITS_PER_BYTE = 5
PTQ1_TRIT_BYTES = -(-GROUP // TRITS_PER_BYTE)  # 26


def _check_k(K):
    if K <= 0 or K % GROUP:
        raise ValueError(f"K={K} is not a positive multiple of {GROUP}")


def _scale_bytes(scales):
    """fp16 scales (N, G) -> their little-endian bytes (N, G, 2)."""
    s = np.asarray(scales)
    if s.dtype == np.float16:
        s = s.view(np.uint16)
    if s.dtype != np.uint16:
        raise TypeError("scales must be float16 (or their uint16 bits)")
    return np.stack([(s & 0xFF).astype(np.uint8), (s >> 8).astype(np.uint8)], axis=-1)


def _scales_of(blocks):
    """(N, G, block bytes) -> fp16 scales (N, G) from the first two bytes."""
    lo = blocks[:, :, 0].astype(np.uint16)
    hi = blocks[:, :, 1].astype(np.uint16)
    return (lo | (hi << 8)).view(np.float16)


# --------------------------------------------------------------------------
# PQ2_0
# --------------------------------------------------------------------------
def pq2_from_mlx(codes, scales, biases) -> np.ndarray:
    """Transcode an MLX affine container (codes uint32 (N, K/16), fp16 scales
    and biases (N, K/128)) to PQ2_0 blocks, uint8 (N, K/128 * 34).

    Lossless exactly when every bias is the negated scale and no code is 3
    (PQ2_0 stores no bias); otherwise ValueError."""
    codes = np.asarray(codes, dtype=np.uint32)
    N, W = codes.shape
    K = W * 16
    _check_k(K)
    G = K // GROUP
    s = np.asarray(scales).view(np.uint16).reshape(N, G)
    b = np.asarray(biases).view(np.uint16).reshape(N, G)
    if not np.array_equal(b, s ^ np.uint16(0x8000)):
        raise ValueError("a bias differs from the negated scale: not representable in PQ2_0")
    c = codes_of(codes, K)
    if (c == 3).any():
        raise ValueError("code 3 is not a ternary code")
    cb = c.reshape(N, G, 32, 4).astype(np.uint8)
    qs = cb[..., 0] | (cb[..., 1] << 2) | (cb[..., 2] << 4) | (cb[..., 3] << 6)
    out = np.concatenate([_scale_bytes(s), qs], axis=2)
    return out.reshape(N, G * PQ2_BLOCK_BYTES)


def _pq2_blocks(blocks, K):
    _check_k(K)
    blocks = np.asarray(blocks, dtype=np.uint8)
    G = K // GROUP
    if blocks.ndim != 2 or blocks.shape[1] != G * PQ2_BLOCK_BYTES:
        raise ValueError(f"PQ2_0 rows of K={K} hold {G * PQ2_BLOCK_BYTES} bytes")
    return blocks.reshape(blocks.shape[0], G, PQ2_BLOCK_BYTES)


def pq2_codes(blocks, K) -> np.ndarray:
    """2-bit code of every weight, uint8 (N, K)."""
    bl = _pq2_blocks(blocks, K)
    qs = bl[:, :, 2:]
    c = np.stack([(qs >> (2 * j)) & 3 for j in range(4)], axis=-1)  # (N, G, 32, 4)
    return c.reshape(bl.shape[0], K)


def pq2_to_mlx(blocks, K):
    """PQ2_0 blocks -> MLX container (codes, scales, biases = -scales), the
    inverse of pq2_from_mlx.  Code 3: ValueError."""
    c = pq2_codes(blocks, K)
    if (c == 3).any():
        raise ValueError("code 3 is not a ternary code")
    return pack(c.astype(np.int8) - 1, _scales_of(_pq2_blocks(blocks, K)))


def pq2_dequantize_rows(blocks, K, rows) -> np.ndarray:
    """W~[r, k] = d[r, k // 128] * (c[r, k] - 1) for the selected rows, fp64
    (code 3 decodes to 2 d, the affine value)."""
    bl = _pq2_blocks(blocks, K)[np.asarray(rows, dtype=np.int64)]
    c = pq2_codes(bl.reshape(bl.shape[0], -1), K).astype(np.float64)
    d = f16_to_f64(_scales_of(bl))
    return d[:, np.arange(K) // GROUP] * (c - 1.0)


def pq2_packed_linear(x, signs, block, blocks, K) -> np.ndarray:
    """y = W~ (R x) per row of x with W~ from PQ2_0 blocks."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    xr = _rotate(x, signs, block)
    N = np.asarray(blocks).shape[0]
    return xr @ pq2_dequantize_rows(blocks, K, np.arange(N)).T


# --------------------------------------------------------------------------
# PTQ1_0
# --------------------------------------------------------------------------
def ptq1_pack(t, scales) -> np.ndarray:
    """Ternary t (N, K) in {-1, 0, 1} and fp16 scales (N, K/128) -> PTQ1_0
    blocks uint8 (N, K/128 * 28)."""
    t = np.asarray(t)
    if t.ndim != 2:
        raise ValueError("t must be 2-D (N, K)")
    N, K = t.shape
    _check_k(K)
    if not np.isin(t, (-1, 0, 1)).all():
        raise ValueError("ternary weights must be -1, 0 or 1")
    G = K // GROUP
    c = (t.astype(np.int64) + 1).reshape(N, G, GROUP)
    pad = np.zeros((N, G, PTQ1_TRIT_BYTES * TRITS_PER_BYTE - GROUP), np.int64)
    d = np.concatenate([c, pad], axis=2).reshape(N, G, PTQ1_TRIT_BYTES, TRITS_PER_BYTE)
    byte = np.zeros((N, G, PTQ1_TRIT_BYTES), np.int64)
    for j in reversed(range(TRITS_PER_BYTE)):  # Horner: lowest digit = first code
        byte = byte * 3 + d[..., j]
    sc = np.asarray(scales)
    if sc.shape != (N, G):
        raise ValueError("scales must have shape (N, K/128)")
    sb = _scale_bytes(sc)
    return np.concatenate([sb, byte.astype(np.uint8)], axis=2).reshape(N, G * PTQ1_BLOCK_BYTES)


def _ptq1_blocks(blocks, K):
    _check_k(K)
    blocks = np.asarray(blocks, dtype=np.uint8)
    G = K // GROUP
    if blocks.ndim != 2 or blocks.shape[1] != G * PTQ1_BLOCK_BYTES:
        raise ValueError(f"PTQ1_0 rows of K={K} hold {G * PTQ1_BLOCK_BYTES} bytes")
    return blocks.reshape(blocks.shape[0], G, PTQ1_BLOCK_BYTES)


def ptq1_codes(blocks, K) -> np.ndarray:
    """Code c = t + 1 of every weight, uint8 (N, K).  A byte above 242 (or a
    last byte above 26) holds no valid trits: ValueError."""
    bl = _ptq1_blocks(blocks, K)
    q = bl[:, :, 2:].astype(np.int64)
    if (q > 242).any() or (q[:, :, -1] > 26).any():
        raise ValueError("a trit byte is out of range (not a PTQ1_0 block)")
    digits = []
    for _ in range(TRITS_PER_BYTE):
        digits.append(q % 3)
        q = q // 3
    c = np.stack(digits, axis=-1).reshape(bl.shape[0], bl.shape[1], -1)[:, :, :GROUP]
    return c.reshape(bl.shape[0], K).astype(np.uint8)


def ptq1_unpack(blocks, K):
    """PTQ1_0 blocks -> (t int8 (N, K), fp16 scales (N, K/128))."""
    c = ptq1_codes(blocks, K)
    return (c.astype(np.int16) - 1).astype(np.int8), _scales_of(_ptq1_blocks(blocks, K))


def ptq1_dequantize_rows(blocks, K, rows) -> np.ndarray:
    """W~[r, k] = d[r, k // 128] * t[r, k] for the selected rows, fp64."""
    bl = _ptq1_blocks(blocks, K)[np.asarray(rows, dtype=np.int64)]
    t, d = ptq1_unpack(bl.reshape(bl.shape[0], -1), K)
    return f16_to_f64(d)[:, np.arange(K) // GROUP] * t.astype(np.float64)


def ptq1_packed_linear(x, signs, block, blocks, K) -> np.ndarray:
    """y = W~ (R x) per row of x with W~ from PTQ1_0 blocks."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    xr = _rotate(x, signs, block)
    N = np.asarray(blocks).shape[0]
    return xr @ ptq1_dequantize_rows(blocks, K, np.arange(N)).T


def container_bytes_pq2(N: int, K: int) -> int:
    return N * (K // GROUP) * PQ2_BLOCK_BYTES


def container_bytes_ptq1(N: int, K: int) -> int:
    return N * (K // GROUP) * PTQ1_BLOCK_BYTES
