"""fp64 reference for the Packed-linear path (test infrastructure only).

Every function states the passage it follows.  Page references:

* [P2] kwkr.cn/news/564617, section "ternary weights + folded Hadamard
  rotation" (block-1024 orthogonal rotation with explicit +-1 signs of widths
  5120/6144/17408, folded into the stored weights; the runtime's fwht() uses a
  normalized Hadamard transform with scale 1/sqrt(block), signs multiplied on
  the forward pass and multiplied again on the inverse; quantized_matmul with
  transpose, group 128, 2 bits) and section "packing-format engineering" (MLX
  container stores an fp16 scale and an fp16 bias per group of 128, bias equal
  to minus the scale, 2-bit codes {0,1,2} decode to -s/0/s, 2.25 bits/weight).
* [P3] lpnh.cn/news/2438023, section "text model loading: artifact.load_model
  and the Packed module" (signs first, then the normalized Hadamard transform;
  packed uint32 code words consumed directly; embedding path dequantizes the
  looked-up row and then applies the inverse transform) and section "affine
  2-bit format and Prism contract v1" (block sizes 512/1024/2048/4096,
  normalized Sylvester-Walsh-Hadamard, axis = input last dimension, explicit
  signs that must all be +-1).
* [P1] trdm.cn/news/822023, section 2.2 (Sylvester recurrence
  H_2n = [[H_n, H_n], [H_n, -H_n]]) and section 3.2 (ternary value -1/0/1
  stored as code 0/1/2).

Readings where the pages are silent are listed in the repository's design
notes; the ones that shape arithmetic here are:

* bit order inside a uint32 word: code k of a 16-code word sits at bits
  2k..2k+1 (little-end first);
* code 3 never comes out of the packer; when decoding it is treated affinely
  as 3*s + b so every 2-bit word has a defined value;
* the bias is read from storage and never assumed to equal -scale;
* an embedding id outside [0, V) yields a row of NaN.

Inputs are widened exactly to float64 (bf16 and fp16 are subsets of fp64) and
all arithmetic is fp64.
"""
from __future__ import annotations

import math

import numpy as np

#: block sizes the contract accepts [P3 "affine 2-bit format and Prism contract v1"]
BLOCK_SIZES = (512, 1024, 2048, 4096)
#: weights sharing one fp16 scale and one fp16 bias [P2 "packing-format engineering"]
GROUP = 128
#: 2-bit codes per uint32 word [P3 "text model loading"; bit order is a reading]
CODES_PER_WORD = 16

_ROW_CHUNK = 512


# --------------------------------------------------------------------------
# exact widening of stored element types
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 values given as their uint16 bit patterns to float64 (exact:
    a bf16 value is the fp32 value whose low 16 bits are zero)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(h) -> np.ndarray:
    """Widen fp16 values (np.float16, or uint16 bit patterns) to float64."""
    a = np.asarray(h)
    if a.dtype == np.uint16:
        a = a.view(np.float16)
    if a.dtype != np.float16:
        raise TypeError(f"expected float16 or uint16 bit patterns, got {a.dtype}")
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# transform
# --------------------------------------------------------------------------
def fwht_blocks(v, block: int) -> np.ndarray:
    """Normalized Sylvester Walsh-Hadamard transform of every contiguous
    `block`-wide slice of the last axis, in fp64.

    [P1 section 2.2] H_2n = [[H_n, H_n], [H_n, -H_n]] gives, in natural
    (Sylvester) order, H[i, j] = (-1)^popcount(i & j).  One butterfly stage per
    bit h of the index maps the pair (v[i], v[i + h]) with bit h of i clear to
    (v[i] + v[i + h], v[i] - v[i + h]).  [P2 "ternary weights + folded Hadamard
    rotation"] the transform is normalized by 1/sqrt(block).
    """
    v = np.asarray(v, dtype=np.float64)
    if block <= 0 or block & (block - 1):
        raise ValueError(f"block must be a power of two, got {block}")
    K = v.shape[-1]
    if K % block:
        raise ValueError(f"last axis {K} is not a multiple of block {block}")
    lead = v.shape[:-1]
    a = v.reshape(-1, K // block, block).copy()
    rows, nb = a.shape[0], a.shape[1]
    h = 1
    while h < block:
        a = a.reshape(rows, nb, block // (2 * h), 2, h)
        lo = a[:, :, :, 0, :]
        hi = a[:, :, :, 1, :]
        a = np.stack((lo + hi, lo - hi), axis=3)
        h *= 2
    return a.reshape(*lead, K) / math.sqrt(block)


def _check_signs(signs, K: int) -> np.ndarray:
    s = np.asarray(signs)
    if s.shape != (K,):
        raise ValueError(f"sign vector must have shape ({K},), got {s.shape}")
    # [P3 "affine 2-bit format and Prism contract v1"]: every sign is +-1.
    if not np.isin(s, (-1, 1)).all():
        raise ValueError("sign vector holds a value other than +-1")
    return s.astype(np.float64)


def fwht_signed(x, signs, block: int, inverse: bool = False) -> np.ndarray:
    """Signed block transform along the input (last) axis.

    Forward [P3 "text model loading"]: multiply by the explicit sign vector
    first, then apply the normalized transform: H (sigma * x).
    Inverse [P2 "ternary weights + folded Hadamard rotation"]: the signs are
    multiplied again after the transform: sigma * (H y).  Because H H = I and
    sigma * sigma = 1, this inverse undoes the forward transform.
    The sign vector has one entry per input element (width = K), block j uses
    signs[j*block:(j+1)*block].
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if block not in BLOCK_SIZES:
        raise ValueError(f"block {block} not accepted by the contract")
    s = _check_signs(signs, K)
    if inverse:
        return fwht_blocks(x, block) * s
    return fwht_blocks(x * s, block)


# --------------------------------------------------------------------------
# container: pack / unpack / decode
# --------------------------------------------------------------------------
def _check_container(codes, scales, biases, K: int):
    codes = np.asarray(codes)
    if codes.dtype != np.uint32 or codes.ndim != 2:
        raise TypeError("codes must be a 2-D uint32 array (N, K/16)")
    if K % GROUP:
        raise ValueError(f"K={K} is not a multiple of the group size {GROUP}")
    N = codes.shape[0]
    if codes.shape[1] * CODES_PER_WORD != K:
        raise ValueError(f"codes has {codes.shape[1]} words per row, K={K} needs {K // CODES_PER_WORD}")
    sc = f16_to_f64(scales)
    bi = f16_to_f64(biases)
    if sc.shape != (N, K // GROUP) or bi.shape != (N, K // GROUP):
        raise ValueError("scales/biases must have shape (N, K/128)")
    return codes, sc, bi


def codes_of(codes, K: int) -> np.ndarray:
    """2-bit code of every weight: c[n, k] = (codes[n, k // 16] >> 2 (k % 16)) & 3.

    [P3 "text model loading"] the weight tensor is uint32 words of packed 2-bit
    codes; the position of code k inside its word is the little-end-first
    reading.
    """
    codes = np.asarray(codes, dtype=np.uint32)
    N, W = codes.shape
    if W * CODES_PER_WORD != K:
        raise ValueError("word count does not match K")
    shifts = (2 * np.arange(CODES_PER_WORD, dtype=np.uint32))
    c = (codes[:, :, None] >> shifts[None, None, :]) & np.uint32(3)
    return c.reshape(N, K).astype(np.uint8)


def dequantize_rows(codes, scales, biases, K: int, rows) -> np.ndarray:
    """Dequantized weights W~[r, k] = s[r, k // 128] * c[r, k] + b[r, k // 128]
    for the selected rows, fp64.

    [P2 "packing-format engineering"] each group of 128 weights stores an fp16
    scale s and an fp16 bias b; code q decodes to s*q + b (so {0,1,2} give
    -s/0/s when b = -s).  The stored bias is used as is.
    """
    codes, sc, bi = _check_container(codes, scales, biases, K)
    rows = np.asarray(rows, dtype=np.int64)
    c = codes_of(codes[rows], K).astype(np.float64)
    g = np.arange(K) // GROUP
    return sc[rows][:, g] * c + bi[rows][:, g]


def dequantize(codes, scales, biases, K: int) -> np.ndarray:
    """Dense fp64 W~ (N, K); see dequantize_rows."""
    N = np.asarray(codes).shape[0]
    return dequantize_rows(codes, scales, biases, K, np.arange(N))


def pack(t, scales):
    """Pack ternary weights into the MLX affine 2-bit container.

    t: int array (N, K) with values in {-1, 0, 1}; scales: fp16 (N, K/128).
    Returns (codes uint32 (N, K/16), scales fp16, biases fp16).

    [P1 section 3.2] ternary -1/0/1 is stored as code 0/1/2, i.e. code = t + 1;
    [P3 "text model loading"] codes are packed into uint32 words; [P2
    "packing-format engineering"] bias = -scale.  Raises ValueError on a value
    outside {-1, 0, 1}.
    """
    t = np.asarray(t)
    if t.ndim != 2:
        raise ValueError("t must be 2-D (N, K)")
    N, K = t.shape
    if K % GROUP:
        raise ValueError(f"K={K} is not a multiple of {GROUP}")
    if not np.isin(t, (-1, 0, 1)).all():
        raise ValueError("ternary weights must be -1, 0 or 1")
    sc = np.asarray(scales)
    if sc.dtype == np.uint16:
        sc = sc.view(np.float16)
    if sc.dtype != np.float16 or sc.shape != (N, K // GROUP):
        raise ValueError("scales must be float16 of shape (N, K/128)")
    c = (t.astype(np.int64) + 1).astype(np.uint32).reshape(N, K // CODES_PER_WORD, CODES_PER_WORD)
    shifts = (2 * np.arange(CODES_PER_WORD, dtype=np.uint32))
    words = np.bitwise_or.reduce(c << shifts[None, None, :], axis=2).astype(np.uint32)
    return words, sc.copy(), (-sc).astype(np.float16)


def unpack(codes, K: int) -> np.ndarray:
    """Inverse of `pack` on the codes: t = code - 1 as int8 (N, K).

    [P2 "packing-format engineering"] an independent unpack() verifies the
    packing.  Code 3 is outside the ternary alphabet: ValueError.
    """
    c = codes_of(codes, K)
    if (c == 3).any():
        raise ValueError("code 3 found: not a ternary container")
    return (c.astype(np.int16) - 1).astype(np.int8)


def container_bytes(N: int, K: int) -> int:
    """Bytes of the container: uint32 codes + fp16 scales + fp16 biases.
    [P2 "packing-format engineering"]: 2 + 16/128 + 16/128 = 2.25 bits/weight."""
    return N * (K // CODES_PER_WORD) * 4 + 2 * N * (K // GROUP) * 2


# --------------------------------------------------------------------------
# the Packed-linear step and the embedding path
# --------------------------------------------------------------------------
def _rotate(x, signs, block: int) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if block == 0:
        if signs is not None:
            raise ValueError("block=0 (no rotation) takes no sign vector")
        return x
    return fwht_signed(x, signs, block)


def packed_linear_rows(x, signs, block: int, codes, scales, biases, rows) -> np.ndarray:
    """Selected output columns of the Packed linear: y[b, j] = sum_k
    W~[rows[j], k] * xr[b, k] with xr = H (sigma * x[b]) blockwise.

    [P3 "text model loading"] when the module declares a block, the
    activation goes through fwht(x, block, signs) and then through
    quantized_matmul(x, weight, scales, biases, transpose=True, group 128,
    bits 2) -- i.e. y = xr @ W~^T with W~ of shape (N, K).  block = 0 means the
    module has no rotation (plain affine 2-bit matmul).
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    K = x.shape[-1]
    xr = _rotate(x, signs, block)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((x.shape[0], rows.size), dtype=np.float64)
    for i in range(0, rows.size, _ROW_CHUNK):
        w = dequantize_rows(codes, scales, biases, K, rows[i:i + _ROW_CHUNK])
        out[:, i:i + _ROW_CHUNK] = xr @ w.T
    return out


def packed_linear(x, signs, block: int, codes, scales, biases) -> np.ndarray:
    """Full Packed-linear output y (B, N) in fp64; see packed_linear_rows."""
    N = np.asarray(codes).shape[0]
    return packed_linear_rows(x, signs, block, codes, scales, biases, np.arange(N))


def embed_inverse(ids, codes, scales, biases, signs, block: int) -> np.ndarray:
    """Embedding path: out[t] = sigma * (H W~[ids[t], :]) blockwise, fp64.

    [P3 "text model loading"] the embedding module dequantizes the looked-up
    row and then applies fwht(..., inverse=True); [P2 "ternary weights +
    folded Hadamard rotation"] the inverse multiplies the signs again after
    the transform.  block = 0 returns the dequantized row.  An id outside
    [0, V) gives a NaN row (a reading: the pages do not define it).
    """
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    codes = np.asarray(codes)
    V = codes.shape[0]
    K = codes.shape[1] * CODES_PER_WORD
    out = np.full((ids.size, K), np.nan, dtype=np.float64)
    ok = (ids >= 0) & (ids < V)
    if ok.any():
        rows = dequantize_rows(codes, scales, biases, K, ids[ok])
        if block == 0:
            if signs is not None:
                raise ValueError("block=0 takes no sign vector")
            out[ok] = rows
        else:
            out[ok] = fwht_signed(rows, signs, block, inverse=True)
    return out


# --------------------------------------------------------------------------
# the offline fold
# --------------------------------------------------------------------------
def fold_rotation(w, signs, block: int) -> np.ndarray:
    """Fold the rotation into a dense weight matrix: W_s = W R^T, fp64.

    [P2 "ternary weights + folded Hadamard rotation"] each matrix is rotated
    block by block before it is quantized, and the stored weights already sit
    in the rotated basis, so that W x = (W R^T)(R x) with R x the activation
    transform of the Packed linear.  With R = blockdiag(H) diag(sigma) and H
    symmetric, row n of W R^T is (R w_n)^T, i.e. the forward signed transform
    of that row.  The ternarization of W_s that follows is not given by the
    pages and is not part of this function.
    """
    w = np.atleast_2d(np.asarray(w, dtype=np.float64))
    return fwht_signed(w, signs, block)
