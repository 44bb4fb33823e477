"""Python binding of libtb, the gfx950 folded-Hadamard ternary Packed-linear
library.  Argument marshalling only: every step of the path runs in the HIP
kernels behind the C ABI declared in include/tb.h.  Functions carry the C
names; device functions take torch tensors already on the GPU and enqueue on
torch's current stream.  There is no fallback: if libtb.so is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libtb.so")

TB_OK = 0
TB_F32 = 0
TB_BF16 = 1
TB_GEMV_MAX_BATCH = 8
STATUS = {
    0: "TB_OK", -1: "TB_ERR_ARG", -2: "TB_ERR_SHAPE", -3: "TB_ERR_BLOCK", -4: "TB_ERR_UNSUPPORTED",
    -5: "TB_ERR_SIGN", -6: "TB_ERR_CODE", -7: "TB_ERR_DTYPE", -8: "TB_ERR_ALIGN", -9: "TB_ERR_HIP",
    -10: "TB_ERR_WORKSPACE",
}

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "tb_abi_version": (_I, []),
    "tb_last_error": (ctypes.c_char_p, []),
    "tb_status_str": (ctypes.c_char_p, [_I]),
    "tb_pack": (_I, [_P, _P, _I64, _I64, _P, _P, _P]),
    "tb_unpack": (_I, [_P, _I64, _I64, _P]),
    "tb_signs_validate": (_I, [_P, _I64]),
    "tb_pack_device": (_I, [_P, _P, _I64, _I64, _P, _P, _P, _P, _P]),
    "tb_fwht_signed": (_I, [_P, _I, _P, _P, _I64, _I64, _I, _I, _P]),
    "tb_ternary_gemv_workspace_size": (_SZ, [_I64, _I64]),
    "tb_ternary_gemv_workspace_size_n": (_SZ, [_I64, _I64, _I64]),
    "tb_ternary_gemv": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "tb_ternary_gemv_noalloc": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P, _I64, _P, _P]),
    "tb_ternary_gemv_prepare": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "tb_ternary_gemv_run": (_I, [_P, _SZ, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "tb_ternary_gemm_workspace_size": (_SZ, [_I64, _I64]),
    "tb_ternary_gemm_workspace_size_n": (_SZ, [_I64, _I64, _I64]),
    "tb_ternary_gemm_prepare": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _SZ, _P]),
    "tb_ternary_gemm_run": (_I, [_P, _SZ, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "tb_ternary_gemm": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "tb_embed_inverse": (_I, [_P, _I64, _P, _P, _P, _I64, _I64, _P, _I, _P, _P]),
    "tb_pq2_from_mlx": (_I, [_P, _P, _P, _I64, _I64, _P]),
    "tb_pq2_to_mlx": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "tb_ptq1_pack": (_I, [_P, _P, _I64, _I64, _P]),
    "tb_ptq1_unpack": (_I, [_P, _I64, _I64, _P, _P]),
    "tb_pq2_gemv": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _I64, _P, _P]),
    "tb_ptq1_gemv": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _I64, _P, _P]),
    "tb_gemv_multi_plan_size": (_SZ, [_P, _I64]),
    "tb_gemv_multi_plan": (_I, [_P, _I64, _I, _I, _P, _SZ, ctypes.POINTER(_SZ)]),
    "tb_pq2_gemv_multi_plan": (_I, [_P, _I64, _I, _I, _P, _SZ, ctypes.POINTER(_SZ)]),
    "tb_ptq1_gemv_multi_plan": (_I, [_P, _I64, _I, _I, _P, _SZ, ctypes.POINTER(_SZ)]),
    "tb_ternary_gemv_multi": (_I, [_P, _P, _P, _SZ, _P]),
}


class TbGemvModule(ctypes.Structure):
    """tb_gemv_module of include/tb.h (device pointers, N, K)."""
    _fields_ = [("x", _P), ("signs", _P), ("codes", _P), ("scales", _P), ("biases", _P), ("y", _P),
                ("N", _I64), ("K", _I64)]


class TBError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded libtb.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m hadamard_rotated_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != TB_OK:
        raise TBError(status, lib().tb_last_error().decode())


# ---------------------------------------------------------------------------
# host container functions (numpy)
# ---------------------------------------------------------------------------
def tb_pack(t: np.ndarray, scales: np.ndarray):
    """t int8 (N, K) in {-1,0,1}, scales float16 (N, K/128) ->
    (codes uint32 (N, K/16), scales float16, biases float16)."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    sc = np.ascontiguousarray(scales)
    if sc.dtype == np.float16:
        sc = sc.view(np.uint16)
    if t.ndim != 2:
        raise ValueError(f"t must be 2-D (N, K), got shape {t.shape}")
    N, K = t.shape
    _check_width(K)
    if sc.shape != (N, K // 128) or sc.dtype != np.uint16:
        raise ValueError("scales must be float16 (N, K/128)")
    codes = np.empty((N, K // 16), np.uint32)
    so = np.empty_like(sc)
    bo = np.empty_like(sc)
    _check(lib().tb_pack(t.ctypes.data, sc.ctypes.data, N, K, codes.ctypes.data, so.ctypes.data,
                         bo.ctypes.data))
    return codes, so.view(np.float16), bo.view(np.float16)


def tb_unpack(codes: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    _check_width(K)
    if codes.ndim != 2 or codes.shape[1] != K // 16:
        raise ValueError(f"codes has shape {codes.shape}, expected (N, {K // 16})")
    N = codes.shape[0]
    out = np.empty((N, K), np.int8)
    _check(lib().tb_unpack(codes.ctypes.data, N, K, out.ctypes.data))
    return out


def tb_signs_validate(signs: np.ndarray) -> None:
    s = np.ascontiguousarray(signs, dtype=np.int8)
    _check(lib().tb_signs_validate(s.ctypes.data, s.size))


# ---------------------------------------------------------------------------
# device functions (torch tensors on the GPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _xdtype(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return TB_F32
    if x.dtype == torch.bfloat16:
        return TB_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def tb_pack_device(t, scales, check: bool = True):
    """Pack on the device.  t int8 (N, K), scales float16 (N, K/128), both on
    the GPU.  With check=True, synchronizes and raises on invalid values."""
    torch = _torch()
    N, K = _rows(t, "t")
    _check_width(K)
    _shape(scales, (N, K // 128), "scales")
    _dev(t, "t", torch.int8)
    _dev(scales, "scales", torch.float16)
    codes = torch.empty((N, K // 16), dtype=torch.int32, device=t.device)
    so = torch.empty_like(scales)
    bo = torch.empty_like(scales)
    bad = torch.zeros(1, dtype=torch.int32, device=t.device)
    _check(lib().tb_pack_device(t.data_ptr(), scales.data_ptr(), N, K, codes.data_ptr(), so.data_ptr(),
                                bo.data_ptr(), bad.data_ptr(), _stream()))
    if check and int(bad.item()) != 0:
        raise TBError(-6, f"tb_pack_device: {int(bad.item())} values outside {{-1,0,1}}")
    return codes, so, bo


def tb_fwht_signed(x, signs, block: int, inverse: bool = False, out=None):
    torch = _torch()
    rows, K = _rows(x)
    _shape(signs, (K,), "signs")
    if out is not None:
        _shape(out, (rows, K), "out")
    _dev(x, "x")
    _dev(signs, "signs", torch.int8)
    if out is None:
        out = torch.empty((rows, K), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    _check(lib().tb_fwht_signed(x.data_ptr(), _xdtype(x), out.data_ptr(), signs.data_ptr(), rows, K,
                                block, int(bool(inverse)), _stream()))
    return out


def tb_ternary_gemv_workspace_size(B: int, K: int) -> int:
    return int(lib().tb_ternary_gemv_workspace_size(B, K))


def tb_ternary_gemv_workspace_size_n(B: int, K: int, N: int) -> int:
    return int(lib().tb_ternary_gemv_workspace_size_n(B, K, N))


def tb_ternary_gemm_workspace_size(M: int, K: int) -> int:
    return int(lib().tb_ternary_gemm_workspace_size(M, K))


def tb_ternary_gemm_workspace_size_n(M: int, K: int, N: int) -> int:
    return int(lib().tb_ternary_gemm_workspace_size_n(M, K, N))


def _shape(t, shape, name):
    """Raise ValueError unless tensor t has exactly this shape.  Checked
    before any pointer reaches the library: the C ABI receives only pointers
    and the sizes claimed here, so a mismatched tensor would be read past its
    end on the device."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_width(K, name="K"):
    if K <= 0 or K % 128:
        raise ValueError(f"{name}={K} must be a positive multiple of 128")


def _container_shapes(codes, scales, biases, N, K):
    """codes (N, K/16) words, scales and biases (N, K/128)."""
    _check_width(K)
    _shape(codes, (N, K // 16), "codes")
    _shape(scales, (N, K // 128), "scales")
    _shape(biases, (N, K // 128), "biases")


def _signs_shape(signs, K, block):
    if block == 0:
        if signs is not None:
            raise ValueError("block 0 (no rotation) takes no sign vector")
        return
    if signs is None:
        raise ValueError(f"block {block} needs a sign vector of {K} elements")
    _shape(signs, (K,), "signs")


def _rows(x, name="x"):
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D (rows, K), got shape {tuple(x.shape)}")
    return int(x.shape[0]), int(x.shape[1])


def _container(codes, scales, biases):
    torch = _torch()
    _dev(codes, "codes")
    if codes.dtype not in (torch.int32, torch.uint32):
        raise TypeError("codes must be int32/uint32 words")
    _dev(scales, "scales", torch.float16)
    _dev(biases, "biases", torch.float16)


def tb_ternary_gemv(x, signs, block: int, codes, scales, biases, out=None, workspace=None):
    """y (B, N) float32 = Packed linear of x (B, K) for B <= 8."""
    torch = _torch()
    B, K = _rows(x)
    N = int(codes.shape[0])
    _container_shapes(codes, scales, biases, N, K)
    _signs_shape(signs, K, block)
    if out is not None:
        _shape(out, (B, N), "out")
    _dev(x, "x")
    _container(codes, scales, biases)
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    need = tb_ternary_gemv_workspace_size_n(B, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().tb_ternary_gemv(x.data_ptr(), _xdtype(x), B, K, _ptr(signs), block, codes.data_ptr(),
                                 scales.data_ptr(), biases.data_ptr(), N, out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), _stream()))
    return out


def tb_ternary_gemv_noalloc(x, signs, block: int, codes, scales, biases, out=None):
    """tb_ternary_gemv with the library's static device scratch as its
    workspace (no device allocation by the library; `out` is allocated here
    only when the caller passes none)."""
    torch = _torch()
    B, K = _rows(x)
    N = int(codes.shape[0])
    _container_shapes(codes, scales, biases, N, K)
    _signs_shape(signs, K, block)
    if out is not None:
        _shape(out, (B, N), "out")
    _dev(x, "x")
    _container(codes, scales, biases)
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    _check(lib().tb_ternary_gemv_noalloc(x.data_ptr(), _xdtype(x), B, K, _ptr(signs), block, codes.data_ptr(),
                                         scales.data_ptr(), biases.data_ptr(), N, out.data_ptr(), _stream()))
    return out


def tb_ternary_gemv_prepare(x, signs, block: int, workspace=None):
    """Rotate and split x (B, K) into a workspace (uint8 tensor) for
    tb_ternary_gemv_run; returns the workspace."""
    torch = _torch()
    B, K = _rows(x)
    _check_width(K)
    _signs_shape(signs, K, block)
    _dev(x, "x")
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    need = tb_ternary_gemv_workspace_size(B, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().tb_ternary_gemv_prepare(x.data_ptr(), _xdtype(x), B, K, _ptr(signs), block,
                                         workspace.data_ptr(), workspace.numel(), _stream()))
    return workspace


def tb_ternary_gemv_run(workspace, B: int, K: int, codes, scales, biases, out=None):
    torch = _torch()
    N = int(codes.shape[0])
    _container_shapes(codes, scales, biases, N, K)
    if out is not None:
        _shape(out, (B, N), "out")
    _dev(workspace, "workspace", torch.uint8)
    _container(codes, scales, biases)
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=workspace.device)
    _dev(out, "out", torch.float32)
    _check(lib().tb_ternary_gemv_run(workspace.data_ptr(), workspace.numel(), B, K, codes.data_ptr(),
                                     scales.data_ptr(), biases.data_ptr(), N, out.data_ptr(), _stream()))
    return out


def tb_ternary_gemm_prepare(x, signs, block: int, workspace=None, N: int | None = None):
    """Rotate x (M, K) into a new (or the given) workspace; with N, the new
    workspace is sized for runs against N output columns (tail split)."""
    torch = _torch()
    M, K = _rows(x)
    _check_width(K)
    _signs_shape(signs, K, block)
    _dev(x, "x")
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    need = tb_ternary_gemm_workspace_size(M, K) if N is None else tb_ternary_gemm_workspace_size_n(M, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().tb_ternary_gemm_prepare(x.data_ptr(), _xdtype(x), M, K, _ptr(signs), block,
                                         workspace.data_ptr(), workspace.numel(), _stream()))
    return workspace


def tb_ternary_gemm_run(workspace, M: int, K: int, codes, scales, biases, out=None):
    torch = _torch()
    N = int(codes.shape[0])
    _container_shapes(codes, scales, biases, N, K)
    if out is not None:
        _shape(out, (M, N), "out")
    _dev(workspace, "workspace", torch.uint8)
    _container(codes, scales, biases)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=workspace.device)
    _dev(out, "out", torch.float32)
    _check(lib().tb_ternary_gemm_run(workspace.data_ptr(), workspace.numel(), M, K, codes.data_ptr(),
                                     scales.data_ptr(), biases.data_ptr(), N, out.data_ptr(), _stream()))
    return out


def tb_ternary_gemm(x, signs, block: int, codes, scales, biases, out=None, workspace=None):
    """y (M, N) float32 = Packed linear of x (M, K), block-scaled fp6 x fp4
    MFMA path."""
    torch = _torch()
    M, K = _rows(x)
    N = int(codes.shape[0])
    _container_shapes(codes, scales, biases, N, K)
    _signs_shape(signs, K, block)
    if out is not None:
        _shape(out, (M, N), "out")
    _dev(x, "x")
    _container(codes, scales, biases)
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    need = tb_ternary_gemm_workspace_size_n(M, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib().tb_ternary_gemm(x.data_ptr(), _xdtype(x), M, K, _ptr(signs), block, codes.data_ptr(),
                                 scales.data_ptr(), biases.data_ptr(), N, out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), _stream()))
    return out


def tb_embed_inverse(ids, codes, scales, biases, signs, block: int, out=None):
    """(T, K) float32 rows: inverse-transformed dequantized table rows."""
    torch = _torch()
    if ids.dim() != 1:
        raise ValueError(f"ids must be 1-D, got shape {tuple(ids.shape)}")
    T = int(ids.numel())
    V = int(codes.shape[0])
    K = int(codes.shape[1]) * 16 if codes.dim() == 2 else 0
    _container_shapes(codes, scales, biases, V, K)
    _signs_shape(signs, K, block)
    if out is not None:
        _shape(out, (T, K), "out")
    _dev(ids, "ids", torch.int32)
    _container(codes, scales, biases)
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=ids.device)
    _dev(out, "out", torch.float32)
    _check(lib().tb_embed_inverse(ids.data_ptr(), T, codes.data_ptr(), scales.data_ptr(),
                                  biases.data_ptr(), V, K, _ptr(signs), block, out.data_ptr(), _stream()))
    return out


# ---------------------------------------------------------------------------
# multi-module decode (batch 1)
# ---------------------------------------------------------------------------
def tb_gemv_multi_plan(modules, block: int, x_dtype: int = TB_BF16):
    """Plan a multi-module decode call.  modules: sequence of (x, signs, codes,
    scales, biases, y) tensors on the GPU (x: (K,) or (1, K); y: (N,) or
    (1, N) float32, overwritten by each run).  Returns (plan, workspace_bytes)
    with plan a host uint8 numpy array; the plan embeds the tensors' device
    pointers, so they must stay alive (and in place) while it is used."""
    torch = _torch()
    arr = (TbGemvModule * len(modules))()
    for i, (x, signs, codes, scales, biases, y) in enumerate(modules):
        if x.dim() not in (1, 2) or (x.dim() == 2 and x.shape[0] != 1):
            raise ValueError(f"module {i}: x must be (K,) or (1, K), got {tuple(x.shape)}")
        K = int(x.shape[-1])
        N = int(codes.shape[0])
        _container_shapes(codes, scales, biases, N, K)
        _signs_shape(signs, K, block)
        if y.numel() != N or y.dim() not in (1, 2):
            raise ValueError(f"module {i}: y must hold N={N} outputs, got shape {tuple(y.shape)}")
        _dev(x, "x")
        _container(codes, scales, biases)
        _dev(y, "y", torch.float32)
        if signs is not None:
            _dev(signs, "signs", torch.int8)
        arr[i] = TbGemvModule(x.data_ptr(), _ptr(signs), codes.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                              y.data_ptr(), N, K)
    size = int(lib().tb_gemv_multi_plan_size(arr, len(modules)))
    plan = np.zeros(max(size, 64), np.uint8)
    ws = _SZ(0)
    _check(lib().tb_gemv_multi_plan(arr, len(modules), x_dtype, block, plan.ctypes.data, plan.nbytes,
                                    ctypes.byref(ws)))
    return plan, int(ws.value)


def tb_pq2_gemv_multi_plan(modules, block: int, x_dtype: int = TB_BF16):
    """tb_gemv_multi_plan on PQ2_0 blocks: modules is a sequence of (x, signs,
    blocks, y) with blocks the module's (N, K / 128 * 34) uint8 PQ2_0 array
    on the GPU.  Returns (plan, workspace_bytes); run it with
    tb_ternary_gemv_multi."""
    return _blocks_multi_plan(lib().tb_pq2_gemv_multi_plan, PQ2_BLOCK_BYTES, modules, block, x_dtype)


def tb_ptq1_gemv_multi_plan(modules, block: int, x_dtype: int = TB_BF16):
    """tb_gemv_multi_plan on PTQ1_0 blocks: modules is a sequence of (x,
    signs, blocks, y) with blocks the module's (N, K / 128 * 28) uint8
    PTQ1_0 array on the GPU.  Returns (plan, workspace_bytes)."""
    return _blocks_multi_plan(lib().tb_ptq1_gemv_multi_plan, PTQ1_BLOCK_BYTES, modules, block, x_dtype)


def _blocks_multi_plan(fn, nbytes, modules, block, x_dtype):
    torch = _torch()
    arr = (TbGemvModule * len(modules))()
    for i, (x, signs, blocks, y) in enumerate(modules):
        if x.dim() not in (1, 2) or (x.dim() == 2 and x.shape[0] != 1):
            raise ValueError(f"module {i}: x must be (K,) or (1, K), got {tuple(x.shape)}")
        K = int(x.shape[-1])
        _check_width(K)
        if blocks.dim() != 2 or blocks.shape[1] != K // 128 * nbytes:
            raise ValueError(f"module {i}: blocks has shape {tuple(blocks.shape)}, "
                             f"expected (N, {K // 128 * nbytes})")
        N = int(blocks.shape[0])
        _signs_shape(signs, K, block)
        if y.numel() != N or y.dim() not in (1, 2):
            raise ValueError(f"module {i}: y must hold N={N} outputs, got shape {tuple(y.shape)}")
        _dev(x, "x")
        _dev(blocks, "blocks", torch.uint8)
        _dev(y, "y", torch.float32)
        if signs is not None:
            _dev(signs, "signs", torch.int8)
        arr[i] = TbGemvModule(x.data_ptr(), _ptr(signs), blocks.data_ptr(), None, None, y.data_ptr(), N, K)
    size = int(lib().tb_gemv_multi_plan_size(arr, len(modules)))
    plan = np.zeros(max(size, 64), np.uint8)
    ws = _SZ(0)
    _check(fn(arr, len(modules), x_dtype, block, plan.ctypes.data, plan.nbytes, ctypes.byref(ws)))
    return plan, int(ws.value)


def tb_ternary_gemv_multi(plan, plan_device, workspace):
    """Run a plan: plan (host numpy array from tb_gemv_multi_plan), plan_device
    (uint8 tensor on the GPU holding the same bytes), workspace (uint8 tensor of
    the reported size).  Enqueues on the current stream."""
    torch = _torch()
    _dev(plan_device, "plan_device", torch.uint8)
    _dev(workspace, "workspace", torch.uint8)
    _check(lib().tb_ternary_gemv_multi(plan.ctypes.data, plan_device.data_ptr(), workspace.data_ptr(),
                                       workspace.numel(), _stream()))


# ---------------------------------------------------------------------------
# block containers: PQ2_0 (34 bytes per 128 weights) and PTQ1_0 (28 bytes)
# ---------------------------------------------------------------------------
PQ2_BLOCK_BYTES = 34
PTQ1_BLOCK_BYTES = 28


def _u16(a, shape, name):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16 or a.shape != tuple(shape):
        raise ValueError(f"{name} must be float16 of shape {tuple(shape)}")
    return a


def tb_pq2_from_mlx(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    """MLX container (host arrays) -> PQ2_0 blocks uint8 (N, K/128 * 34)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    if codes.ndim != 2:
        raise ValueError("codes must be (N, K/16)")
    N, K = codes.shape[0], codes.shape[1] * 16
    _check_width(K)
    sc = _u16(scales, (N, K // 128), "scales")
    bi = _u16(biases, (N, K // 128), "biases")
    out = np.empty((N, K // 128 * PQ2_BLOCK_BYTES), np.uint8)
    _check(lib().tb_pq2_from_mlx(codes.ctypes.data, sc.ctypes.data, bi.ctypes.data, N, K, out.ctypes.data))
    return out


def tb_pq2_to_mlx(blocks: np.ndarray, K: int):
    """PQ2_0 blocks (host) -> (codes uint32, scales float16, biases float16)."""
    _check_width(K)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    if blocks.ndim != 2 or blocks.shape[1] != K // 128 * PQ2_BLOCK_BYTES:
        raise ValueError(f"blocks must be (N, {K // 128 * PQ2_BLOCK_BYTES})")
    N = blocks.shape[0]
    codes = np.empty((N, K // 16), np.uint32)
    sc = np.empty((N, K // 128), np.uint16)
    bi = np.empty((N, K // 128), np.uint16)
    _check(lib().tb_pq2_to_mlx(blocks.ctypes.data, N, K, codes.ctypes.data, sc.ctypes.data, bi.ctypes.data))
    return codes, sc.view(np.float16), bi.view(np.float16)


def tb_ptq1_pack(t: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Ternary t int8 (N, K) and float16 scales (N, K/128) -> PTQ1_0 blocks
    uint8 (N, K/128 * 28)."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    if t.ndim != 2:
        raise ValueError("t must be (N, K)")
    N, K = t.shape
    _check_width(K)
    sc = _u16(scales, (N, K // 128), "scales")
    out = np.empty((N, K // 128 * PTQ1_BLOCK_BYTES), np.uint8)
    _check(lib().tb_ptq1_pack(t.ctypes.data, sc.ctypes.data, N, K, out.ctypes.data))
    return out


def tb_ptq1_unpack(blocks: np.ndarray, K: int):
    """PTQ1_0 blocks (host) -> (t int8 (N, K), scales float16 (N, K/128))."""
    _check_width(K)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    if blocks.ndim != 2 or blocks.shape[1] != K // 128 * PTQ1_BLOCK_BYTES:
        raise ValueError(f"blocks must be (N, {K // 128 * PTQ1_BLOCK_BYTES})")
    N = blocks.shape[0]
    t = np.empty((N, K), np.int8)
    sc = np.empty((N, K // 128), np.uint16)
    _check(lib().tb_ptq1_unpack(blocks.ctypes.data, N, K, t.ctypes.data, sc.ctypes.data))
    return t, sc.view(np.float16)


def _blocks_gemv(fn, nbytes, x, signs, block, blocks, out):
    torch = _torch()
    B, K = _rows(x)
    _check_width(K)
    _signs_shape(signs, K, block)
    if blocks.dim() != 2 or blocks.shape[1] != K // 128 * nbytes:
        raise ValueError(f"blocks has shape {tuple(blocks.shape)}, expected (N, {K // 128 * nbytes})")
    N = int(blocks.shape[0])
    if out is not None:
        _shape(out, (B, N), "out")
    _dev(x, "x")
    _dev(blocks, "blocks", torch.uint8)
    if signs is not None:
        _dev(signs, "signs", torch.int8)
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    _check(fn(x.data_ptr(), _xdtype(x), B, K, _ptr(signs), block, blocks.data_ptr(), N, out.data_ptr(), _stream()))
    return out


def tb_pq2_gemv(x, signs, block: int, blocks, out=None):
    """y (1, N) float32 = Packed linear of x (1, K) on PQ2_0 blocks (uint8
    (N, K/128 * 34) on the GPU)."""
    return _blocks_gemv(lib().tb_pq2_gemv, PQ2_BLOCK_BYTES, x, signs, block, blocks, out)


def tb_ptq1_gemv(x, signs, block: int, blocks, out=None):
    """y (1, N) float32 = Packed linear of x (1, K) on PTQ1_0 blocks (uint8
    (N, K/128 * 28) on the GPU)."""
    return _blocks_gemv(lib().tb_ptq1_gemv, PTQ1_BLOCK_BYTES, x, signs, block, blocks, out)
