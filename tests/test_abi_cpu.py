"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, the host container functions match the oracle bit for bit, and the
device entry points reject bad arguments on the host before any GPU work.

The device-entry cases below all fail host validation, so no kernel is ever
launched (the pointers passed are aligned dummies that are never read)."""
import ctypes
import os
import re

import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb
import oracle
from hadamard_rotated_quantized_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tb.h")

DUMMY = 0x10000  # aligned, never dereferenced (validation fails first)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tb_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = tb.lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    # and nothing unexpected is missing from the binding's signature table
    assert set(names) == set(tb._SIGNATURES)


def test_abi_version_and_status_strings():
    L = tb.lib()
    assert L.tb_abi_version() == 1
    for code, name in tb.STATUS.items():
        assert L.tb_status_str(code).decode() == name


@pytest.mark.parametrize("N,K", [(1, 128), (7, 1024), (33, 5120)])
def test_host_pack_matches_oracle_bitwise(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    t = synth.draw_ternary(rng, N, K)
    sc = synth.draw_scales(rng, N, K)
    c1, s1, b1 = tb.tb_pack(t, sc)
    c2, s2, b2 = oracle.pack(t, sc)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1.view(np.uint16), s2.view(np.uint16))
    np.testing.assert_array_equal(b1.view(np.uint16), b2.view(np.uint16))
    np.testing.assert_array_equal(tb.tb_unpack(c1, K), t)
    assert c1.nbytes + s1.nbytes + b1.nbytes == oracle.container_bytes(N, K)


def test_host_pack_rejects_non_ternary():
    t = np.zeros((2, 128), np.int8)
    t[1, 77] = 2
    with pytest.raises(tb.TBError) as e:
        tb.tb_pack(t, np.ones((2, 1), np.float16))
    assert e.value.status == -6


def test_host_unpack_rejects_code3():
    codes = np.zeros((1, 8), np.uint32)
    codes[0, 3] = 3 << 10
    with pytest.raises(tb.TBError) as e:
        tb.tb_unpack(codes, 128)
    assert e.value.status == -6


def test_signs_validate():
    s = np.ones(1024, np.int8)
    tb.tb_signs_validate(s)
    s[100] = 0
    with pytest.raises(tb.TBError) as e:
        tb.tb_signs_validate(s)
    assert e.value.status == -5


def test_pack_empty_is_noop():
    L = tb.lib()
    assert L.tb_pack(None, None, 0, 128, None, None, None) == 0
    assert L.tb_unpack(None, 0, 128, None) == 0


# --- device entry points: host-side validation only ------------------------
def _gemv(**kw):
    a = dict(x=DUMMY, dt=tb.TB_BF16, B=1, K=1024, signs=DUMMY, block=1024, codes=DUMMY, scales=DUMMY,
             biases=DUMMY, N=16, y=DUMMY, ws=DUMMY, wsb=0, st=None)
    a.update(kw)
    return tb.lib().tb_ternary_gemv(a["x"], a["dt"], a["B"], a["K"], a["signs"], a["block"], a["codes"],
                                    a["scales"], a["biases"], a["N"], a["y"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=300), -3),
    (dict(block=256), -3),
    (dict(K=1000), -2),
    (dict(K=1536), -2),           # not a multiple of block 1024
    (dict(K=0), -1),
    (dict(K=-128), -1),
    (dict(B=9), -2),
    (dict(B=-1), -1),
    (dict(N=-5), -1),
    (dict(signs=None), -1),       # block > 0 needs signs
    (dict(block=0), -1),          # block 0 takes no signs
    (dict(dt=7), -7),
    (dict(x=None), -1),
    (dict(codes=None), -1),
    (dict(codes=DUMMY + 4), -8),  # codes need 16-byte alignment
    (dict(y=DUMMY + 2), -8),
    (dict(x=DUMMY + 4), -8),      # x needs 16-byte alignment (vector loads)
    (dict(signs=DUMMY + 8), -8),
    (dict(y=None), -1),
    (dict(ws=None), -10),
    (dict(wsb=16), -10),
])
def test_gemv_rejects(kw, status):
    assert _gemv(**kw) == status
    assert tb.lib().tb_last_error().decode().startswith("tb_ternary_gemv")


def test_gemv_empty_is_noop():
    assert _gemv(B=0, x=None, y=None) == 0
    assert _gemv(N=0, codes=None, y=None) == 0


def test_gemv_workspace_size():
    L = tb.lib()
    assert L.tb_ternary_gemv_workspace_size(1, 5120) > 0
    assert L.tb_ternary_gemv_workspace_size(0, 5120) == 0
    assert L.tb_ternary_gemv_workspace_size(1, 100) == 0
    big = L.tb_ternary_gemv_workspace_size(8, 17408)
    # A operand: 3 int8 limbs per input, plus one float2 per group of 128
    assert big >= 8 * 17408 * 3 + 8 * (17408 // 128) * 8


def _gemm(**kw):
    a = dict(x=DUMMY, dt=tb.TB_BF16, M=64, K=1024, signs=DUMMY, block=1024, codes=DUMMY, scales=DUMMY,
             biases=DUMMY, N=16, y=DUMMY, ws=DUMMY, wsb=0, st=None)
    a.update(kw)
    return tb.lib().tb_ternary_gemm(a["x"], a["dt"], a["M"], a["K"], a["signs"], a["block"], a["codes"],
                                    a["scales"], a["biases"], a["N"], a["y"], a["ws"], a["wsb"], a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(block=100), -3), (dict(K=1100), -2), (dict(M=-1), -1), (dict(dt=3), -7),
    (dict(wsb=8), -10), (dict(scales=DUMMY + 1), -8), (dict(signs=None), -1),
    (dict(x=DUMMY + 4), -8),      # x needs 16-byte alignment (vector loads in the rotation)
    (dict(signs=DUMMY + 8), -8),
])
def test_gemm_rejects(kw, status):
    assert _gemm(**kw) == status


def test_gemm_prepare_rejects_misaligned_inputs():
    L = tb.lib()
    for x, sg in ((DUMMY + 4, DUMMY), (DUMMY, DUMMY + 8)):
        assert L.tb_ternary_gemm_prepare(x, tb.TB_BF16, 64, 1024, sg, 1024, DUMMY, 1 << 30, None) == -8


def test_gemm_workspace_size_n():
    L = tb.lib()
    base = L.tb_ternary_gemm_workspace_size(2048, 5120)
    assert base > 0 and L.tb_ternary_gemm_workspace_size(1, 100) == 0
    # invalid N falls back to the base size; a valid one is never smaller
    assert L.tb_ternary_gemm_workspace_size_n(2048, 5120, 0) == base
    assert L.tb_ternary_gemm_workspace_size_n(2048, 5120, 17408) >= base
    assert L.tb_ternary_gemm_workspace_size_n(64, 1024, 512) == L.tb_ternary_gemm_workspace_size(64, 1024)


def test_gemm_empty_is_noop():
    assert _gemm(M=0) == 0


@pytest.mark.parametrize("args,status", [
    (dict(block=0), -3),          # the standalone transform needs a block
    (dict(block=1024, K=1536), -2),
    (dict(inverse=2), -1),
    (dict(dt=5), -7),
    (dict(y=DUMMY + 2), -8),
    (dict(signs=None), -1),
])
def test_fwht_rejects(args, status):
    a = dict(x=DUMMY, dt=tb.TB_F32, y=DUMMY, signs=DUMMY, rows=2, K=2048, block=1024, inverse=0)
    a.update(args)
    assert tb.lib().tb_fwht_signed(a["x"], a["dt"], a["y"], a["signs"], a["rows"], a["K"], a["block"],
                                   a["inverse"], None) == status


@pytest.mark.parametrize("args,status", [
    (dict(block=333), -3), (dict(K=5000), -2), (dict(T=-1), -1), (dict(ids=None), -1),
    (dict(codes=DUMMY + 8), -8), (dict(signs=None), -1),
])
def test_embed_rejects(args, status):
    a = dict(ids=DUMMY, T=3, codes=DUMMY, scales=DUMMY, biases=DUMMY, V=10, K=5120, signs=DUMMY,
             block=1024, out=DUMMY)
    a.update(args)
    assert tb.lib().tb_embed_inverse(a["ids"], a["T"], a["codes"], a["scales"], a["biases"], a["V"], a["K"],
                                     a["signs"], a["block"], a["out"], None) == status


@pytest.mark.parametrize("args,status", [
    (dict(K=100), -2), (dict(bad=None), -1), (dict(t=DUMMY + 1), -8), (dict(N=-1), -1),
])
def test_pack_device_rejects(args, status):
    a = dict(t=DUMMY, s=DUMMY, N=4, K=256, c=DUMMY, so=DUMMY, bo=DUMMY, bad=DUMMY)
    a.update(args)
    assert tb.lib().tb_pack_device(a["t"], a["s"], a["N"], a["K"], a["c"], a["so"], a["bo"], a["bad"],
                                   None) == status


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        tb.tb_fwht_signed(torch.zeros(1, 1024), torch.ones(1024, dtype=torch.int8), 1024)


def test_gemv_rejects_scales_not_dword_aligned():
    # the decode-matmul kernels load scales and biases as dwords and vectors
    assert _gemv(scales=DUMMY + 2) == -8
    assert _gemv(biases=DUMMY + 2) == -8
    assert tb.lib().tb_ternary_gemv_run(DUMMY, 1 << 30, 1, 1024, DUMMY, DUMMY + 2, DUMMY, 16, DUMMY, None) == -8


# --- the Python binding checks tensor shapes before any pointer is passed ---
def _host_linear(N=32, K=1024, B=2):
    torch = pytest.importorskip("torch")
    return dict(x=torch.zeros(B, K, dtype=torch.bfloat16), signs=torch.ones(K, dtype=torch.int8),
                codes=torch.zeros(N, K // 16, dtype=torch.int32), scales=torch.zeros(N, K // 128, dtype=torch.float16),
                biases=torch.zeros(N, K // 128, dtype=torch.float16))


def _bad_variants():
    torch = pytest.importorskip("torch")
    return [
        ("codes", torch.zeros(32, 1024 // 16 - 1, dtype=torch.int32)),   # one word short per row
        ("codes", torch.zeros(32 * 64, dtype=torch.int32)),              # flat
        ("scales", torch.zeros(32, 4, dtype=torch.float16)),             # K/128 = 8
        ("biases", torch.zeros(31, 8, dtype=torch.float16)),             # N - 1 rows
        ("signs", torch.ones(512, dtype=torch.int8)),                    # half width
        ("x", torch.zeros(2, 1000, dtype=torch.bfloat16)),               # K not a multiple of 128
        ("x", torch.zeros(1024, dtype=torch.bfloat16)),                  # not 2-D
    ]


@pytest.mark.parametrize("i", range(7))
def test_binding_gemv_gemm_reject_mismatched_shapes(i):
    name, bad = _bad_variants()[i]
    for fn in (tb.tb_ternary_gemv, tb.tb_ternary_gemm):
        a = _host_linear()
        a[name] = bad
        with pytest.raises(ValueError):
            fn(a["x"], a["signs"], 1024, a["codes"], a["scales"], a["biases"])


def test_binding_rejects_wrong_out_and_sign_presence():
    torch = pytest.importorskip("torch")
    a = _host_linear()
    with pytest.raises(ValueError):
        tb.tb_ternary_gemv(a["x"], a["signs"], 1024, a["codes"], a["scales"], a["biases"],
                           out=torch.zeros(2, 31))
    with pytest.raises(ValueError):   # block 0 takes no signs
        tb.tb_ternary_gemv(a["x"], a["signs"], 0, a["codes"], a["scales"], a["biases"])
    with pytest.raises(ValueError):   # a block needs signs
        tb.tb_ternary_gemm(a["x"], None, 1024, a["codes"], a["scales"], a["biases"])
    with pytest.raises(ValueError):
        tb.tb_ternary_gemv_run(torch.zeros(16, dtype=torch.uint8), 2, 2048, a["codes"], a["scales"], a["biases"])
    with pytest.raises(ValueError):
        tb.tb_ternary_gemm_run(torch.zeros(16, dtype=torch.uint8), 2, 1024, a["codes"], a["scales"][:, :4],
                               a["biases"])


def test_binding_embed_fwht_pack_reject_mismatched_shapes():
    torch = pytest.importorskip("torch")
    a = _host_linear()
    ids = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError):
        tb.tb_embed_inverse(ids, a["codes"], a["scales"][:, :7], a["biases"], a["signs"], 1024)
    with pytest.raises(ValueError):
        tb.tb_embed_inverse(ids, a["codes"], a["scales"], a["biases"], a["signs"][:1000], 1024)
    with pytest.raises(ValueError):
        tb.tb_embed_inverse(ids.view(3, 1), a["codes"], a["scales"], a["biases"], a["signs"], 1024)
    with pytest.raises(ValueError):
        tb.tb_fwht_signed(torch.zeros(2, 2048), torch.ones(1024, dtype=torch.int8), 1024)
    with pytest.raises(ValueError):
        tb.tb_fwht_signed(torch.zeros(2, 1024), torch.ones(1024, dtype=torch.int8), 1024, out=torch.zeros(1, 1024))
    with pytest.raises(ValueError):
        tb.tb_pack_device(torch.zeros(4, 256, dtype=torch.int8), torch.zeros(4, 3, dtype=torch.float16))


def test_binding_multi_plan_rejects_mismatched_module():
    torch = pytest.importorskip("torch")
    a = _host_linear(B=1)
    y = torch.zeros(1, 32)
    mod = [a["x"], a["signs"], a["codes"], a["scales"], a["biases"], y]
    for j, bad in ((2, a["codes"][:, :10]), (3, a["scales"][:5]), (1, a["signs"][:100]), (5, torch.zeros(1, 30)),
                   (0, torch.zeros(2, 1024, dtype=torch.bfloat16))):
        m = list(mod)
        m[j] = bad
        with pytest.raises(ValueError):
            tb.tb_gemv_multi_plan([tuple(m)], 1024)


def test_host_pack_unpack_reject_bad_shapes():
    with pytest.raises(ValueError):
        tb.tb_pack(np.zeros((4, 100), np.int8), np.zeros((4, 0), np.float16))
    with pytest.raises(ValueError):
        tb.tb_unpack(np.zeros((4, 63), np.uint32), 1024)
