"""tb_ternary_gemv_noalloc: tb_ternary_gemv with the library's static device
scratch as its workspace.  Through the C ABI, against tb_ternary_gemv with
a caller workspace on the same inputs (the same kernels: bitwise equal) and
against the fp64 oracle under the parity bar, on calls in a row that shrink,
so each call finds the previous call's contents in the scratch."""
import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb
import oracle
from hadamard_rotated_quantized_amd import synth
from gpu_util import announce, compare, cuda_available, pack_to_device, signs_to_device, torch, x_to_device

DUMMY = 0x10000  # aligned, never dereferenced (validation fails first)


def test_noalloc_refuses_a_workspace_beyond_its_scratch():
    """Host-side refusal before any device work: B = 8 at K = 2^20 needs more
    than the scratch holds even on its smallest path."""
    L = tb.lib()
    K = 1 << 20
    assert L.tb_ternary_gemv_workspace_size(8, K) > 16 << 20
    st = L.tb_ternary_gemv_noalloc(DUMMY, tb.TB_BF16, 8, K, DUMMY, 1024, DUMMY, DUMMY, DUMMY, 64, DUMMY, None)
    assert st == -10
    assert "scratch" in L.tb_last_error().decode()
    # ordinary argument errors come first, as in tb_ternary_gemv
    assert L.tb_ternary_gemv_noalloc(DUMMY, tb.TB_BF16, 9, 1024, DUMMY, 1024, DUMMY, DUMMY, DUMMY, 64, DUMMY,
                                     None) == -2
    assert L.tb_ternary_gemv_noalloc(DUMMY, tb.TB_BF16, 1, 1024, DUMMY, 1024, DUMMY, DUMMY + 2, DUMMY, 64, DUMMY,
                                     None) == -8


CALLS = [
    # (N, K, B, seed, sampled oracle rows or None for all rows)
    (5120, 17408, 8, 91, None),      # decode-batch path, 6 K slices of partial rows in the scratch
    (700, 5120, 2, 92, None),        # smaller: fewer partial rows over the previous call's
    (300000, 5120, 8, 93, 256),      # partial rows (19.2 MB) would exceed the scratch: prepared activation in it
    (6144, 5120, 1, 94, None),       # batch 1 (single-launch kernel)
    (300, 1152, 3, 95, None),        # block 0, K not a multiple of 256
]


def _problem(N, K, B, seed, block):
    """(t rows getter, scales rows getter, x64, device tensors): host draws,
    except for the largest case, drawn on the device."""
    T = torch()
    if N * K <= 1 << 28:
        p = synth.make_problem("noalloc", N, K, B, seed, "bf16", block)
        codes, s, b = pack_to_device(p.t, p.scales)
        return (lambda r: p.t[r]), (lambda r: p.scales[r]), p.x64, p.signs, (x_to_device(p), codes, s, b)
    t, sc, x = synth.device_module_draw(seed, N, K, B, "cuda")
    codes, s, b = tb.tb_pack_device(t, sc)
    sig = synth.draw_signs(np.random.default_rng(seed), K) if block else None
    return ((lambda r: t[T.from_numpy(r).cuda()].cpu().numpy()), (lambda r: sc[T.from_numpy(r).cuda()].cpu().numpy()),
            x.float().cpu().numpy().astype(np.float64), sig, (x, codes, s, b))


@pytest.mark.gpu
@pytest.mark.skipif(not cuda_available(), reason="needs a GPU")
def test_noalloc_matches_workspace_calls_and_oracle_on_shrinking_calls():
    T = torch()
    for N, K, B, seed, sample in CALLS:
        announce(f"noalloc N={N} K={K} B={B}")
        block = 1024 if K % 1024 == 0 else 0
        t_rows, sc_rows, x64, sig, (x, codes, s, b) = _problem(N, K, B, seed, block)
        sg = signs_to_device(sig)
        need_n = tb.tb_ternary_gemv_workspace_size_n(B, K, N)
        ws = T.empty(need_n if need_n <= (16 << 20) else tb.tb_ternary_gemv_workspace_size(B, K),
                     dtype=T.uint8, device="cuda")
        y_ref = tb.tb_ternary_gemv(x, sg, block, codes, s, b, workspace=ws)
        y = tb.tb_ternary_gemv_noalloc(x, sg, block, codes, s, b)
        y2 = tb.tb_ternary_gemv_noalloc(x, sg, block, codes, s, b)
        T.cuda.synchronize()
        assert T.equal(y, y_ref), (N, K, B)
        assert T.equal(y2, y_ref), (N, K, B)
        rows = np.arange(N) if sample is None else np.unique(np.concatenate(
            [[0, N - 1], np.random.default_rng(seed).integers(0, N, sample)]))
        oc, osc, ob = oracle.pack(t_rows(rows), sc_rows(rows))
        want = oracle.packed_linear(x64, sig, block, oc, osc, ob)
        compare(y[:, T.from_numpy(rows).cuda()].cpu().numpy(), want, f"noalloc N={N} K={K} B={B}")
