"""Parity of the HIP path against the fp64 oracle on the GPU.

Bars: relative L2 <= 1e-4 and max |err| <= 1e-3 * max |y| for floating point
results; bit-exact for packing and for code decoding (one-hot inputs through
the unrotated GEMV, and unrotated embedding rows)."""
import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb
import oracle
from hadamard_rotated_quantized_amd import synth
from gpu_util import (announce, compare, cuda_available, oracle_pack, pack_to_device, signs_to_device,
                      torch, x_to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _gemv_case(p, B=None):
    T = torch()
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    y = tb.tb_ternary_gemv(x, sg, p.block, codes, s, b)
    T.cuda.synchronize()
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, p.block, oc, osc, ob)
    return y.cpu().numpy(), want


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------
def test_tiny_packed_linear():
    announce("tiny K=1024 N=256 B=1 fp32 seed 0")
    p = synth.config_problem("tiny")
    got, want = _gemv_case(p)
    compare(got, want, "tiny")


def test_q_proj_gemv():
    announce("q_proj K=5120 N=6144 B=1 bf16 seed 2")
    p = synth.config_problem("q_proj")
    got, want = _gemv_case(p)
    compare(got, want, "q_proj")


def test_down_proj_gemv_batches():
    announce("down_proj K=17408 N=5120 B=1/2/4/8 bf16 seed 3")
    T = torch()
    p = synth.config_problem("down_proj")
    codes, s, b = pack_to_device(p.t, p.scales)
    sg = signs_to_device(p.signs)
    x8 = x_to_device(p)
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, 1024, oc, osc, ob)  # rows are independent
    for B in (1, 2, 4, 8):
        announce(f"down_proj B={B}")
        y = tb.tb_ternary_gemv(x8[:B].contiguous(), sg, 1024, codes, s, b)
        T.cuda.synchronize()
        compare(y.cpu().numpy(), want[:B], f"down_proj B={B}")


def test_prefill_gemm_full():
    """Every one of the 2048 x 17408 outputs against the fp64 oracle, in the
    launch configuration the benchmark times (the workspace that enables the
    tail split)."""
    announce("prefill_gate_up M=2048 K=5120 N=17408 bf16 seed 4 (all outputs)")
    T = torch()
    p = synth.config_problem("prefill_gate_up")
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    ws = T.empty(tb.tb_ternary_gemm_workspace_size_n(p.B, p.K, p.N), dtype=T.uint8, device="cuda")
    y = tb.tb_ternary_gemm(x, sg, 1024, codes, s, b, workspace=ws)
    T.cuda.synchronize()
    got = y.cpu().numpy()
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, 1024, oc, osc, ob)
    compare(got, want, "prefill all outputs")
    # and per 64 x 512 output tile (whole tiles and the tail's K-sliced tiles)
    tile_err = np.abs(got - want).reshape(p.B // 64, 64, -1).max(axis=1)
    assert np.isfinite(tile_err).all()
    assert tile_err.max() <= 1e-3 * np.abs(want).max()


# --------------------------------------------------------------------------
# ragged shapes, other block sizes, batches, dtypes
# --------------------------------------------------------------------------
RAGGED = [
    # (N, K, B, block, xdtype)
    (1, 1024, 1, 1024, "bf16"),
    (4352, 384, 1, 0, "bf16"),    # G = 3 odd: band rows rounded to a multiple of 8 (17 -> 24)
    (4099, 1152, 1, 0, "f32"),    # G = 9 odd, ragged last band
    (17, 2048, 3, 512, "f32"),
    (1000, 6144, 2, 2048, "bf16"),
    (100, 8192, 5, 4096, "bf16"),
    (45, 384, 1, 0, "f32"),       # 3 groups: partial super-span
    (300, 640, 7, 0, "bf16"),     # 5 groups
    (4099, 1024, 8, 1024, "f32"),
    (16, 5120, 6, 1024, "bf16"),
]


@pytest.mark.parametrize("N,K,B,block,xd", RAGGED)
def test_gemv_ragged(N, K, B, block, xd):
    announce(f"gemv ragged N={N} K={K} B={B} block={block} x={xd}")
    p = synth.make_problem("ragged", N, K, B, [N, K, B, block], xd, block)
    got, want = _gemv_case(p)
    compare(got, want, f"gemv N={N} K={K} B={B} block={block}")


GEMM_CASES = [
    (200, 300, 2048, 1024, "bf16"),
    (100, 260, 4096, 2048, "bf16"),
    (33, 70, 2048, 2048, "f32"),
    (1, 77, 1024, 512, "f32"),
    (129, 129, 4096, 4096, "bf16"),
    (64, 256, 384, 0, "f32"),
]


@pytest.mark.parametrize("M,N,K,block,xd", GEMM_CASES)
def test_gemm_small_full(M, N, K, block, xd):
    announce(f"gemm M={M} N={N} K={K} block={block} x={xd}")
    T = torch()
    p = synth.make_problem("gemm", N, K, M, [M, N, K, block, 9], xd, block)
    codes, s, b = pack_to_device(p.t, p.scales)
    y = tb.tb_ternary_gemm(x_to_device(p), signs_to_device(p.signs), block, codes, s, b)
    T.cuda.synchronize()
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, block, oc, osc, ob)
    compare(y.cpu().numpy(), want, f"gemm M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,block,xd", [
    (1083, 8092, 2560, 512, "f32"),    # 272 tiles: 16 tail tiles x 8 slices of 2-3 groups, ragged M, N
    (640, 13312, 2048, 1024, "bf16"),  # 260 tiles: 4 tail tiles x 8 slices of 2 groups
])
def test_gemm_tail_split_matches_oracle_and_whole_tiles(M, N, K, block, xd):
    """More output tiles than one round of the chip with a short last round:
    the tail tiles run as K slices whose partials a second kernel adds in
    order.  Against the oracle, against a run whose workspace is too small
    for the split (every tile whole), and bitwise against itself."""
    announce(f"gemm tail split M={M} N={N} K={K} block={block} x={xd}")
    T = torch()
    p = synth.make_problem("gemm_split", N, K, M, [M, N, K, block, 13], xd, block)
    codes, s, b = pack_to_device(p.t, p.scales)
    x, sg = x_to_device(p), signs_to_device(p.signs)
    need, base = tb.tb_ternary_gemm_workspace_size_n(M, K, N), tb.tb_ternary_gemm_workspace_size(M, K)
    assert need > base
    ws = T.empty(need, dtype=T.uint8, device="cuda")
    y1 = tb.tb_ternary_gemm(x, sg, block, codes, s, b, workspace=ws)
    y2 = tb.tb_ternary_gemm(x, sg, block, codes, s, b, workspace=ws)
    yw = tb.tb_ternary_gemm(x, sg, block, codes, s, b, workspace=T.empty(base, dtype=T.uint8, device="cuda"))
    T.cuda.synchronize()
    assert T.equal(y1, y2)
    d = (y1.double() - yw.double()).abs().max().item()
    assert d <= 1e-5 * yw.abs().max().item(), d
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, block, oc, osc, ob)
    compare(y1.cpu().numpy(), want, f"gemm split M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,block,xd", [
    (300, 1000, 1024, 1024, "bf16"),  # 5 row tiles, ragged last column tile (488 rows)
    (256, 512, 2560, 512, "f32"),     # exactly 4 row tiles, one column tile
])
def test_gemm_packed_weights_match_stored_layout(M, N, K, block, xd):
    """With at least 4 row tiles and a workspace of
    tb_ternary_gemm_workspace_size_n, the run first copies the codes and
    scales into one contiguous record per (column tile, group) and the matmul
    reads that copy; the arithmetic is the same as reading the weights as
    stored (a workspace of tb_ternary_gemm_workspace_size), so the two agree
    bitwise when no tile is split, and both match the oracle."""
    announce(f"gemm packed weights M={M} N={N} K={K} block={block} x={xd}")
    T = torch()
    p = synth.make_problem("gemm_pack", N, K, M, [M, N, K, block, 17], xd, block)
    codes, s, b = pack_to_device(p.t, p.scales)
    x, sg = x_to_device(p), signs_to_device(p.signs)
    need, base = tb.tb_ternary_gemm_workspace_size_n(M, K, N), tb.tb_ternary_gemm_workspace_size(M, K)
    assert need > base
    yp = tb.tb_ternary_gemm(x, sg, block, codes, s, b, workspace=T.empty(need, dtype=T.uint8, device="cuda"))
    ys = tb.tb_ternary_gemm(x, sg, block, codes, s, b, workspace=T.empty(base, dtype=T.uint8, device="cuda"))
    T.cuda.synchronize()
    assert T.equal(yp, ys)
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, block, oc, osc, ob)
    compare(yp.cpu().numpy(), want, f"gemm packed M={M} N={N} K={K}")


def test_gemm_biases_not_16_byte_aligned():
    """The epilogue reads the biases as 16-byte vectors only when they are
    16-byte aligned; a pack whose biases start 4 elements into a buffer takes
    the 2-byte loads and must give the same result."""
    announce("gemm M=96 N=600 K=1024 with biases at a 8-byte offset")
    T = torch()
    M, N, K = 96, 600, 1024
    p = synth.make_problem("gemm_unaligned", N, K, M, [M, N, K, 21], "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x, sg = x_to_device(p), signs_to_device(p.signs)
    buf = T.empty(b.numel() + 4, dtype=b.dtype, device="cuda")
    b_off = buf[4:].view(b.shape)
    b_off.copy_(b)
    assert b_off.data_ptr() % 16 == 8
    y_al = tb.tb_ternary_gemm(x, sg, 1024, codes, s, b)
    y_un = tb.tb_ternary_gemm(x, sg, 1024, codes, s, b_off)
    T.cuda.synchronize()
    assert T.equal(y_al, y_un)
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, 1024, oc, osc, ob)
    compare(y_un.cpu().numpy(), want, "gemm unaligned biases")


# --------------------------------------------------------------------------
# exact decode, general affine decode, degenerate cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("xd", ["f32", "bf16"])
def test_gemv_one_hot_decode_is_exact(xd):
    """Unrotated GEMV with x = e_k returns column k of W~ exactly."""
    announce(f"gemv one-hot decode x={xd}")
    T = torch()
    N, K = 300, 1024
    rng = np.random.default_rng(7)
    t = synth.draw_ternary(rng, N, K)
    sc = synth.draw_scales(rng, N, K)
    codes, s, b = pack_to_device(t, sc)
    oc, osc, ob = oracle.pack(t, sc)
    W = oracle.dequantize(oc, osc, ob, K)
    ks = [0, 1, 5, 15, 16, 127, 128, 511, 512, 1023]
    dt = T.float32 if xd == "f32" else T.bfloat16
    x = T.zeros((len(ks), K), dtype=dt)
    for i, k in enumerate(ks):
        x[i, k] = 1
    xs = x.cuda()
    for i0 in range(0, len(ks), 8):
        y = tb.tb_ternary_gemv(xs[i0:i0 + 8].contiguous(), None, 0, codes, s, b)
        T.cuda.synchronize()
        for j, k in enumerate(ks[i0:i0 + 8]):
            np.testing.assert_array_equal(y[j].cpu().numpy(), W[:, k].astype(np.float32))


def test_gemv_general_bias_and_code3():
    """Stored biases unrelated to the scales, and code 3 present: the kernel
    decodes s*c + b from storage and does not assume b = -s."""
    announce("gemv general affine decode")
    T = torch()
    N, K, B = 513, 3072, 3
    rng = np.random.default_rng(8)
    words = rng.integers(0, 2 ** 32, size=(N, K // 16), dtype=np.uint64).astype(np.uint32)
    sc = (rng.standard_normal((N, K // 128)) * 0.05).astype(np.float16)
    bi = (rng.standard_normal((N, K // 128)) * 0.05).astype(np.float16)
    sig = synth.draw_signs(rng, K)
    x64, xs = synth.draw_activations(rng, B, K, "bf16")
    y = tb.tb_ternary_gemv(T.from_numpy(xs.view(np.int16)).view(T.bfloat16).cuda(),
                           T.from_numpy(sig).cuda(), 1024, T.from_numpy(words.view(np.int32)).cuda(),
                           T.from_numpy(sc).cuda(), T.from_numpy(bi).cuda())
    T.cuda.synchronize()
    want = oracle.packed_linear(x64, sig, 1024, words, sc, bi)
    compare(y.cpu().numpy(), want, "general affine")
    # the same container through the GEMM
    yg = tb.tb_ternary_gemm(T.from_numpy(xs.view(np.int16)).view(T.bfloat16).cuda(),
                            T.from_numpy(sig).cuda(), 1024, T.from_numpy(words.view(np.int32)).cuda(),
                            T.from_numpy(sc).cuda(), T.from_numpy(bi).cuda())
    T.cuda.synchronize()
    compare(yg.cpu().numpy(), want, "general affine gemm")


def test_gemv_zero_weights_give_zero():
    """All ternary zeros (W~ = 0): the per-group factorization s*sum(c x) +
    b*sum(x) cancels up to fp32 rounding of the two group terms, so |y| is
    bounded by 1e-6 * max(s) * sum|xr| (exact zero is not promised)."""
    announce("gemv all-zero ternary")
    T = torch()
    N, K = 77, 2048
    rng = np.random.default_rng(9)
    sc = synth.draw_scales(rng, N, K)
    codes, s, b = pack_to_device(np.zeros((N, K), np.int8), sc)
    sig = synth.draw_signs(rng, K)
    x64, xs = synth.draw_activations(rng, 4, K, "bf16")
    y = tb.tb_ternary_gemv(T.from_numpy(xs.view(np.int16)).view(T.bfloat16).cuda(), signs_to_device(sig),
                           1024, codes, s, b)
    T.cuda.synchronize()
    xr = oracle.fwht_signed(x64, sig, 1024)
    bound = 1e-6 * float(sc.astype(np.float64).max()) * np.abs(xr).sum(axis=1)
    assert (np.abs(y.cpu().numpy()).max(axis=1) <= bound).all()


def test_gemv_batch_rows_match_single_rows():
    """Row b of a batched call equals the call on x[b] alone.  Batch sizes
    that share a kernel configuration ({2, 3, 4} and {5, ..., 8}) give
    bitwise-identical rows; across configurations (batch 1 runs a different
    MFMA shape) rows agree within 1e-6 relative."""
    announce("gemv batch consistency")
    T = torch()
    p = synth.make_problem("batch", 700, 5120, 8, 31, "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    y = {B: tb.tb_ternary_gemv(x[:B].contiguous(), sg, 1024, codes, s, b) for B in range(1, 9)}
    T.cuda.synchronize()
    for B in (3, 4):
        assert T.equal(y[B][:2], y[2]), B
    for B in (6, 7, 8):
        assert T.equal(y[B][:5], y[5]), B
    for i in range(8):
        y1 = tb.tb_ternary_gemv(x[i:i + 1].contiguous(), sg, 1024, codes, s, b)
        T.cuda.synchronize()
        d = (y1[0].double() - y[8][i].double()).abs().max().item()
        assert d <= 1e-6 * y1[0].abs().max().item(), (i, d)


def test_gemv_linearity():
    announce("gemv linearity")
    T = torch()
    p = synth.make_problem("lin", 256, 2048, 2, 32, "f32", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    y = tb.tb_ternary_gemv(x, sg, 1024, codes, s, b)
    z = tb.tb_ternary_gemv((2.5 * x[0:1] - 0.5 * x[1:2]).contiguous(), sg, 1024, codes, s, b)
    T.cuda.synchronize()
    want = 2.5 * y[0].double() - 0.5 * y[1].double()
    err = (z[0].double() - want).abs().max().item()
    assert err <= 1e-5 * want.abs().max().item()


def test_gemv_writes_only_its_output():
    announce("gemv output bounds")
    T = torch()
    p = synth.make_problem("bounds", 33, 1024, 2, 33, "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    out = T.full((2 * 33 + 64,), 12345.0, device="cuda")
    y = out[:66].view(2, 33)
    tb.tb_ternary_gemv(x_to_device(p), signs_to_device(p.signs), 1024, codes, s, b, out=y)
    T.cuda.synchronize()
    assert (out[66:] == 12345.0).all()


# --------------------------------------------------------------------------
# standalone transform
# --------------------------------------------------------------------------
@pytest.mark.parametrize("block", [512, 1024, 2048, 4096])
def test_fwht_matches_oracle_and_inverts(block):
    announce(f"fwht block={block}")
    T = torch()
    rng = np.random.default_rng(block)
    K = 2 * block if block < 4096 else 8192
    rows = 5
    x = rng.standard_normal((rows, K)).astype(np.float32)
    sig = synth.draw_signs(rng, K)
    xd = T.from_numpy(x).cuda()
    sd = T.from_numpy(sig).cuda()
    y = tb.tb_fwht_signed(xd, sd, block)
    back = tb.tb_fwht_signed(y, sd, block, inverse=True)
    T.cuda.synchronize()
    want = oracle.fwht_signed(x.astype(np.float64), sig, block)
    np.testing.assert_allclose(y.cpu().numpy(), want, rtol=0, atol=2e-6 * np.abs(want).max())
    np.testing.assert_allclose(back.cpu().numpy(), x, rtol=0, atol=2e-6 * np.abs(x).max())
    wi = oracle.fwht_signed(x.astype(np.float64), sig, block, inverse=True)
    yi = tb.tb_fwht_signed(xd, sd, block, inverse=True)
    xb = xd.clone()
    tb.tb_fwht_signed(xb, sd, block, out=xb)  # in place
    T.cuda.synchronize()
    np.testing.assert_allclose(yi.cpu().numpy(), wi, rtol=0, atol=2e-6 * np.abs(wi).max())
    assert T.equal(xb, y)


@pytest.mark.parametrize("block", [512, 1024])
def test_offline_fold_on_device_recovers_packed_weights(block):
    """The offline fold W_s = W R^T is the forward signed transform of each
    weight row, so tb_fwht_signed over the rows of a dense W performs it.
    W is built on the host as W~ R from packed ternary weights W~; the device
    fold must give back W~ (and its ternary codes), and the Packed linear on
    W~ must equal the unrotated product W x."""
    announce(f"offline fold block={block}")
    T = torch()
    rng = np.random.default_rng(31 + block)
    N, K = 96, 3 * block * (2 if block == 512 else 1)
    t = synth.draw_ternary(rng, N, K)
    sc = synth.draw_scales(rng, N, K)
    sig = synth.draw_signs(rng, K)
    oc, osc, ob = oracle.pack(t, sc)
    w_packed = oracle.dequantize(oc, osc, ob, K)
    W = oracle.fwht_signed(w_packed, sig, block, inverse=True)  # W~ R, row by row
    sd = signs_to_device(sig)
    Wd = T.from_numpy(W.astype(np.float32)).cuda()
    Ws = tb.tb_fwht_signed(Wd, sd, block)
    T.cuda.synchronize()
    got = Ws.cpu().numpy().astype(np.float64)
    compare(got, oracle.fold_rotation(W.astype(np.float32), sig, block), "fold vs oracle")
    g = np.arange(K) // 128
    s64 = sc.astype(np.float64)[:, g]
    assert np.array_equal(np.rint(got / s64).astype(np.int8), t)
    x64, x = synth.draw_activations(rng, 2, K, "f32")
    codes, s, b = pack_to_device(t, sc)
    y = tb.tb_ternary_gemv(T.from_numpy(np.ascontiguousarray(x)).cuda(), sd, block, codes, s, b)
    T.cuda.synchronize()
    compare(y.cpu().numpy(), x64 @ W.T, "Packed linear vs unrotated product")


def test_fwht_bf16_input():
    announce("fwht bf16")
    T = torch()
    rng = np.random.default_rng(5)
    x64, xs = synth.draw_activations(rng, 3, 5120, "bf16")
    sig = synth.draw_signs(rng, 5120)
    y = tb.tb_fwht_signed(T.from_numpy(xs.view(np.int16)).view(T.bfloat16).cuda(), T.from_numpy(sig).cuda(),
                          1024)
    T.cuda.synchronize()
    want = oracle.fwht_signed(x64, sig, 1024)
    np.testing.assert_allclose(y.cpu().numpy(), want, rtol=0, atol=2e-6 * np.abs(want).max())


# --------------------------------------------------------------------------
# embedding
# --------------------------------------------------------------------------
def test_embed_inverse_parity_and_invalid_ids():
    announce("embed V=1000 K=5120")
    T = torch()
    V, K = 1000, 5120
    rng = np.random.default_rng(10)
    t = synth.draw_ternary(rng, V, K)
    sc = synth.draw_scales(rng, V, K)
    sig = synth.draw_signs(rng, K)
    codes, s, b = pack_to_device(t, sc)
    ids = np.array([0, V - 1, 17, 17, -1, V, 512, 2 ** 31 - 1], np.int32)
    out = tb.tb_embed_inverse(T.from_numpy(ids).cuda(), codes, s, b, signs_to_device(sig), 1024)
    T.cuda.synchronize()
    oc, osc, ob = oracle.pack(t, sc)
    want = oracle.embed_inverse(ids, oc, osc, ob, sig, 1024)
    got = out.cpu().numpy()
    ok = (ids >= 0) & (ids < V)
    assert np.isnan(got[~ok]).all()
    compare(got[ok], want[ok], "embed")


def test_embed_unrotated_decode_is_exact():
    announce("embed block 0 exact decode")
    T = torch()
    V, K = 64, 640
    rng = np.random.default_rng(11)
    t = synth.draw_ternary(rng, V, K)
    sc = synth.draw_scales(rng, V, K)
    codes, s, b = pack_to_device(t, sc)
    ids = np.arange(V, dtype=np.int32)[::-1].copy()
    out = tb.tb_embed_inverse(T.from_numpy(ids).cuda(), codes, s, b, None, 0)
    T.cuda.synchronize()
    oc, osc, ob = oracle.pack(t, sc)
    np.testing.assert_array_equal(out.cpu().numpy(),
                                  oracle.dequantize_rows(oc, osc, ob, K, ids).astype(np.float32))


def test_embed_gemv_duality():
    """<embed(r), x> == gemv(x)[r] for the same pack and signs."""
    announce("embed/gemv duality")
    T = torch()
    V, K = 96, 5120
    rng = np.random.default_rng(12)
    t = synth.draw_ternary(rng, V, K)
    sc = synth.draw_scales(rng, V, K)
    sig = synth.draw_signs(rng, K)
    codes, s, b = pack_to_device(t, sc)
    sd = signs_to_device(sig)
    x64, xs = synth.draw_activations(rng, 1, K, "f32")
    x = T.from_numpy(xs).cuda()
    y = tb.tb_ternary_gemv(x, sd, 1024, codes, s, b)[0].double()
    e = tb.tb_embed_inverse(T.arange(V, dtype=T.int32).cuda(), codes, s, b, sd, 1024).double()
    T.cuda.synchronize()
    d = e @ x[0].double()
    assert (d - y).abs().max().item() <= 1e-4 * y.abs().max().item()


# --------------------------------------------------------------------------
# device packer
# --------------------------------------------------------------------------
def test_pack_device_matches_host_pack():
    announce("pack_device")
    T = torch()
    N, K = 333, 5120
    rng = np.random.default_rng(13)
    t = synth.draw_ternary(rng, N, K)
    sc = synth.draw_scales(rng, N, K)
    c, s, b = tb.tb_pack_device(T.from_numpy(t).cuda(), T.from_numpy(sc).cuda())
    T.cuda.synchronize()
    hc, hs, hb = tb.tb_pack(t, sc)
    np.testing.assert_array_equal(c.cpu().numpy().view(np.uint32), hc)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint16), hs.view(np.uint16))
    np.testing.assert_array_equal(b.cpu().numpy().view(np.uint16), hb.view(np.uint16))
    t[5, 9] = 3
    t[300, 0] = -2
    with pytest.raises(tb.TBError):
        tb.tb_pack_device(T.from_numpy(t).cuda(), T.from_numpy(sc).cuda())


# --------------------------------------------------------------------------
# graph capture of the step (prepare + run)
# --------------------------------------------------------------------------
def test_gemv_graph_replays_match_eager():
    """Capture prepare + run in a HIP graph, replay it several times with
    eager work in between, and compare every replay bitwise with the eager
    result (the kernels are deterministic)."""
    announce("gemv graph replay")
    T = torch()
    p = synth.make_problem("graph", 1000, 5120, 2, 41, "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    ws = tb.tb_ternary_gemv_prepare(x, sg, 1024)
    eager = tb.tb_ternary_gemv_run(ws, 2, 5120, codes, s, b)
    T.cuda.synchronize()
    y = T.empty_like(eager)
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        tb.tb_ternary_gemv_prepare(x, sg, 1024, ws)
        tb.tb_ternary_gemv_run(ws, 2, 5120, codes, s, b, out=y)
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        T.cuda.synchronize()
        assert T.equal(y, eager), i
        tb.tb_ternary_gemv(x, sg, 1024, codes, s, b)  # eager work between replays
        T.cuda.synchronize()


# --------------------------------------------------------------------------
# the single-launch path (tb_ternary_gemv on short inputs) against the
# oracle and against the two-kernel prepare/run path on the same inputs
# --------------------------------------------------------------------------
TWO_PATHS = [
    # (N, K, B, block, xdtype)
    (6144, 5120, 1, 1024, "bf16"),   # the q_proj shape
    (777, 17408, 1, 1024, "bf16"),   # 17 chunks: three transforms on wave 0
    (1000, 3072, 8, 1024, "bf16"),   # 24 chunk transforms: three per wave
    (333, 1024, 4, 512, "f32"),
    (250, 2304, 3, 0, "bf16"),       # partial last chunk, 18 groups (2 padding)
    (5000, 640, 2, 0, "f32"),
    (9000, 1024, 1, 1024, "bf16"),   # 563 tiles: 4 waves per tile
    (45, 640, 1, 0, "f32"),          # 5 groups (3 padding), last band of 13 rows
    (1000, 384, 2, 0, "bf16"),       # 6-byte scale rows: band ends mid 16 bytes
    (6000, 8192, 1, 1024, "bf16"),   # band kernel, 4 matmul items per wave
    (6000, 4096, 1, 512, "f32"),     # band kernel, 2 items per wave, 512-blocks
    (1500, 3072, 6, 512, "f32"),     # K-split batch kernel, two sets of 4 batch rows
    (777, 17408, 3, 1024, "f32"),    # K-split batch kernel, several slices, ragged N
    (1003, 2304, 7, 0, "bf16"),      # batch kernel: second set of 3 batch rows, 18 groups (partial last chunk)
    (517, 5120, 5, 1024, "f32"),     # batch kernel: fp32 x in registers, staged signs, second set of 1 row
    (2000, 17408, 7, 1024, "bf16"),  # batch kernel: six slices, staged bf16 x, ragged last row block
    (300, 9216, 2, 512, "bf16"),     # batch kernel: 512-blocks, 9 chunks
    (4997, 17408, 1, 1024, "bf16"),  # fused, 20-row bands: 4-row remainder blocks, last band of 17 rows
    (4370, 17408, 1, 1024, "f32"),   # fused, 18-row bands (2-row remainder), last band of 14 rows
    (4352, 16896, 1, 512, "bf16"),   # fused, 17-row bands (1-row remainder), 132 groups: last unit half padding
    (4998, 6144, 1, 1024, "f32"),    # band kernel, 20-row bands: one remainder quad, last band of 18 rows
]


@pytest.mark.parametrize("N,K,B,block,xd", TWO_PATHS)
def test_gemv_single_launch_matches_oracle_and_two_kernel_path(N, K, B, block, xd):
    announce(f"gemv one call vs prepare/run N={N} K={K} B={B} block={block} x={xd}")
    T = torch()
    p = synth.make_problem("paths", N, K, B, [N, K, B, block, 3], xd, block)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    y1 = tb.tb_ternary_gemv(x, sg, block, codes, s, b)
    ws = tb.tb_ternary_gemv_prepare(x, sg, block)
    y2 = tb.tb_ternary_gemv_run(ws, B, K, codes, s, b)
    T.cuda.synchronize()
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear(p.x64, p.signs, block, oc, osc, ob)
    compare(y1.cpu().numpy(), want, "one call")
    compare(y2.cpu().numpy(), want, "prepare/run")
    d = (y1.double() - y2.double()).abs().max().item()
    assert d <= 1e-6 * y2.abs().max().item(), d


@pytest.mark.parametrize("N,B", [(70000, 1), (140000, 4)])
def test_gemv_wide_layer_sampled_rows(N, B):
    """Wide layers: one wave per tile and workgroups that loop over several
    tile groups; checked on sampled output rows, the last rows included."""
    announce(f"gemv wide N={N} K=1024 B={B}")
    T = torch()
    p = synth.make_problem("wide", N, 1024, B, [N, B, 5], "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    y = tb.tb_ternary_gemv(x_to_device(p), signs_to_device(p.signs), 1024, codes, s, b)
    T.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 15, 16, 31, 32, N // 2, N - 33, N - 17, N - 1],
                                     np.random.default_rng(N).integers(0, N, 200)]))
    oc, osc, ob = oracle_pack(p)
    want = oracle.packed_linear_rows(p.x64, p.signs, 1024, oc, osc, ob, rows)
    compare(y.cpu().numpy()[:, rows], want, f"wide N={N} B={B}")


def test_maximum_size_lm_head_and_embedding_table():
    """The largest module: the lm_head / embedding table of V = 248,320 rows
    of K = 5120 (1.27 G weights, 357.6 MB packed), drawn and packed on the
    device.  The GEMV is checked on sampled rows (first and last rows and tile
    edges included), the embedding on ids 0, V - 1 and one drawn id."""
    V, K = synth.VOCAB, 5120
    announce(f"maximum size: lm_head GEMV N={V} K={K} and embedding rows")
    T = torch()
    dev = T.device("cuda")
    t, sc, x = synth.device_module_draw(4242, V, K, 1, dev)
    codes, s, b = tb.tb_pack_device(t, sc)
    sig = synth.sweep_signs()[K]
    sd = signs_to_device(sig)
    y = tb.tb_ternary_gemv(x, sd, 1024, codes, s, b)
    rng = np.random.default_rng(4242)
    ids = np.array([0, V - 1, int(rng.integers(0, V))], np.int32)
    out = tb.tb_embed_inverse(T.from_numpy(ids).to(dev), codes, s, b, sd, 1024)
    T.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 15, 16, V // 2, V - 17, V - 16, V - 1],
                                     rng.integers(0, V, 1000)]))
    rt = T.from_numpy(rows).to(dev)
    oc, osc, ob = oracle.pack(t[rt].cpu().numpy(), sc[rt].cpu().numpy())
    want = oracle.packed_linear(x.float().cpu().numpy().astype(np.float64), sig, 1024, oc, osc, ob)
    compare(y[:, rt].cpu().numpy(), want, "lm_head sampled rows")
    it = T.from_numpy(ids.astype(np.int64)).to(dev)
    ec, es, eb = oracle.pack(t[it].cpu().numpy(), sc[it].cpu().numpy())
    compare(out.cpu().numpy(), oracle.embed_inverse(np.arange(3), ec, es, eb, sig, 1024), "embedding edge ids")


def test_gemv_one_call_graph_replays_match_eager():
    """The single-launch call captured in a HIP graph: every replay, with
    eager work in between, equals the eager result bitwise."""
    announce("gemv one-call graph replay")
    T = torch()
    p = synth.make_problem("graph1", 6144, 5120, 1, 43, "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    ws = T.empty(tb.tb_ternary_gemv_workspace_size(1, 5120), dtype=T.uint8, device="cuda")
    eager = tb.tb_ternary_gemv(x, sg, 1024, codes, s, b, workspace=ws)
    T.cuda.synchronize()
    y = T.empty_like(eager)
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        tb.tb_ternary_gemv(x, sg, 1024, codes, s, b, out=y, workspace=ws)
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        T.cuda.synchronize()
        assert T.equal(y, eager), i
        tb.tb_ternary_gemv_run(tb.tb_ternary_gemv_prepare(x, sg, 1024), 1, 5120, codes, s, b)
        T.cuda.synchronize()


def test_gemv_batch_graph_replays_match_eager():
    """Decode batch on the down_proj shape (K split over several workgroups,
    partial rows in the workspace, slice sums in a second launch), captured in
    a HIP graph: every replay, with eager work in between, equals the eager
    result bitwise."""
    announce("gemv batch graph replay")
    T = torch()
    p = synth.make_problem("graphb", 5120, 17408, 4, 47, "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    ws = T.empty(tb.tb_ternary_gemv_workspace_size_n(4, 17408, 5120), dtype=T.uint8, device="cuda")
    eager = tb.tb_ternary_gemv(x, sg, 1024, codes, s, b, workspace=ws)
    T.cuda.synchronize()
    oc, osc, ob = oracle_pack(p)
    compare(eager.cpu().numpy(), oracle.packed_linear(p.x64, p.signs, 1024, oc, osc, ob), "batch eager")
    y = T.empty_like(eager)
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        tb.tb_ternary_gemv(x, sg, 1024, codes, s, b, out=y, workspace=ws)
    for i in range(4):
        y.fill_(float("nan"))
        g.replay()
        T.cuda.synchronize()
        assert T.equal(y, eager), i
        tb.tb_ternary_gemv(x[:2].contiguous(), sg, 1024, codes, s, b)  # eager work between replays
        T.cuda.synchronize()


def test_gemv_batch_with_small_workspace_takes_another_path():
    """A workspace sized for the prepare/run pair only (smaller than the
    K-split partial rows) is still a valid call: tb_ternary_gemv then runs a
    path that fits it, with the same result to 1e-6 relative."""
    announce("gemv batch small workspace")
    T = torch()
    B, K, N = 4, 17408, 5120
    small = tb.tb_ternary_gemv_workspace_size(B, K)
    full = tb.tb_ternary_gemv_workspace_size_n(B, K, N)
    assert full > small
    p = synth.make_problem("smallws", N, K, B, 48, "bf16", 1024)
    codes, s, b = pack_to_device(p.t, p.scales)
    x = x_to_device(p)
    sg = signs_to_device(p.signs)
    y_small = tb.tb_ternary_gemv(x, sg, 1024, codes, s, b,
                                 workspace=T.empty(small, dtype=T.uint8, device="cuda"))
    y_full = tb.tb_ternary_gemv(x, sg, 1024, codes, s, b,
                                workspace=T.empty(full, dtype=T.uint8, device="cuda"))
    T.cuda.synchronize()
    oc, osc, ob = oracle_pack(p)
    compare(y_small.cpu().numpy(), oracle.packed_linear(p.x64, p.signs, 1024, oc, osc, ob), "small workspace")
    d = (y_small.double() - y_full.double()).abs().max().item()
    assert d <= 1e-6 * y_full.abs().max().item(), d


# --------------------------------------------------------------------------
# scale / bias views at a 4-byte (not 16-byte) offset
# --------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,B", [(6144, 5120, 1), (5120, 17408, 1), (700, 5120, 4), (300, 1152, 3)])
def test_gemv_scales_biases_at_dword_offset(N, K, B):
    """Scales and biases that start 4 bytes into their buffers (dword- but not
    16-byte aligned) give the same result as aligned ones on every GEMV path
    (band, fused, batch, prepare/run)."""
    announce(f"gemv scales/biases at +4 bytes N={N} K={K} B={B}")
    T = torch()
    p = synth.make_problem("offset_sb", N, K, B, [N, K, B, 77], "bf16", 1024 if K % 1024 == 0 else 0)
    codes, s, b = pack_to_device(p.t, p.scales)
    x, sg = x_to_device(p), signs_to_device(p.signs)

    def shifted(t):
        buf = T.empty(t.numel() + 2, dtype=t.dtype, device="cuda")
        v = buf[2:].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 16 == 4
        return v

    s4, b4 = shifted(s), shifted(b)
    y_al = tb.tb_ternary_gemv(x, sg, p.block, codes, s, b)
    y_off = tb.tb_ternary_gemv(x, sg, p.block, codes, s4, b4)
    T.cuda.synchronize()
    d = (y_al.double() - y_off.double()).abs().max().item()
    assert d <= 1e-6 * y_al.abs().max().item(), d
    oc, osc, ob = oracle_pack(p)
    compare(y_off.cpu().numpy(), oracle.packed_linear(p.x64, p.signs, p.block, oc, osc, ob), "offset views")


# --------------------------------------------------------------------------
# other contract block sizes on the embedding path; calls past 65535 rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("block", [512, 2048, 4096])
def test_embed_inverse_other_blocks(block):
    announce(f"embed V=300 K=8192 block={block}")
    T = torch()
    V, K = 300, 8192
    rng = np.random.default_rng(100 + block)
    t = synth.draw_ternary(rng, V, K)
    sc = synth.draw_scales(rng, V, K)
    sig = synth.draw_signs(rng, K)
    codes, s, b = pack_to_device(t, sc)
    ids = np.array([0, V - 1, 5, 5, -3, V, 150], np.int32)
    out = tb.tb_embed_inverse(T.from_numpy(ids).cuda(), codes, s, b, signs_to_device(sig), block)
    T.cuda.synchronize()
    oc, osc, ob = oracle.pack(t, sc)
    want = oracle.embed_inverse(ids, oc, osc, ob, sig, block)
    got = out.cpu().numpy()
    ok = (ids >= 0) & (ids < V)
    assert np.isnan(got[~ok]).all()
    compare(got[ok], want[ok], f"embed block {block}")


def test_fold_and_embed_past_65535_rows():
    """The transform and the embedding put rows in the grid's y dimension
    (65535 at most per launch); a call of 70,000 rows is launched in chunks.
    Rows on both sides of each chunk boundary, the last row, and drawn rows
    against the oracle."""
    announce("fwht 70000 x 1024 (fold) and embed of 70000 ids")
    T = torch()
    R, K = 70000, 1024
    rng = np.random.default_rng(65536)
    sig = synth.draw_signs(rng, K)
    sd = signs_to_device(sig)
    g = T.Generator(device="cuda")
    g.manual_seed(65536)
    W = T.randn((R, K), generator=g, device="cuda")
    Ws = tb.tb_fwht_signed(W, sd, 1024)
    T.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 65534, 65535, 65536, R - 1], rng.integers(0, R, 58)]))
    rt = T.from_numpy(rows).cuda()
    compare(Ws[rt].cpu().numpy(), oracle.fold_rotation(W[rt].cpu().numpy(), sig, 1024), "fold 70000 rows")
    V = 2000
    t = synth.draw_ternary(rng, V, 2048)
    sc = synth.draw_scales(rng, V, 2048)
    sig2 = synth.draw_signs(rng, 2048)
    codes, s, b = pack_to_device(t, sc)
    ids = rng.integers(0, V, R).astype(np.int32)
    ids[65535] = V - 1
    ids[R - 1] = 0
    out = tb.tb_embed_inverse(T.from_numpy(ids).cuda(), codes, s, b, signs_to_device(sig2), 2048)
    T.cuda.synchronize()
    oc, osc, ob = oracle.pack(t, sc)
    want = oracle.embed_inverse(ids[rows], oc, osc, ob, sig2, 2048)
    compare(out[rt].cpu().numpy(), want, "embed 70000 ids")
