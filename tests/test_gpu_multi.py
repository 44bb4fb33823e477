"""Parity of the multi-module decode path (tb_gemv_multi_plan +
tb_ternary_gemv_multi) with the fp64 oracle, module by module, on the GPU."""
import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb
import oracle
from hadamard_rotated_quantized_amd import synth
from gpu_util import announce, compare, cuda_available, pack_to_device, signs_to_device, torch, x_to_device

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]


def _run_multi(shapes, block, xd, seed):
    T = torch()
    probs, mods, keep = [], [], []
    for i, (N, K) in enumerate(shapes):
        p = synth.make_problem("multi", N, K, 1, [seed, i, N, K], xd, block)
        codes, s, b = pack_to_device(p.t, p.scales)
        x = x_to_device(p)
        sg = signs_to_device(p.signs)
        y = T.full((1, N), float("nan"), dtype=T.float32, device="cuda")
        mods.append((x, sg, codes, s, b, y))
        probs.append(p)
    plan, wsb = tb.tb_gemv_multi_plan(mods, block, tb.TB_F32 if xd == "f32" else tb.TB_BF16)
    pd = T.from_numpy(plan).cuda()
    ws = T.empty(wsb, dtype=T.uint8, device="cuda")
    tb.tb_ternary_gemv_multi(plan, pd, ws)
    T.cuda.synchronize()
    return probs, mods, plan, pd, ws


CASES = [
    ("bf16", 1024, [(1, 1024), (45, 2048), (300, 5120), (1000, 6144), (16, 17408), (0, 1024), (4099, 1024),
                    (31, 3072)]),
    ("f32", 512, [(17, 1024), (33, 1536), (200, 512)]),
    ("bf16", 0, [(45, 256), (300, 768), (16, 1024)]),
]


@pytest.mark.parametrize("xd,block,shapes", CASES)
def test_multi_matches_oracle(xd, block, shapes):
    announce(f"multi x={xd} block={block} shapes={shapes}")
    probs, mods, *_ = _run_multi(shapes, block, xd, 70)
    for p, m in zip(probs, mods):
        if p.N == 0:
            continue
        oc, osc, ob = oracle.pack(p.t, p.scales)
        want = oracle.packed_linear(p.x64, p.signs, block, oc, osc, ob)
        compare(m[5].cpu().numpy(), want, f"multi module N={p.N} K={p.K}")


def test_multi_rerun_is_bitwise_stable_and_matches_single_calls():
    announce("multi rerun + single-call agreement")
    T = torch()
    shapes = [(300, 5120), (1024, 5120), (77, 6144), (513, 17408)]
    probs, mods, plan, pd, ws = _run_multi(shapes, 1024, "bf16", 71)
    first = [m[5].clone() for m in mods]
    for m in mods:
        m[5].fill_(float("nan"))
    tb.tb_ternary_gemv_multi(plan, pd, ws)
    T.cuda.synchronize()
    for f, m in zip(first, mods):
        assert T.equal(f, m[5])
    for p, m in zip(probs, mods):
        x, sg, codes, s, b, y = m
        y1 = tb.tb_ternary_gemv(x, sg, 1024, codes, s, b)
        T.cuda.synchronize()
        d = (y1.double() - y.double()).abs().max().item()
        assert d <= 1e-6 * y1.abs().max().item(), (p.N, p.K, d)


def test_multi_graph_replays_match_eager():
    announce("multi graph replay")
    T = torch()
    shapes = [(600, 5120), (100, 17408)]
    probs, mods, plan, pd, ws = _run_multi(shapes, 1024, "bf16", 72)
    eager = [m[5].clone() for m in mods]
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        tb.tb_ternary_gemv_multi(plan, pd, ws)
    for r in range(3):
        for m in mods:
            m[5].zero_()
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        for e, m in zip(eager, mods):
            assert T.equal(e, m[5]), r


def test_multi_shared_inputs_match_oracle_and_single_calls():
    """Modules that read one activation (same x tensor and signs) share one
    transform and one operand image; interleaved with modules that read
    others, every module must still match the oracle and its single call."""
    announce("multi shared inputs")
    T = torch()
    rng = np.random.default_rng(73)
    inputs = {}
    for key, K in (("a", 5120), ("b", 17408), ("c", 5120)):
        x64, xs = synth.draw_activations(rng, 1, K, "bf16")
        sig = synth.draw_signs(rng, K)
        inputs[key] = (x64, T.from_numpy(xs.view(np.int16)).view(T.bfloat16).cuda(), sig, signs_to_device(sig))
    plan_spec = [("a", 300), ("a", 1024), ("b", 513), ("a", 77), ("c", 640), ("b", 100), ("c", 16)]
    mods, want = [], []
    for j, (key, N) in enumerate(plan_spec):
        x64, x, sig, sg = inputs[key]
        K = x.shape[-1]
        t = synth.draw_ternary(rng, N, K)
        sc = synth.draw_scales(rng, N, K)
        codes, s, b = pack_to_device(t, sc)
        y = T.full((1, N), float("nan"), dtype=T.float32, device="cuda")
        mods.append((x, sg, codes, s, b, y))
        oc, osc, ob = oracle.pack(t, sc)
        want.append(oracle.packed_linear(x64, sig, 1024, oc, osc, ob))
    plan, wsb = tb.tb_gemv_multi_plan(mods, 1024)
    assert int(plan[:32].view(np.int32)[2]) == 5 + 17 + 5   # one transform per distinct input
    pd = T.from_numpy(plan).cuda()
    ws = T.empty(wsb, dtype=T.uint8, device="cuda")
    tb.tb_ternary_gemv_multi(plan, pd, ws)
    T.cuda.synchronize()
    for (key, N), m, w in zip(plan_spec, mods, want):
        compare(m[5].cpu().numpy(), w, f"shared input {key} N={N}")
        y1 = tb.tb_ternary_gemv(m[0], m[1], 1024, m[2], m[3], m[4])
        T.cuda.synchronize()
        d = (y1.double() - m[5].double()).abs().max().item()
        assert d <= 1e-6 * y1.abs().max().item(), (key, N, d)


def _run_multi_blocks(shapes, block, xd, seed, fmt="pq2"):
    """PQ2_0 or PTQ1_0 modules (host packers, checked against the oracle's
    blocks byte for byte) in one plan, run once."""
    T = torch()
    probs, mods, blks = [], [], []
    for i, (N, K) in enumerate(shapes):
        p = synth.make_problem("multi", N, K, 1, [seed, i, N, K], xd, block)
        if fmt == "pq2":
            c, s, b = tb.tb_pack(p.t, p.scales)
            blk = tb.tb_pq2_from_mlx(c, s, b)
            assert np.array_equal(blk, oracle.pq2_from_mlx(*oracle.pack(p.t, p.scales)))
        else:
            blk = tb.tb_ptq1_pack(p.t, p.scales)
            assert np.array_equal(blk, oracle.ptq1_pack(p.t, p.scales))
        y = T.full((1, N), float("nan"), dtype=T.float32, device="cuda")
        mods.append((x_to_device(p), signs_to_device(p.signs), T.from_numpy(blk).cuda(), y))
        probs.append(p)
        blks.append(blk)
    planner = tb.tb_pq2_gemv_multi_plan if fmt == "pq2" else tb.tb_ptq1_gemv_multi_plan
    plan, wsb = planner(mods, block, tb.TB_F32 if xd == "f32" else tb.TB_BF16)
    pd = T.from_numpy(plan).cuda()
    ws = T.empty(wsb, dtype=T.uint8, device="cuda")
    tb.tb_ternary_gemv_multi(plan, pd, ws)
    T.cuda.synchronize()
    return probs, mods, blks, plan, pd, ws


BLOCK_CASES = [
    ("bf16", 1024, [(1, 1024), (45, 2048), (300, 5120), (1000, 6144), (16, 17408), (0, 1024), (4099, 1024)]),
    ("f32", 512, [(17, 1024), (33, 1536), (200, 512)]),
    ("bf16", 0, [(45, 256), (300, 768), (16, 1024)]),
]


@pytest.mark.parametrize("fmt", ["pq2", "ptq1"])
@pytest.mark.parametrize("xd,block,shapes", BLOCK_CASES)
def test_block_multi_matches_oracle(fmt, xd, block, shapes):
    announce(f"{fmt} multi x={xd} block={block} shapes={shapes}")
    probs, mods, blks, *_ = _run_multi_blocks(shapes, block, xd, 80, fmt)
    ref = oracle.pq2_packed_linear if fmt == "pq2" else oracle.ptq1_packed_linear
    for p, m, blk in zip(probs, mods, blks):
        if p.N == 0:
            continue
        want = ref(p.x64, p.signs, block, blk, p.K)
        compare(m[3].cpu().numpy(), want, f"{fmt} multi module N={p.N} K={p.K}")


@pytest.mark.parametrize("fmt", ["pq2", "ptq1"])
def test_block_multi_rerun_is_bitwise_stable_and_matches_single_calls(fmt):
    """Rerunning a PQ2_0 / PTQ1_0 plan gives the same bits; each module
    agrees with its single tb_pq2_gemv / tb_ptq1_gemv call within 1e-6 of
    max |y|."""
    announce(f"{fmt} multi rerun + single-call agreement")
    T = torch()
    shapes = [(300, 5120), (1024, 5120), (77, 6144), (513, 17408)]
    probs, mods, blks, plan, pd, ws = _run_multi_blocks(shapes, 1024, "bf16", 81, fmt)
    first = [m[3].clone() for m in mods]
    for m in mods:
        m[3].fill_(float("nan"))
    tb.tb_ternary_gemv_multi(plan, pd, ws)
    T.cuda.synchronize()
    for f, m in zip(first, mods):
        assert T.equal(f, m[3])
    for p, m in zip(probs, mods):
        x, sg, bd, y = m
        y1 = (tb.tb_pq2_gemv if fmt == "pq2" else tb.tb_ptq1_gemv)(x, sg, 1024, bd)
        T.cuda.synchronize()
        d = (y1.double() - y.double()).abs().max().item()
        assert d <= 1e-6 * y1.abs().max().item(), (p.N, p.K, d)


@pytest.mark.parametrize("fmt", ["pq2", "ptq1"])
def test_block_multi_graph_replays_match_eager(fmt):
    """A PQ2_0 / PTQ1_0 plan captured in a HIP graph: every replay (with the
    outputs cleared between them) gives the eager run's bits."""
    announce(f"{fmt} multi graph replay")
    T = torch()
    shapes = [(600, 5120), (100, 17408)]
    probs, mods, blks, plan, pd, ws = _run_multi_blocks(shapes, 1024, "bf16", 82, fmt)
    eager = [m[3].clone() for m in mods]
    g = T.cuda.CUDAGraph()
    with T.cuda.graph(g):
        tb.tb_ternary_gemv_multi(plan, pd, ws)
    for r in range(3):
        for m in mods:
            m[3].zero_()
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        for e, m in zip(eager, mods):
            assert T.equal(e, m[3]), r
