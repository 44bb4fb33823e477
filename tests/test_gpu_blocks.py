"""GPU parity of the batch-1 Packed linear on the PQ2_0 and PTQ1_0 block
containers against the fp64 oracle (the blocks the library's host packers
write are first checked equal to the oracle's, byte for byte), under the
bar relative L2 <= 1e-4 and max |err| <= 1e-3 max |y|."""
import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb
import oracle
from hadamard_rotated_quantized_amd import synth
from gpu_util import announce, compare, cuda_available, signs_to_device, torch, x_to_device

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_available(), reason="needs a GPU")]

SHAPES = [
    # (N, K, block, x dtype, seed)
    (256, 1024, 1024, "f32", 0),        # the tiny workload's shape
    (6144, 5120, 1024, "bf16", 2),      # q_proj
    (5120, 17408, 1024, "bf16", 3),     # down_proj (17 chunks)
    (1000, 1280, 0, "bf16", 5),         # G = 10: half-filled last span, ragged last tile, no rotation
    (77, 1536, 512, "f32", 6),          # 512-blocks, 3 chunks
    (17, 6144, 1024, "bf16", 7),        # one partial tile
    (40000, 2048, 1024, "bf16", 8),     # several tiles per wave
    (300, 26624, 1024, "bf16", 9),      # 26 chunks: two past the 24 a workgroup loads up front
    (4352, 1280, 0, "bf16", 10),        # 17-row bands: band starts off 16-byte boundaries (both formats)
    (4352, 2560, 512, "f32", 11),       # 17-row bands, 512-blocks, 3 chunks
]


def _blocks(fmt, p):
    if fmt == "pq2":
        c, s, b = tb.tb_pack(p.t, p.scales)
        blk = tb.tb_pq2_from_mlx(c, s, b)
        assert np.array_equal(blk, oracle.pq2_from_mlx(*oracle.pack(p.t, p.scales)))
        return blk
    blk = tb.tb_ptq1_pack(p.t, p.scales)
    assert np.array_equal(blk, oracle.ptq1_pack(p.t, p.scales))
    return blk


@pytest.mark.parametrize("fmt", ["pq2", "ptq1"])
@pytest.mark.parametrize("N,K,block,xd,seed", SHAPES)
def test_blocks_gemv_matches_oracle(fmt, N, K, block, xd, seed):
    announce(f"{fmt} gemv N={N} K={K} block={block} x={xd}")
    T = torch()
    p = synth.make_problem(fmt, N, K, 1, [seed, N, K], xd, block)
    blk = _blocks(fmt, p)
    bd = T.from_numpy(blk).cuda()
    fn = tb.tb_pq2_gemv if fmt == "pq2" else tb.tb_ptq1_gemv
    y = fn(x_to_device(p), signs_to_device(p.signs), block, bd)
    y2 = fn(x_to_device(p), signs_to_device(p.signs), block, bd)
    T.cuda.synchronize()
    assert T.equal(y, y2)
    want = (oracle.pq2_packed_linear if fmt == "pq2" else oracle.ptq1_packed_linear)(p.x64, p.signs, block, blk, K)
    compare(y.cpu().numpy(), want, f"{fmt} N={N} K={K}")


def test_blocks_equal_the_mlx_container_on_the_same_weights():
    """The three containers of one set of ternary weights give one result:
    PQ2_0 and PTQ1_0 against the MLX path within 1e-6 of max |y|."""
    announce("pq2 / ptq1 / mlx agreement")
    T = torch()
    p = synth.config_problem("q_proj")
    c, s, b = tb.tb_pack(p.t, p.scales)
    x, sg = x_to_device(p), signs_to_device(p.signs)
    y_mlx = tb.tb_ternary_gemv(x, sg, 1024, T.from_numpy(c.view(np.int32)).cuda(), T.from_numpy(s).cuda(),
                               T.from_numpy(b).cuda())
    y_pq2 = tb.tb_pq2_gemv(x, sg, 1024, T.from_numpy(tb.tb_pq2_from_mlx(c, s, b)).cuda())
    y_ptq = tb.tb_ptq1_gemv(x, sg, 1024, T.from_numpy(tb.tb_ptq1_pack(p.t, p.scales)).cuda())
    T.cuda.synchronize()
    m = y_mlx.abs().max().item()
    assert (y_pq2 - y_mlx).abs().max().item() <= 1e-6 * m
    assert (y_ptq - y_mlx).abs().max().item() <= 1e-6 * m


def test_pq2_lm_head_sized_sampled_rows():
    """The largest module (lm_head, 248,320 x 5120) as PQ2_0: drawn and packed
    on the device, transcoded on the host, every 16-row tile edge of the
    first and last rows and 2000 drawn rows against the oracle."""
    announce("pq2 lm_head N=248320 K=5120 (sampled rows)")
    T = torch()
    N, K = synth.VOCAB, 5120
    t, sc, x = synth.device_module_draw(400, N, K, 1, "cuda")
    c, s, b = tb.tb_pack_device(t, sc)
    blk = tb.tb_pq2_from_mlx(c.cpu().numpy().view(np.uint32), s.cpu().numpy(), b.cpu().numpy())
    sig = synth.sweep_signs()[K]
    y = tb.tb_pq2_gemv(x, signs_to_device(sig), 1024, T.from_numpy(blk).cuda())
    T.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 15, 16, N - 17, N - 16, N - 1],
                                     np.random.default_rng(400).integers(0, N, 2000)]))
    rt = T.from_numpy(rows).cuda()
    ob = oracle.pq2_from_mlx(*oracle.pack(t[rt].cpu().numpy(), sc[rt].cpu().numpy()))
    assert np.array_equal(ob, blk[rows])
    want = oracle.pq2_packed_linear(x.float().cpu().numpy().astype(np.float64), sig, 1024, ob, K)
    compare(y[:, rt].cpu().numpy(), want, "pq2 lm_head rows")


@pytest.mark.parametrize("fmt", ["pq2", "ptq1"])
def test_blocks_off_16_byte_alignment_take_the_ring_path(fmt):
    """A block array 4 bytes past a 16-byte boundary (allowed: the entry
    points take 4-byte aligned blocks) cannot be staged by 16-byte
    direct-to-LDS loads; the call takes the register-ring kernel and gives
    the aligned array's result bit for bit."""
    announce(f"{fmt} gemv on a block array 4 bytes off a 16-byte boundary")
    T = torch()
    N, K, block = 6144, 5120, 1024
    p = synth.make_problem(fmt, N, K, 1, [12, N, K], "bf16", block)
    blk = _blocks(fmt, p)
    bd = T.from_numpy(blk).cuda()
    raw = T.zeros(blk.size + 16, dtype=T.uint8, device="cuda")
    off = raw[4:4 + blk.size].view(blk.shape)
    off.copy_(bd)
    assert off.data_ptr() % 16 == 4
    fn = tb.tb_pq2_gemv if fmt == "pq2" else tb.tb_ptq1_gemv
    x, sg = x_to_device(p), signs_to_device(p.signs)
    y_al = fn(x, sg, block, bd)
    y_off = fn(x, sg, block, off)
    T.cuda.synchronize()
    want = (oracle.pq2_packed_linear if fmt == "pq2" else oracle.ptq1_packed_linear)(p.x64, p.signs, block, blk, K)
    compare(y_off.cpu().numpy(), want, f"{fmt} offset blocks")
    compare(y_al.cpu().numpy(), want, f"{fmt} aligned blocks")
