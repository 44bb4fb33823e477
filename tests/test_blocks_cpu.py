"""Host side of the PQ2_0 / PTQ1_0 block containers through the C ABI: the
library's transcode and packers equal the oracle's bit for bit, round trip
losslessly (group scales bit-compared), reject what the blocks cannot hold,
and the device entry points refuse bad arguments on the host before any
launch (aligned dummy pointers that are never read)."""
import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb
import oracle
from hadamard_rotated_quantized_amd import synth

DUMMY = 0x10000


def _mlx(seed, N, K):
    rng = np.random.default_rng(seed)
    t = synth.draw_ternary(rng, N, K)
    sc = synth.draw_scales(rng, N, K)
    return t, sc, oracle.pack(t, sc)


@pytest.mark.parametrize("N,K", [(1, 128), (7, 1024), (33, 5120), (3, 17408)])
def test_pq2_transcode_matches_oracle_and_round_trips(N, K):
    t, sc, (c, s, b) = _mlx(N * 7 + K, N, K)
    pq = tb.tb_pq2_from_mlx(c, s, b)
    assert np.array_equal(pq, oracle.pq2_from_mlx(c, s, b))
    assert pq.nbytes == oracle.container_bytes_pq2(N, K) == N * K * 34 // 128
    c2, s2, b2 = tb.tb_pq2_to_mlx(pq, K)
    assert np.array_equal(c2, c)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))   # group scales, bit for bit
    assert np.array_equal(b2.view(np.uint16), b.view(np.uint16))
    # the independent unpack of the transcoded blocks gives the ternary weights back
    assert np.array_equal(oracle.pq2_codes(pq, K).astype(np.int8) - 1, t)


def test_pq2_transcode_rejects_what_pq2_cannot_hold():
    t, sc, (c, s, b) = _mlx(1, 4, 256)
    b2 = b.copy()
    b2[2, 1] = np.float16(0.125)
    with pytest.raises(tb.TBError) as e:
        tb.tb_pq2_from_mlx(c, s, b2)
    assert e.value.status == -6
    c3 = c.copy()
    c3[1, 5] |= np.uint32(0xC0000000)
    with pytest.raises(tb.TBError):
        tb.tb_pq2_from_mlx(c3, s, b)
    pq = tb.tb_pq2_from_mlx(c, s, b)
    pq[0, 40] = 0xFF
    with pytest.raises(tb.TBError):
        tb.tb_pq2_to_mlx(pq, 256)


@pytest.mark.parametrize("N,K", [(1, 128), (7, 1024), (33, 5120), (3, 17408)])
def test_ptq1_pack_matches_oracle_and_round_trips(N, K):
    t, sc, _ = _mlx(N * 11 + K, N, K)
    pt = tb.tb_ptq1_pack(t, sc)
    assert np.array_equal(pt, oracle.ptq1_pack(t, sc))
    assert pt.nbytes == oracle.container_bytes_ptq1(N, K) == N * K * 28 // 128
    t2, s2 = tb.tb_ptq1_unpack(pt, K)
    assert np.array_equal(t2, t)
    assert np.array_equal(s2.view(np.uint16), sc.view(np.uint16))


def test_ptq1_rejects_invalid_values_and_bytes():
    t, sc, _ = _mlx(2, 3, 256)
    bad_t = t.copy()
    bad_t[1, 7] = 2
    with pytest.raises(tb.TBError):
        tb.tb_ptq1_pack(bad_t, sc)
    pt = tb.tb_ptq1_pack(t, sc)
    for pos, val in ((2 + 3, 243), (28 + 27, 27), (27, 200)):
        bad = pt.copy()
        bad[0, pos] = val
        with pytest.raises(tb.TBError):
            tb.tb_ptq1_unpack(bad, 256)


@pytest.mark.parametrize("fn", ["tb_pq2_gemv", "tb_ptq1_gemv"])
@pytest.mark.parametrize("kw,status", [
    (dict(B=2), -4),            # batch 1 only
    (dict(block=2048, K=4096), -4),
    (dict(block=300), -3),
    (dict(K=1536 + 128), -2),   # not a multiple of 128 x 2 (256)
    (dict(K=384, block=0, signs=None), -2),
    (dict(K=34816, block=1024), -4),   # operand image beyond the kernel's LDS
    (dict(blocks=DUMMY + 2), -8),
    (dict(x=DUMMY + 4), -8),
    (dict(dt=9), -7),
    (dict(blocks=None), -1),
])
def test_blocks_gemv_rejects(fn, kw, status):
    a = dict(x=DUMMY, dt=tb.TB_BF16, B=1, K=1024, signs=DUMMY, block=1024, blocks=DUMMY, N=32, y=DUMMY)
    a.update(kw)
    f = getattr(tb.lib(), fn)
    assert f(a["x"], a["dt"], a["B"], a["K"], a["signs"], a["block"], a["blocks"], a["N"], a["y"], None) == status
    assert f(DUMMY, tb.TB_BF16, 0, 1024, DUMMY, 1024, None, 32, None, None) == 0  # B = 0: no-op
