"""Host logic of the multi-module decode plan (no GPU): argument checks, and
that the per-workgroup tile ranges partition the concatenated tile list with
about equal weight bytes per workgroup.  The plan layout parsed here is the
one tb_gemv_multi.hip writes: a 64-byte header (int32 magic, count, tasks,
grid, block, x_dtype, max_nch, ring; int64 modules_off, tasks_off,
ranges_off, total_bytes), 64 bytes per module, int32 pairs (module, chunk)
per transform task, and int32 quadruples (first module, first tile, end
tile, 0) per workgroup."""
import ctypes

import numpy as np
import pytest

import hadamard_rotated_quantized_amd as tb

FAKE = 1 << 20  # non-null, aligned fake device addresses (the plan never dereferences them)


def _mods(shapes, block=1024):
    arr = (tb.TbGemvModule * len(shapes))()
    for i, (N, K) in enumerate(shapes):
        base = FAKE * (8 * i + 1)
        arr[i] = tb.TbGemvModule(base, base + FAKE if block else None, base + 2 * FAKE, base + 3 * FAKE,
                                 base + 4 * FAKE, base + 5 * FAKE, N, K)
    return arr


def _plan(shapes, block=1024, dtype=tb.TB_BF16):
    arr = _mods(shapes, block)
    size = tb.lib().tb_gemv_multi_plan_size(arr, len(shapes))
    plan = np.zeros(max(size, 64), np.uint8)
    ws = ctypes.c_size_t(0)
    st = tb.lib().tb_gemv_multi_plan(arr, len(shapes), dtype, block, plan.ctypes.data, plan.nbytes, ctypes.byref(ws))
    return st, plan, ws.value


def _parse(plan):
    hd = plan[:32].view(np.int32)
    offs = plan[32:64].view(np.int64)
    magic, count, tasks, grid, block, xdt, max_nch, ring = [int(v) for v in hd]
    mods = plan[offs[0]:offs[0] + 64 * count].reshape(count, 64)
    NK = mods[:, 48:64].copy().view(np.int32)  # N, K, tile0, ws_off
    tk = plan[offs[1]:offs[1] + 8 * tasks].view(np.int32).reshape(tasks, 2)
    rg = plan[offs[2]:offs[2] + 16 * grid].view(np.int32).reshape(grid, 4)
    return dict(magic=magic, count=count, tasks=tasks, grid=grid, max_nch=max_nch, NK=NK, tk=tk, rg=rg)


SWEEPLIKE = [(10240, 5120), (6144, 5120), (5120, 6144), (17408, 5120), (17408, 5120), (5120, 17408),
             (6144, 5120), (1024, 5120), (1024, 5120), (5120, 6144), (0, 5120), (45, 2048), (248320, 5120)]


def test_plan_tasks_and_ranges_partition_tiles():
    st, plan, ws = _plan(SWEEPLIKE)
    assert st == tb.TB_OK, tb.lib().tb_last_error()
    p = _parse(plan)
    assert p["magic"] == 0x4D504254 and p["count"] == len(SWEEPLIKE)
    nch = [(K + 1023) // 1024 for N, K in SWEEPLIKE]
    assert p["tasks"] == sum(c for c, (N, K) in zip(nch, SWEEPLIKE) if N > 0)
    # every chunk of every non-empty module is one task, in order
    want = [(i, c) for i, (N, K) in enumerate(SWEEPLIKE) if N > 0 for c in range((K + 1023) // 1024)]
    assert [tuple(t) for t in p["tk"]] == want
    tiles = [(N + 15) // 16 for N, K in SWEEPLIKE]
    total = sum(tiles)
    tile0 = np.cumsum([0] + tiles[:-1])
    assert list(p["NK"][:, 2]) == list(tile0)
    # workspace: 4 KB of operand image (8 groups x 4 limbs x 128 B) + 64 B of group sums per chunk
    assert ws == sum((4096 + 64) * c for c, (N, K) in zip(nch, SWEEPLIKE) if N > 0)
    # ranges: contiguous, cover [0, total) once, start module owns the start tile
    rg = p["rg"]
    assert rg[0, 1] == 0
    for g in range(p["grid"] - 1):
        assert rg[g, 2] == rg[g + 1, 1]
    assert rg[-1, 2] == total
    cost_tile = np.concatenate([np.full(t, K // 128 + 2) for t, (N, K) in zip(tiles, SWEEPLIKE)])
    cum = np.concatenate([[0], np.cumsum(cost_tile)])
    share = cum[-1] / p["grid"]
    for g in range(p["grid"]):
        a, b = rg[g, 1], rg[g, 2]
        if a < b:
            m = rg[g, 0]
            assert tile0[m] <= a < tile0[m] + tiles[m]
            # no workgroup exceeds its share by more than one tile
            assert cum[b] - cum[a] <= share + cost_tile.max()


@pytest.mark.parametrize("shapes,block,status", [
    ([(16, 1000)], 1024, -2),                      # K % 256
    ([(16, 1536)], 1024, -2),                      # K % block
    ([(16, 1024)], 2048, -4),                      # block the multi path does not take
    ([(16, 1024)], 300, -3),                       # not a contract block
    ([(-1, 1024)], 1024, -1),                      # negative N
    ([(16, 64 * 1024)], 1024, -4),                 # operand image beyond the LDS budget
])
def test_plan_rejects(shapes, block, status):
    st, _, _ = _plan(shapes, block)
    assert st == status, tb.lib().tb_last_error()


def test_plan_rejects_misaligned_and_null():
    arr = _mods([(16, 1024)])
    arr[0].codes = FAKE * 3 + 4
    size = tb.lib().tb_gemv_multi_plan_size(arr, 1)
    plan = np.zeros(size, np.uint8)
    ws = ctypes.c_size_t(0)
    assert tb.lib().tb_gemv_multi_plan(arr, 1, tb.TB_BF16, 1024, plan.ctypes.data, plan.nbytes,
                                       ctypes.byref(ws)) == -8
    arr = _mods([(16, 1024)])
    arr[0].signs = None  # block > 0 needs signs
    assert tb.lib().tb_gemv_multi_plan(arr, 1, tb.TB_BF16, 1024, plan.ctypes.data, plan.nbytes,
                                       ctypes.byref(ws)) == -1
    # too small a plan buffer
    arr = _mods([(16, 1024)])
    assert tb.lib().tb_gemv_multi_plan(arr, 1, tb.TB_BF16, 1024, plan.ctypes.data, 64, ctypes.byref(ws)) == -10


def test_run_refuses_foreign_plan():
    junk = np.zeros(256, np.uint8)
    st = tb.lib().tb_ternary_gemv_multi(junk.ctypes.data, FAKE, FAKE, 1 << 20, None)
    assert st == -1
