"""Host logic of the multi-module decode plan (no GPU): argument checks, and
that the pieces partition the concatenated tile list, each within one
module, shrinking toward the end.  The plan layout parsed here is the one
tb_gemv_multi.hip writes: a 64-byte header (int32 magic, count, tasks, grid,
block, x_dtype, max_nch, pieces; int64 modules_off, tasks_off, pieces_off;
int32 total_bytes, format), 64 bytes per module, int32 pairs (module, chunk) per transform
task, and int32 quadruples (module, first tile, end tile, 0) per piece."""
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
    magic, count, tasks, grid, block, xdt, max_nch, npieces = [int(v) for v in hd]
    mods = plan[offs[0]:offs[0] + 64 * count].reshape(count, 64)
    NK = mods[:, 48:64].copy().view(np.int32)  # N, K, tile0, ws_off
    tk = plan[offs[1]:offs[1] + 8 * tasks].view(np.int32).reshape(tasks, 2)
    pc = plan[offs[2]:offs[2] + 16 * npieces].view(np.int32).reshape(npieces, 4)
    return dict(magic=magic, count=count, tasks=tasks, grid=grid, max_nch=max_nch, NK=NK, tk=tk, pc=pc)


SWEEPLIKE = [(10240, 5120), (6144, 5120), (5120, 6144), (17408, 5120), (17408, 5120), (5120, 17408),
             (6144, 5120), (1024, 5120), (1024, 5120), (5120, 6144), (0, 5120), (45, 2048), (248320, 5120)]


def test_plan_tasks_and_pieces_partition_tiles():
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
    # workspace: a 256-byte head (the piece counter), then per chunk 4 KB of
    # operand image (8 groups x 4 limbs x 128 B) + 64 B of group sums
    assert ws == 256 + sum((4096 + 64) * c for c, (N, K) in zip(nch, SWEEPLIKE) if N > 0)
    assert list(p["NK"][:, 3][np.array(tiles) > 0][:1]) == [256]
    # pieces: contiguous, cover [0, total) once in order, each inside its module
    pc = p["pc"]
    assert pc[0, 1] == 0 and pc[-1, 2] == total
    assert (pc[1:, 1] == pc[:-1, 2]).all() and (pc[:, 2] > pc[:, 1]).all()
    for m, a, b, _ in pc:
        assert tile0[m] <= a < b <= tile0[m] + tiles[m]
    # sizes: about 1/grid of the cost still left, never below the floor
    # (1/64 of a workgroup's mean share) unless a module ends first
    cost_tile = np.concatenate([np.full(t, K // 128 + 2) for t, (N, K) in zip(tiles, SWEEPLIKE)])
    cum = np.concatenate([[0], np.cumsum(cost_tile)])
    floor = max(1, cum[-1] // (p["grid"] * 64))
    # and a whole number of rounds of the workgroup's 8 waves (unless a
    # module ends first)
    for m, a, b, _ in pc:
        left = cum[-1] - cum[a]
        want = max(floor, left // p["grid"])
        tc = SWEEPLIKE[m][1] // 128 + 2
        ends_module = b == tile0[m] + tiles[m]
        rounds = -(-(-(-want // tc)) // 8)  # ceil(ceil(want / tc) / 8)
        assert cum[b] - cum[a] <= 8 * rounds * tc
        assert ends_module or ((b - a) % 8 == 0 and cum[b] - cum[a] >= want)
    # the first pieces are large, the last ones small
    assert (cum[pc[0, 2]] - cum[pc[0, 1]]) > 4 * (cum[pc[-2, 2]] - cum[pc[-2, 1]])


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


def _mods_shared(spec, block=1024):
    """spec: (N, K, input id) per module; modules with the same input id get
    the same fake x and sign pointers."""
    arr = (tb.TbGemvModule * len(spec))()
    for i, (N, K, inp) in enumerate(spec):
        xb = FAKE * (64 * inp + 1)
        wb = FAKE * (64 * i + 1000)
        arr[i] = tb.TbGemvModule(xb, xb + FAKE if block else None, wb, wb + FAKE, wb + 2 * FAKE, wb + 3 * FAKE, N, K)
    return arr


def _plan_arr(arr, n, block=1024):
    size = tb.lib().tb_gemv_multi_plan_size(arr, n)
    plan = np.zeros(max(size, 64), np.uint8)
    ws = ctypes.c_size_t(0)
    st = tb.lib().tb_gemv_multi_plan(arr, n, tb.TB_BF16, block, plan.ctypes.data, plan.nbytes, ctypes.byref(ws))
    assert st == tb.TB_OK, tb.lib().tb_last_error()
    return _parse(plan), ws.value


def test_modules_reading_one_input_share_transform_and_image():
    # one full-attention layer + MLP: q/k/v read input 0, o_proj input 1,
    # gate/up input 2, down_proj input 3 (as a decode layer feeds them)
    spec = [(6144, 5120, 0), (1024, 5120, 0), (1024, 5120, 0), (5120, 6144, 1),
            (17408, 5120, 2), (17408, 5120, 2), (5120, 17408, 3)]
    p, ws = _plan_arr(_mods_shared(spec), len(spec))
    # tasks: one set per distinct input (5 + 6 + 5 + 17 chunks), owned by the
    # first module that reads it
    assert p["tasks"] == 5 + 6 + 5 + 17
    assert sorted({int(m) for m in p["tk"][:, 0]}) == [0, 3, 4, 6]
    off = p["NK"][:, 3]
    assert off[0] == off[1] == off[2] and off[4] == off[5]
    assert len({off[0], off[3], off[4], off[6]}) == 4
    # the same modules with distinct inputs need one image each
    p2, ws2 = _plan_arr(_mods_shared([(N, K, i) for i, (N, K, _) in enumerate(spec)]), len(spec))
    assert p2["tasks"] == 5 + 5 + 5 + 6 + 5 + 5 + 17
    img = lambda K: (K + 1023) // 1024 * (8 * 4 * 128 + 64)
    assert ws2 - ws == 2 * img(5120) + img(5120)


def test_same_x_different_signs_or_width_is_not_shared():
    arr = _mods_shared([(256, 5120, 0), (256, 5120, 0)])
    arr[1].signs = arr[1].signs + 16 * FAKE   # same x, another sign vector
    p, _ = _plan_arr(arr, 2)
    assert p["tasks"] == 10 and p["NK"][0, 3] != p["NK"][1, 3]
    arr = _mods_shared([(256, 5120, 0), (256, 4096, 0)])  # same pointers, another width
    p, _ = _plan_arr(arr, 2)
    assert p["tasks"] == 9 and p["NK"][0, 3] != p["NK"][1, 3]


@pytest.mark.parametrize("fmt,word", [("pq2", 1), ("ptq1", 2)])
def test_block_plan_format_and_checks(fmt, word):
    """PQ2_0 / PTQ1_0 plans: the header's format word is 1 / 2 (0 for the
    MLX container), the pieces and tasks are those of the same shapes in the
    MLX container, scales or biases given are refused, and the blocks need
    4-byte (not 16-byte) alignment."""
    shapes = [(10240, 5120), (1024, 5120), (5120, 17408), (45, 2048)]
    fn = tb.lib().tb_pq2_gemv_multi_plan if fmt == "pq2" else tb.lib().tb_ptq1_gemv_multi_plan

    def pq2_plan(arr):
        size = tb.lib().tb_gemv_multi_plan_size(arr, len(shapes))
        plan = np.zeros(max(size, 64), np.uint8)
        ws = ctypes.c_size_t(0)
        st = fn(arr, len(shapes), tb.TB_BF16, 1024, plan.ctypes.data, plan.nbytes, ctypes.byref(ws))
        return st, plan, ws.value

    arr = _mods(shapes)
    for m in arr:
        m.scales = None
        m.biases = None
        m.codes += 4  # 4-byte aligned blocks are accepted
    st, plan, ws = pq2_plan(arr)
    assert st == tb.TB_OK, tb.lib().tb_last_error()
    st0, plan0, ws0 = _plan(shapes)
    assert st0 == tb.TB_OK
    assert int(plan[60:64].view(np.int32)[0]) == word and int(plan0[60:64].view(np.int32)[0]) == 0
    p, p0 = _parse(plan), _parse(plan0)
    assert ws == ws0 and np.array_equal(p["pc"], p0["pc"]) and np.array_equal(p["tk"], p0["tk"])
    # scales given: refused
    arr = _mods(shapes)
    for m in arr:
        m.biases = None
    assert pq2_plan(arr)[0] == -1
    # blocks 2 bytes off a dword: refused
    arr = _mods(shapes)
    for m in arr:
        m.scales = None
        m.biases = None
    arr[1].codes += 2
    assert pq2_plan(arr)[0] == -8
