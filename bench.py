"""Benchmark of the Packed-linear hot path on one MI355X.

Default workload (the headline metric): the q_proj-shaped decode GEMV,
K = 5120, N = 6144, batch 1, bf16 activations, 2.25-bit packed weights.
One step = one full pass of the path over one input vector: the signed
1024-block transform of x, its exact split into integer limbs, and the
weight-streaming ternary matmul -- one tb_ternary_gemv call, which runs as a
single kernel launch at this shape.  Steps rotate over enough distinct
copies of the packed weights (>= 1 GiB in total) that the 256 MB last-level
cache cannot serve a repeat, so every step streams its weights from HBM.

Prints ONE JSON line.  `value` is effective weight GB/s of the whole step
(N*K*9/32 bytes of codes, scales and biases per step, over the HIP-event
time of the timed region); `roofline` prices that kernel against the 8 TB/s
HBM peak, its average launch duration taken from HIP events around the
back-to-back launches of the timed region; `cpu_baseline` times the fp64
oracle on the host on the same workload.  The default line also carries
`detail.sweep`: the full batch-1 decode step of the 64-layer model (401
packed linears in one multi-module plan + one embedding lookup), its rate,
roofline, per-layer times and its own oracle baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q_proj]
                    [--workload down_proj --batch B | prefill_gate_up | sweep | tiny]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP6_PEAK_TFLOPS = 10100.0      # MI355X dense fp6 / fp4 MFMA
METRIC = "effective weight GB/s (2.25 bpw) for fused FWHT+ternary GEMV; % of HBM peak"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Per workload: the committed rocprofv3 counter summary of its dominant kernel
# and the sources whose change invalidates it (the kernel's code, the headers
# it includes, the build flags).
_CSRC = os.path.join(ROOT, "hadamard_rotated_quantized_amd", "csrc")
_BUILD = os.path.join(ROOT, "hadamard_rotated_quantized_amd", "build.py")
def _srcs(*names):
    return [os.path.join(_CSRC, f) for f in names + ("tb_gemv.h", "tb_device.h", "tb_common.h")] + [_BUILD]


COUNTER_SUMMARIES = {
    "q_proj": (os.path.join(ROOT, "profiles", "gemv_band_kernel_q_proj_counters.txt"),
               _srcs("tb_gemv_band.hip", "tb_xform.h")),
    "prefill_gate_up": (os.path.join(ROOT, "profiles", "gemm_mx_kernel_prefill_gate_up_counters.txt"),
                        _srcs("tb_gemm.hip", "tb_xform.h")),
    "sweep": (os.path.join(ROOT, "profiles", "multi_stream_kernel_sweep_counters.txt"),
              _srcs("tb_gemv_multi.hip", "tb_ptq1_nat.h", "tb_xform.h")),
    "down_proj_b1": (os.path.join(ROOT, "profiles", "gemv_fused_kernel_down_proj_b1_counters.txt"),
                     _srcs("tb_gemv_fused.hip")),
    "down_proj_b2": (os.path.join(ROOT, "profiles", "batch_stream_kernel_down_proj_b2_counters.txt"),
                     _srcs("tb_gemv_batch.hip", "tb_xform.h")),
    "down_proj_b4": (os.path.join(ROOT, "profiles", "batch_stream_kernel_down_proj_b4_counters.txt"),
                     _srcs("tb_gemv_batch.hip", "tb_xform.h")),
    "down_proj_b8": (os.path.join(ROOT, "profiles", "batch_stream_kernel_down_proj_b8_counters.txt"),
                     _srcs("tb_gemv_batch.hip", "tb_xform.h")),
}


def counter_key(workload, batch=None):
    """Key of the counter summary of a workload's dominant kernel."""
    if workload == "down_proj":
        return f"down_proj_b{batch or 1}"
    return workload


def host_info():
    """(cores this process may use, CPU model, BLAS library, BLAS threads)."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = i.get("num_threads")
                break
    except Exception:
        pass
    return cores, model, blas, threads


def _oracle_threads(cores):
    """Context that runs the oracle's BLAS on `cores` threads (no-op without
    threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline_record(value, unit, sample):
    cores, model, blas, threads = host_info()
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle", "sample": sample,
            "cpu_model": model, "blas": f"{blas}, {threads} threads"}


def kernel_source_hash(workload="q_proj"):
    import hashlib
    h = hashlib.sha256()
    for f in COUNTER_SUMMARIES[workload][1]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, each scaled
    by what the counter reads for a plain copy of known size), or None when no
    summary exists for this workload or the kernel's sources changed after it
    was taken."""
    if workload not in COUNTER_SUMMARIES or not os.path.exists(COUNTER_SUMMARIES[workload][0]):
        return None
    kv = {}
    with open(COUNTER_SUMMARIES[workload][0]) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash(workload):
        log("counter summary is stale (kernel sources changed): traffic = null")
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline_gemv(p, codes, scales, biases, budget_s=12.0):
    """Time the fp64 oracle on the same workload (bounded number of calls),
    its BLAS on every core this process may use."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    with _oracle_threads(cores):
        t0 = time.perf_counter()
        oracle.packed_linear(p.x64, p.signs, p.block, codes, scales, biases)
        one = time.perf_counter() - t0
        reps = max(1, min(20, int(budget_s / max(one, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.packed_linear(p.x64, p.signs, p.block, codes, scales, biases)
        per = (time.perf_counter() - t0) / reps
    return per, reps + 1


GEMV_DTYPE = ("int8 MFMA on exact limbs of the rotated activation (4 x 8 bits, ~30-bit fixed point) x 2-bit codes, "
              "int32 accumulate, fp32 scale/bias epilogue")


WARM_SECONDS = 0.1


def _warm(torch, g, seconds=WARM_SECONDS):
    """Replay graph g (untimed) until `seconds` of wall time have passed: the
    GPU runs its first tens of milliseconds after an idle spell (the oracle's
    CPU work, setup) about 5% slow, so every timed region is preceded by this
    much of its own work on top of the requested warm-up steps."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        g.replay()
        torch.cuda.synchronize()


def _time_graph(torch, g, n_replays, spacer=None):
    """Seconds for n_replays back-to-back replays of graph g, from HIP events
    on the stream.  With a spacer graph, one untimed replay of it is enqueued
    first, so the timed replays are already queued behind it when the start
    event fires and the graph's launch latency stays out of the region."""
    torch.cuda.synchronize()
    if spacer is not None:
        spacer.replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def _parity(got, want):
    got = np.asarray(got, dtype=np.float64)
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    mabs = float(np.abs(got - want).max() / np.abs(want).max())
    return rel, mabs


def _device_problem(p, dev):
    import torch
    import hadamard_rotated_quantized_amd as tb
    codes, s, b = tb.tb_pack(p.t, p.scales)
    c0 = torch.from_numpy(codes.view(np.int32)).to(dev)
    s0 = torch.from_numpy(s).to(dev)
    b0 = torch.from_numpy(b).to(dev)
    x = (torch.from_numpy(p.x_store.view(np.int16)).view(torch.bfloat16) if p.xdtype == "bf16"
         else torch.from_numpy(p.x_store)).to(dev)
    sg = torch.from_numpy(p.signs).to(dev) if p.signs is not None else None
    return c0, s0, b0, x, sg


# ---------------------------------------------------------------------------
# the 402-module decode sweep
# ---------------------------------------------------------------------------
def sweep_setup(dev, check_rows=512, lm_head_rows=2048):
    """Draw and pack every sweep module on the device (one activation per
    input site, shared as a layer shares it), keep the host copies of the
    rows the oracle checks (first module of each shape), and build the plan
    of the 401 linears."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    from hadamard_rotated_quantized_amd import synth

    mods = synth.sweep_modules()
    sites = synth.sweep_input_sites()
    signs_h = synth.sweep_signs()
    signs = {K: torch.from_numpy(v).to(dev) for K, v in signs_h.items()}
    xs = {}
    for si, m in zip(sites, mods):
        if si >= 0 and si not in xs:
            xs[si] = synth.device_site_x(si, m[2], dev)
    packs, ys, checks, seen = [], [], {}, set()
    t0 = time.perf_counter()
    for i, (name, N, K, kind) in enumerate(mods):
        t, sc, _ = synth.device_module_draw(i, N, K, 1, dev)
        packs.append(tb.tb_pack_device(t, sc, check=False))
        if (N, K, kind) not in seen:
            seen.add((N, K, kind))
            rng = np.random.default_rng([synth.SWEEP_SEED, i])
            if kind == "embedding":
                rows = np.array([int(np.random.default_rng(synth.SWEEP_SEED).integers(0, N)), 0, N - 1])
            else:
                n = lm_head_rows if N == synth.VOCAB else check_rows
                rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(N, n) - 2, replace=False)]))
            rt = torch.from_numpy(rows).to(dev)
            checks[i] = (rows, t[rt].cpu().numpy(), sc[rt].cpu().numpy())
        del t, sc
        ys.append(torch.empty((1, N) if kind == "linear" else (3, K), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    log(f"sweep: drew and packed {len(mods)} modules on the device in {time.perf_counter() - t0:.1f} s")
    lin = [i for i, m in enumerate(mods) if m[3] == "linear"]
    emb = [i for i, m in enumerate(mods) if m[3] == "embedding"]
    emb_ids = torch.from_numpy(checks[emb[0]][0].astype(np.int32)).to(dev)

    def plan_of(idx):
        plan, wsb = tb.tb_gemv_multi_plan([(xs[sites[i]], signs[mods[i][2]], *packs[i], ys[i]) for i in idx], 1024)
        return plan, torch.from_numpy(plan).to(dev), torch.empty(wsb, dtype=torch.uint8, device=dev)

    return dict(mods=mods, sites=sites, signs=signs, signs_h=signs_h, xs=xs, packs=packs, ys=ys, checks=checks,
                lin=lin, emb=emb, emb_ids=emb_ids, plan=plan_of(lin), plan_of=plan_of)


def _device_blocks(fmt, codes, sc, N, K):
    """The PQ2_0 or PTQ1_0 blocks of one MLX container on the device (bench
    input preparation): PQ2_0 puts each group's scale bytes before its 32 code
    bytes; PTQ1_0 puts the scale before the group's codes in base 3, five per
    byte, the first code the lowest digit (the last byte holds three)."""
    import torch
    G = K // 128
    sb = sc.view(torch.uint8).view(N, G, 2)
    cb = codes.view(torch.uint8).view(N, G, 32)
    if fmt == "pq2":
        return torch.cat([sb, cb], dim=2).reshape(N, G * 34)
    c = torch.stack([(cb >> (2 * j)) & 3 for j in range(4)], dim=-1).reshape(N, G, 128).to(torch.int16)
    c = torch.nn.functional.pad(c, (0, 2)).view(N, G, 26, 5)
    w = torch.tensor([1, 3, 9, 27, 81], dtype=torch.int16, device=codes.device)
    trits = (c * w).sum(dim=-1).to(torch.uint8)
    return torch.cat([sb, trits], dim=2).reshape(N, G * 28)


def sweep_blocks_measure(sw, nrep, wbytes_mlx, fmt):
    """The sweep's 401 linears as PQ2_0 or PTQ1_0 blocks (the same weights,
    2.125 / 1.75 bits/weight) in one multi-module plan: its step time, rate on
    its own bytes, and agreement with the MLX-container sweep module by
    module.  The blocks are built from the MLX containers on the device and
    checked against the library's host packers on the first module's first
    rows."""
    import torch

    import hadamard_rotated_quantized_amd as tb

    mods, ys, packs, signs = sw["mods"], sw["ys"], sw["packs"], sw["signs"]
    dev = ys[0].device
    nb = 34 if fmt == "pq2" else 28
    blocks, yq = [], []
    for i in sw["lin"]:
        codes, sc, b = packs[i]
        blocks.append(_device_blocks(fmt, codes, sc, mods[i][1], mods[i][2]))
        yq.append(torch.empty_like(ys[i]))
    i0 = sw["lin"][0]
    c0, s0, b0 = (t[:16].cpu().numpy() for t in packs[i0])
    if fmt == "pq2":
        want0 = tb.tb_pq2_from_mlx(c0.view(np.uint32), s0.view(np.uint16), b0.view(np.uint16))
    else:
        want0 = tb.tb_ptq1_pack(tb.tb_unpack(c0.view(np.uint32), mods[i0][2]), s0.view(np.uint16))
    if not np.array_equal(want0, blocks[0][:16].cpu().numpy()):
        raise SystemExit(f"sweep {fmt} blocks differ from the library's host packer")
    planner = tb.tb_pq2_gemv_multi_plan if fmt == "pq2" else tb.tb_ptq1_gemv_multi_plan
    plan, wsb = planner(
        [(sw["xs"][sw["sites"][i]], signs[mods[i][2]], blocks[k], yq[k]) for k, i in enumerate(sw["lin"])], 1024)
    pd = torch.from_numpy(plan).to(dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    tb.tb_ternary_gemv_multi(plan, pd, ws)
    torch.cuda.synchronize()
    worst = 0.0
    for k, i in enumerate(sw["lin"]):
        d = (yq[k].double() - ys[i].double()).abs().max().item() / max(ys[i].abs().max().item(), 1e-30)
        worst = max(worst, d)
    if not worst <= 1e-6:
        raise SystemExit(f"sweep {fmt} result differs from the MLX container's: {worst:.2e} of max |y|")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tb.tb_ternary_gemv_multi(plan, pd, ws)
    g.replay()
    _warm(torch, g)
    sec = _time_graph(torch, g, nrep, spacer=g) / nrep
    qbytes = sum(mods[i][1] * (mods[i][2] // 128) * nb for i in sw["lin"])
    rate = qbytes / sec / 1e9
    out = {"about": f"the same 401 linears as {'PQ2_0' if fmt == 'pq2' else 'PTQ1_0'} blocks ({nb} bytes per 128 "
                    "weights) in one multi-module plan (transform launch + persistent streaming launch; no "
                    "embedding lookup)",
           "weight_bytes": qbytes, "ms_per_step": round(sec * 1e3, 4), "GB/s": round(rate, 1),
           "frac_hbm": round(rate / HBM_PEAK_GBS, 4),
           "mlx_equivalent_GBps": round(wbytes_mlx / sec / 1e9, 1),
           "max_abs_diff_vs_mlx_sweep_of_max_y": worst}
    del g, blocks, yq, ws, pd
    torch.cuda.empty_cache()
    return out


def sweep_measure(n_steps, with_cpu, with_context):
    """Time the sweep step (multi-module path for the 401 linears + the
    embedding lookup of one token) and report it; parity of one module of
    every shape against the oracle first."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    import oracle

    dev = torch.device("cuda:0")
    sw = sweep_setup(dev)
    mods, ys, packs, signs = sw["mods"], sw["ys"], sw["packs"], sw["signs"]
    plan, plan_dev, mws = sw["plan"]

    def step(ids=sw["emb_ids"][:1]):
        """One decode token: every linear, and the embedding lookup of one id."""
        tb.tb_ternary_gemv_multi(plan, plan_dev, mws)
        for i in sw["emb"]:
            tb.tb_embed_inverse(ids, *packs[i], signs[mods[i][2]], 1024, out=ys[i][:ids.numel()])

    step(sw["emb_ids"])  # the parity run looks up the drawn id and the first and last rows
    torch.cuda.synchronize()
    checked, worst = [], 0.0
    cpu_s = {}  # oracle seconds per checked row, by shape
    for i, (rows, t_rows, sc_rows) in sw["checks"].items():
        name, N, K, kind = mods[i]
        oc, osc, ob = oracle.pack(t_rows, sc_rows)
        t0 = time.perf_counter()
        if kind == "linear":
            x64 = sw["xs"][sw["sites"][i]].float().cpu().numpy().astype(np.float64)
            want = oracle.packed_linear(x64, sw["signs_h"][K], 1024, oc, osc, ob)
            got = ys[i][:, torch.from_numpy(rows).to(dev)].cpu().numpy()
        else:
            want = oracle.embed_inverse(np.arange(rows.size), oc, osc, ob, sw["signs_h"][K], 1024)
            got = ys[i].cpu().numpy()
        cpu_s[(N, K, kind)] = (time.perf_counter() - t0) / rows.size
        rel, mabs = _parity(got, want)
        worst = max(worst, rel)
        checked.append(f"{name.split('.')[-1]}:{rel:.1e}")
        if not (rel <= 1e-4 and mabs <= 1e-3):
            raise SystemExit(f"sweep parity check failed on {name}: rel {rel:.2e} max-abs {mabs:.2e}")
    log("sweep parity " + ", ".join(checked))

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    _warm(torch, g)
    nrep = max(3, min(n_steps, 50))
    sec = _time_graph(torch, g, nrep, spacer=g) / nrep
    wbytes = sum(N * K * 9 // 32 for (_, N, K, kind) in mods if kind == "linear")
    value = wbytes / sec / 1e9

    # per layer type and lm_head: plans of only those modules, timed alike
    def layer_plan_us(idx, reps):
        pl, pd, ws = sw["plan_of"](idx)
        gl = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gl):
            tb.tb_ternary_gemv_multi(pl, pd, ws)
        gl.replay()
        _warm(torch, gl, 0.05)
        return _time_graph(torch, gl, reps, spacer=gl) / reps * 1e6

    layer_of = lambda m: int(m[0].split(".")[1]) if m[0].startswith("layers.") else -1
    lin_layers = [i for i in sw["lin"] if layer_of(mods[i]) >= 0 and layer_of(mods[i]) % 4 != 3]
    full_layers = [i for i in sw["lin"] if layer_of(mods[i]) >= 0 and layer_of(mods[i]) % 4 == 3]
    lm = [i for i in sw["lin"] if mods[i][0] == "lm_head"]
    lin_us = layer_plan_us(lin_layers, 10) / 48
    full_us = layer_plan_us(full_layers, 10) / 16
    lm_us = layer_plan_us(lm, 20)
    lbytes = lambda idx: sum(mods[i][1] * mods[i][2] * 9 // 32 for i in idx)
    out = {"workload": "batch-1 decode sweep: 401 packed linears of a 64-layer hidden-5120 model (48 linear-"
                       "attention + 16 full-attention layers, MLP 17408, lm_head 248320) in one multi-module plan "
                       "(transform launch + persistent streaming launch) + one embedding lookup",
           "modules": len(mods), "weight_bytes": wbytes, "steps": nrep,
           "ms_per_step": round(sec * 1e3, 4), "GB/s": round(value, 1), "frac": round(value / HBM_PEAK_GBS, 4),
           "us_per_linear_attention_layer_with_mlp": round(lin_us, 2),
           "us_per_full_attention_layer_with_mlp": round(full_us, 2),
           "lm_head_us": round(lm_us, 2),
           "layer_GBps": {"linear_attention+mlp": round(lbytes(lin_layers) / 48 / (lin_us * 1e-6) / 1e9, 1),
                          "full_attention+mlp": round(lbytes(full_layers) / 16 / (full_us * 1e-6) / 1e9, 1),
                          "lm_head": round(lbytes(lm) / (lm_us * 1e-6) / 1e9, 1)},
           "layer_timing": "each from a plan of only those modules (all 48 linear-attention layers with their MLPs, "
                           "all 16 full-attention layers with theirs, lm_head alone), HIP graphs, divided by the "
                           "layer count",
           "roofline": {"bound": "hbm", "kernel": "multi_stream_kernel", "achieved": round(value, 2),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("sweep")},
           "parity_worst_rel_l2": worst, "parity": checked}
    out["pq2"] = sweep_blocks_measure(sw, nrep, wbytes, "pq2")
    out["ptq1"] = sweep_blocks_measure(sw, nrep, wbytes, "ptq1")
    if with_cpu:
        # the oracle per row of each shape (timed above on the checked rows),
        # scaled to every row of every module of the sweep
        est = sum(cpu_s[(N, K, kind)] * (N if kind == "linear" else 1) for (_, N, K, kind) in mods)
        nrows = sum(r[0].size for r in sw["checks"].values())
        spent = sum(cpu_s[tuple(mods[i][1:])] * r[0].size for i, r in sw["checks"].items())
        out["cpu_baseline"] = cpu_baseline_record(
            round(wbytes / est / 1e9, 4), "GB/s",
            f"fp64 oracle on {nrows} rows (one module of each of the {len(cpu_s)} shapes, the rows the parity "
            f"check reads), {spent:.1f} s; scaled per row to every row of the sweep: {est:.0f} s per step")
    if with_context:
        def call(i):
            name, N, K, kind = mods[i]
            if kind == "linear":
                tb.tb_ternary_gemv(sw["xs"][sw["sites"][i]], signs[K], 1024, *packs[i], out=ys[i])
            else:
                tb.tb_embed_inverse(sw["emb_ids"], *packs[i], signs[K], 1024, out=ys[i])
        gsep = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gsep):
            for i in range(len(mods)):
                call(i)
        gsep.replay()
        _warm(torch, gsep, 0.05)
        r = max(3, min(n_steps, 20))
        sep = _time_graph(torch, gsep, r, spacer=gsep) / r
        out["separate_calls_ms"] = round(sep * 1e3, 4)
        out["separate_calls_GBps"] = round(wbytes / sep / 1e9, 1)
    return out


# ---------------------------------------------------------------------------
# the three containers of one layer: MLX affine (2.25 bpw), PQ2_0 (2.125),
# PTQ1_0 (1.75)
# ---------------------------------------------------------------------------
FORMAT_BITS = {"mlx": 2.25, "pq2": 2.125, "ptq1": 1.75}


def format_containers(p, fmt, dev):
    """Device tensors of one container of problem p and the call that runs
    the Packed linear on them (batch 1)."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    c, s, b = tb.tb_pack(p.t, p.scales)
    if fmt == "mlx":
        return (torch.from_numpy(c.view(np.int32)).to(dev), torch.from_numpy(s).to(dev), torch.from_numpy(b).to(dev))
    blk = tb.tb_pq2_from_mlx(c, s, b) if fmt == "pq2" else tb.tb_ptq1_pack(p.t, p.scales)
    return (torch.from_numpy(blk).to(dev),)


def format_step(fmt, x, sg, block, cont, y, ws):
    import hadamard_rotated_quantized_amd as tb
    if fmt == "mlx":
        tb.tb_ternary_gemv(x, sg, block, *cont, out=y, workspace=ws)
    elif fmt == "pq2":
        tb.tb_pq2_gemv(x, sg, block, cont[0], out=y)
    else:
        tb.tb_ptq1_gemv(x, sg, block, cont[0], out=y)


def formats_measure(p, reps_per_graph=None, replays=10):
    """Per container: us per batch-1 call over rotating replicas (>= 1 GiB,
    so no call finds its blocks in the last-level cache), HIP graphs behind
    an untimed replay; parity of each container against the oracle first."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    import oracle

    dev = torch.device("cuda:0")
    x = (torch.from_numpy(p.x_store.view(np.int16)).view(torch.bfloat16) if p.xdtype == "bf16"
         else torch.from_numpy(p.x_store)).to(dev)
    sg = torch.from_numpy(p.signs).to(dev)
    y = torch.empty((1, p.N), dtype=torch.float32, device=dev)
    ws = torch.empty(tb.tb_ternary_gemv_workspace_size_n(1, p.K, p.N), dtype=torch.uint8, device=dev)
    rows = np.unique(np.concatenate([[0, p.N - 1], np.random.default_rng(9).integers(0, p.N, 510)]))
    oc, osc, ob = oracle.pack(p.t[rows], p.scales[rows])
    want = oracle.packed_linear(p.x64[:1], p.signs, p.block, oc, osc, ob)
    out = {}
    for fmt, bits in FORMAT_BITS.items():
        cont = format_containers(p, fmt, dev)
        wbytes = int(p.N * p.K * bits / 8)
        R = max(2, math.ceil((1 << 30) / wbytes))
        reps = [cont] + [tuple(t.clone() for t in cont) for _ in range(R - 1)]
        format_step(fmt, x, sg, p.block, reps[-1], y, ws)
        torch.cuda.synchronize()
        rel, mabs = _parity(y[:, torch.from_numpy(rows).to(dev)].cpu().numpy(), want)
        if not (rel <= 1e-4 and mabs <= 1e-3):
            raise SystemExit(f"{fmt} parity check failed: rel {rel:.2e} max-abs {mabs:.2e}")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                format_step(fmt, x, sg, p.block, reps[i], y, ws)
        g.replay()
        _warm(torch, g, 0.05)
        us = _time_graph(torch, g, replays, spacer=g) / (replays * R) * 1e6
        gbs = wbytes / (us * 1e-6) / 1e9
        out[fmt] = {"bits_per_weight": bits, "weight_bytes": wbytes, "us": round(us, 3), "GB/s": round(gbs, 1),
                    "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "replicas": R, "parity_rel_l2": rel}
        del reps, g
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# counter passes (rocprofv3 --pmc)
# ---------------------------------------------------------------------------
def run_counter_pass(args):
    """Eager launches only, no timing: the command that rocprofv3 --pmc passes
    wrap.  `--workload copy` runs plain device copies of a known size (the
    calibration of the FETCH_SIZE / WRITE_SIZE counters)."""
    import torch

    dev = torch.device("cuda:0")
    if args.workload == "copy":
        nbytes = 64 << 20
        bufs = [torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_() for _ in range(4)]
        dst = torch.empty_like(bufs[0])
        for i in range(40):
            dst.copy_(bufs[i % 4])
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": "copy", "bytes_per_copy": nbytes, "copies": 40}), flush=True)
        return
    import hadamard_rotated_quantized_amd as tb
    from hadamard_rotated_quantized_amd import synth

    if args.workload == "sweep":
        sw = sweep_setup(dev, check_rows=2, lm_head_rows=2)
        plan, pd, ws = sw["plan"]
        for _ in range(3):
            tb.tb_ternary_gemv_multi(plan, pd, ws)
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": "sweep", "launches": 3}), flush=True)
        return
    p = synth.config_problem(args.workload, args.batch)
    c0, s0, b0, x, sg = _device_problem(p, dev)
    if args.workload == "prefill_gate_up":
        ws = torch.empty(tb.tb_ternary_gemm_workspace_size_n(p.B, p.K, p.N), dtype=torch.uint8, device=dev)
        y = torch.empty((p.B, p.N), dtype=torch.float32, device=dev)
        for _ in range(5):
            tb.tb_ternary_gemm(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": args.workload, "launches": 5}), flush=True)
        return
    R = args.replicas or max(1, math.ceil((1 << 30) / (p.N * p.K * 9 // 32)))
    reps = [(c0, s0, b0)] + [(c0.clone(), s0.clone(), b0.clone()) for _ in range(R - 1)]
    ws = torch.empty(tb.tb_ternary_gemv_workspace_size_n(p.B, p.K, p.N), dtype=torch.uint8, device=dev)
    y = torch.empty((p.B, p.N), dtype=torch.float32, device=dev)
    for i in range(3 * R):
        tb.tb_ternary_gemv(x, sg, p.block, *reps[i % R], out=y, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"counter_pass": args.workload, "batch": p.B, "launches": 3 * R, "replicas": R,
                      "weight_bytes": p.N * p.K * 9 // 32}), flush=True)


# ---------------------------------------------------------------------------
# decode GEMV workloads (the headline)
# ---------------------------------------------------------------------------
def run_gemv(args):
    """Decode GEMV workloads: q_proj (default), tiny, down_proj (--batch 1..8).
    The default run also measures the 402-module decode sweep (detail.sweep)."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    import oracle
    from hadamard_rotated_quantized_amd import synth

    p = synth.config_problem(args.workload, args.batch)
    N, K, B = p.N, p.K, p.B
    wbytes = N * K * 9 // 32
    log(f"workload {args.workload}: N={N} K={K} B={B} weight bytes {wbytes}")
    dev = torch.device("cuda:0")
    c0, s0, b0, x, sg = _device_problem(p, dev)
    R = args.replicas or max(1, math.ceil((1 << 30) / wbytes))
    reps = [(c0, s0, b0)] + [(c0.clone(), s0.clone(), b0.clone()) for _ in range(R - 1)]
    ws = torch.empty(tb.tb_ternary_gemv_workspace_size_n(B, K, N), dtype=torch.uint8, device=dev)
    y = torch.empty((B, N), dtype=torch.float32, device=dev)

    # parity of the exact configuration that is timed
    oc, osc, ob = oracle.pack(p.t, p.scales)
    want = oracle.packed_linear(p.x64, p.signs, p.block, oc, osc, ob)
    tb.tb_ternary_gemv(x, sg, p.block, *reps[R - 1], out=y, workspace=ws)
    torch.cuda.synchronize()
    rel, mabs = _parity(y.cpu().numpy(), want)
    log(f"parity rel L2 {rel:.2e} max-abs {mabs:.2e}")
    if not (rel <= 1e-4 and mabs <= 1e-3):
        raise SystemExit("parity check failed; refusing to report a number")

    def capture(n, one_call):
        """HIP graph of n consecutive steps over the replica ring (the kernels
        are recorded exactly as the eager calls enqueue them)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                c, sc, bi = reps[i % R]
                if one_call:
                    tb.tb_ternary_gemv(x, sg, p.block, c, sc, bi, out=y, workspace=ws)
                else:
                    tb.tb_ternary_gemv_prepare(x, sg, p.block, ws)
                    tb.tb_ternary_gemv_run(ws, B, K, c, sc, bi, out=y)
        return g

    y_eager = y.clone()
    full, rem = divmod(args.steps, R)
    g_steps = capture(R, True)
    g_rem = capture(rem, True) if rem and args.steps > 2 * R else None
    # warm-up: every graph the timed region replays is replayed first (the
    # first replay of a graph also uploads it)
    for _ in range(max(1, args.warmup // R)):
        g_steps.replay()
    if g_rem is not None:
        g_rem.replay()
    _warm(torch, g_steps)

    # Timed: exactly `steps` steps, queued behind untimed replays of the ring
    # so that they run back to back from the start event on.  A graph replay
    # carries a fixed cost of about 10 us on top of its kernels, which a
    # long region spreads over thousands of steps; a short region (at most
    # two rings) is issued as eager calls instead, all of them enqueued while
    # the spacer replays still run (each ring replay covers the host time of
    # far more than R calls).
    eager = args.steps <= 2 * R
    for _ in range(3 if eager else 1):
        g_steps.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    if eager:
        for i in range(args.steps):
            tb.tb_ternary_gemv(x, sg, p.block, *reps[i % R], out=y, workspace=ws)
    else:
        for _ in range(full):
            g_steps.replay()
        if g_rem is not None:
            g_rem.replay()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    if not torch.equal(y, y_eager):
        raise SystemExit("the timed steps' result differs from the first call's")

    # Batch 1: one step is one launch of the single-launch kernel, so the
    # kernel's average launch duration is the timed region over the launches
    # (the dispatch gap between back-to-back launches included).  Batches
    # 2..8: a step is the K-split streaming kernel plus, when K is split over
    # several workgroups, the slice-sum kernel; the rate over the whole step
    # is then a lower bound for the streaming kernel alone.
    ms_step = total_ms / args.steps
    main_us = ms_step * 1e3
    value = wbytes * args.steps / (total_ms * 1e-3) / 1e9
    achieved = wbytes / (main_us * 1e-6) / 1e9

    # context: the two-kernel path (prepare + run) on the same ring, and a
    # hot (cache-resident) repeat of one replica, labelled as such
    reps_k = max(1, min(20, args.steps // R))
    g_two = capture(R, False)
    g_two.replay()
    _warm(torch, g_two, 0.05)
    two_us = _time_graph(torch, g_two, reps_k, spacer=g_two) / (reps_k * R) * 1e6
    g_hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_hot):
        for _ in range(100):
            tb.tb_ternary_gemv(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
    g_hot.replay()
    hot_us = _time_graph(torch, g_hot, 5, spacer=g_hot) / 500 * 1e6

    cpu = None
    if not args.no_cpu_baseline:
        per, ncalls = cpu_baseline_gemv(p, oc, osc, ob)
        cpu = cpu_baseline_record(round(wbytes / per / 1e9, 4), "GB/s",
                                  f"{ncalls} full {args.workload} calls (N={N}, K={K}, B={B}), {per * 1e3:.1f} ms "
                                  "each, numpy fp64 (unpack and dequantize single-threaded, matvec on BLAS)")

    kernel = "gemv_band_kernel" if B == 1 and args.workload != "down_proj" else (
        "gemv_fused_kernel" if B == 1 else "batch_stream_kernel (+ batch_reduce_kernel)")
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": GEMV_DTYPE,
        "data": "synthetic",
        "config": {"workload": f"{args.workload} decode GEMV N={N} K={K} batch {B} {p.xdtype} activations, "
                               f"2.25 bpw packed weights, {R} rotating weight replicas",
                   "N": N, "K": K, "batch": B, "block": p.block, "replicas": R},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(counter_key(args.workload, B))},
        "cpu_baseline": cpu,
        "detail": {"kernel": kernel,
                   "kernel_us_mean": round(main_us, 3),
                   "timing": ("eager calls" if eager else "HIP graph replays") +
                             " of back-to-back steps over the replica ring, queued behind untimed replays; " +
                             ("one step is one launch of the single-launch kernel" if B == 1 else
                              "one step is the streaming launch plus the slice-sum launch when K is split"),
                   "step_us": round(ms_step * 1e3, 3),
                   "two_kernel_path_step_us": round(two_us, 3),
                   "hot_step_us_same_replica": round(hot_us, 3),
                   "parity_rel_l2": rel, "parity_max_abs_rel": mabs},
    }
    if args.workload == "q_proj" and not args.no_sweep:
        del reps, g_steps, g_rem, g_two, g_hot
        torch.cuda.empty_cache()
        out["detail"]["sweep"] = sweep_measure(args.steps, not args.no_cpu_baseline, False)
        torch.cuda.empty_cache()
        gate = synth.make_problem("gate_proj", 17408, 5120, 1, 41, "bf16", 1024)
        out["detail"]["formats"] = {
            "about": "batch-1 Packed linear in the three containers of one set of ternary weights: MLX affine "
                     "(2.25 bpw), PQ2_0 (2.125), PTQ1_0 (1.75); us per call over rotating replicas of >= 1 GiB",
            "q_proj N=6144 K=5120": formats_measure(p),
            "gate_proj N=17408 K=5120": formats_measure(gate)}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# prefill GEMM
# ---------------------------------------------------------------------------
def run_prefill(args):
    """Prefill GEMM gate/up_proj: M=2048, K=5120, N=17408, bf16 x.  One step =
    one tb_ternary_gemm call (rotation + fp6 digit kernel, then the
    block-scaled fp6 x fp4 MFMA matmul).  value = algorithmic TFLOP/s
    (2 M N K per step)."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    import oracle
    from hadamard_rotated_quantized_amd import synth

    p = synth.config_problem("prefill_gate_up")
    M, N, K = p.B, p.N, p.K
    flops = 2.0 * M * N * K
    dev = torch.device("cuda:0")
    c0, s0, b0, x, sg = _device_problem(p, dev)
    ws = torch.empty(tb.tb_ternary_gemm_workspace_size_n(M, K, N), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    tb.tb_ternary_gemm(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 1023, M - 1],
                                     np.random.default_rng(44).integers(0, M, 56)]))
    oc, osc, ob = oracle.pack(p.t, p.scales)
    want = oracle.packed_linear(p.x64[rows], p.signs, p.block, oc, osc, ob)
    rel, mabs = _parity(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), want)
    log(f"parity (sampled rows) rel L2 {rel:.2e} max-abs {mabs:.2e}")
    if not (rel <= 1e-4 and mabs <= 1e-3):
        raise SystemExit("parity check failed; refusing to report a number")

    steps = max(10, min(args.steps, 200)) // 10 * 10
    warm = max(1, min(args.warmup, 20))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            tb.tb_ternary_gemm(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        for _ in range(10):
            tb.tb_ternary_gemm_run(ws, M, K, c0, s0, b0, out=y)
    for _ in range(max(1, warm // 10)):
        g.replay()
    g2.replay()
    _warm(torch, g)
    nrep = steps // 10
    t = _time_graph(torch, g, nrep, spacer=g) / steps
    t_run = _time_graph(torch, g2, nrep, spacer=g2) / steps
    tflops = flops / t / 1e12
    run_tflops = flops / t_run / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        sample = 16
        with _oracle_threads(len(os.sched_getaffinity(0))):
            t0 = time.perf_counter()
            oracle.packed_linear(p.x64[:sample], p.signs, p.block, oc, osc, ob)
            per = time.perf_counter() - t0
        cpu = cpu_baseline_record(round(2.0 * sample * N * K / per / 1e12, 6), "TFLOP/s",
                                  f"{sample} of the {M} activation rows against the whole {N}x{K} pack, {per:.1f} s, "
                                  "numpy fp64")

    out = {
        "metric": "algorithmic TFLOP/s of the prefill Packed linear (2 M N K per call)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp6 digits of the rotated activation x fp4 codes (block-scaled MFMA), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"prefill gate/up_proj GEMM M={M} K={K} N={N}, bf16 activations, 2.25 bpw packed "
                               "weights", "M": M, "N": N, "K": K, "block": p.block},
        "roofline": {"bound": "mfma", "achieved": round(run_tflops, 2), "peak": FP6_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(run_tflops / FP6_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_gate_up")},
        "cpu_baseline": cpu,
        "detail": {"kernel": "gemm_mx_kernel", "main_kernel_ms": round(t_run * 1e3, 4),
                   "step_ms_prepare_and_run": round(t * 1e3, 4),
                   "issued_mfma_frac": round(4 * run_tflops / FP6_PEAK_TFLOPS, 4),
                   "note": "each input enters the MFMA as four fp6 digits, so the issued MFMA work is four times "
                           "the algorithmic 2 M N K",
                   "parity_rel_l2": rel, "parity_max_abs_rel": mabs, "parity_rows": int(len(rows))},
    }
    print(json.dumps(out), flush=True)


def run_sweep(args):
    """The full decode sweep at batch 1 as its own line: the 401 packed
    linears of the 64-layer model and one embedding row; one step = the
    multi-module plan + the embedding call, captured as one HIP graph."""
    d = sweep_measure(args.steps, not args.no_cpu_baseline, True)
    out = {
        "metric": "effective weight GB/s (2.25 bpw), full batch-1 decode sweep of 402 packed modules",
        "value": d["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": d["steps"], "warmup": 1,
        "ms_per_step": d["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": GEMV_DTYPE, "data": "synthetic",
        "config": {"workload": d["workload"], "modules": d["modules"], "weight_bytes": d["weight_bytes"]},
        "roofline": d["roofline"], "cpu_baseline": d.get("cpu_baseline"),
        "detail": {k: v for k, v in d.items() if k not in ("roofline", "cpu_baseline", "workload")},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12200)
    ap.add_argument("--warmup", type=int, default=1220)
    ap.add_argument("--workload", default="q_proj",
                    choices=["q_proj", "tiny", "down_proj", "prefill_gate_up", "sweep", "copy"])
    ap.add_argument("--batch", type=int, default=None, help="down_proj batch (1, 2, 4 or 8)")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="q_proj line without the sweep detail")
    ap.add_argument("--counters-only", action="store_true",
                    help="eager launches without timing, for rocprofv3 --pmc passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.workload == "down_proj" and args.batch is None:
        args.batch = 1
    if args.counters_only:
        run_counter_pass(args)
    elif args.workload == "copy":
        raise SystemExit("--workload copy is a counter-calibration pass: use it with --counters-only")
    elif args.workload == "prefill_gate_up":
        run_prefill(args)
    elif args.workload == "sweep":
        run_sweep(args)
    else:
        run_gemv(args)


if __name__ == "__main__":
    main()
