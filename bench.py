"""Benchmark of the Packed-linear hot path on one MI355X.

Default workload (the headline metric): the q_proj-shaped decode GEMV,
K = 5120, N = 6144, batch 1, bf16 activations, 2.25-bit packed weights.
One step = one full pass of the path over one input vector: the signed
1024-block transform of x, its exact split into integer limbs, and the
weight-streaming ternary matmul -- one tb_ternary_gemv call, which runs as a
single kernel launch at this shape.  Steps
rotate over enough distinct copies of the packed weights (>= 1 GiB in
total) that the 256 MB last-level cache cannot serve a repeat, so every
step streams its weights from HBM.

Prints ONE JSON line.  `value` is effective weight GB/s of the whole step
(N*K*9/32 bytes of codes, scales and biases per step, over the HIP-event
time of the timed region); `roofline` prices that kernel against the 8 TB/s
HBM peak, its average launch duration taken from HIP events around the
back-to-back launches of the timed region; `cpu_baseline` times the fp64
oracle on the host on the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q_proj]
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
COUNTER_SUMMARIES = {
    "q_proj": (os.path.join(ROOT, "profiles", "gemv_band_kernel_q_proj_counters.txt"),
               [os.path.join(_CSRC, f) for f in ("tb_gemv_band.hip", "tb_xform.h", "tb_gemv.h", "tb_device.h",
                                                  "tb_common.h")] + [_BUILD]),
    "prefill_gate_up": (os.path.join(ROOT, "profiles", "gemm_mx_kernel_prefill_gate_up_counters.txt"),
                        [os.path.join(_CSRC, f) for f in ("tb_gemm.hip", "tb_xform.h", "tb_gemv.h", "tb_device.h",
                                                           "tb_common.h")] + [_BUILD]),
}


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
    """Time the fp64 oracle on the same workload (bounded number of calls)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    t0 = time.perf_counter()
    oracle.packed_linear(p.x64, p.signs, p.block, codes, scales, biases)
    one = time.perf_counter() - t0
    reps = max(1, min(20, int(budget_s / max(one, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.packed_linear(p.x64, p.signs, p.block, codes, scales, biases)
    per = (time.perf_counter() - t0) / reps
    return per, reps + 1, blas_threads


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

    p = synth.config_problem(args.workload)
    codes, s, b = tb.tb_pack(p.t, p.scales)
    if args.workload == "prefill_gate_up":
        c0 = torch.from_numpy(codes.view(np.int32)).to(dev)
        s0 = torch.from_numpy(s).to(dev)
        b0 = torch.from_numpy(b).to(dev)
        x = torch.from_numpy(p.x_store.view(np.int16)).view(torch.bfloat16).to(dev)
        sg = torch.from_numpy(p.signs).to(dev)
        ws = torch.empty(tb.tb_ternary_gemm_workspace_size_n(p.B, p.K, p.N), dtype=torch.uint8, device=dev)
        y = torch.empty((p.B, p.N), dtype=torch.float32, device=dev)
        for _ in range(5):
            tb.tb_ternary_gemm(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"counter_pass": args.workload, "launches": 5}), flush=True)
        return
    c0 = torch.from_numpy(codes.view(np.int32)).to(dev)
    s0 = torch.from_numpy(s).to(dev)
    b0 = torch.from_numpy(b).to(dev)
    R = args.replicas or max(1, math.ceil((1 << 30) / (p.N * p.K * 9 // 32)))
    reps = [(c0, s0, b0)] + [(c0.clone(), s0.clone(), b0.clone()) for _ in range(R - 1)]
    x = (torch.from_numpy(p.x_store.view(np.int16)).view(torch.bfloat16) if p.xdtype == "bf16"
         else torch.from_numpy(p.x_store)).to(dev)
    sg = torch.from_numpy(p.signs).to(dev)
    ws = torch.empty(tb.tb_ternary_gemv_workspace_size_n(p.B, p.K, p.N), dtype=torch.uint8, device=dev)
    y = torch.empty((p.B, p.N), dtype=torch.float32, device=dev)
    for i in range(3 * R):
        tb.tb_ternary_gemv(x, sg, p.block, *reps[i % R], out=y, workspace=ws)
    torch.cuda.synchronize()
    print(json.dumps({"counter_pass": args.workload, "launches": 3 * R, "replicas": R,
                      "weight_bytes": p.N * p.K * 9 // 32}), flush=True)


def run_gemv(args):
    """Decode GEMV workloads: q_proj (default), tiny, down_proj (--batch 1..8)."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    import oracle
    from hadamard_rotated_quantized_amd import synth

    p = synth.config_problem(args.workload, args.batch)
    N, K, B = p.N, p.K, p.B
    wbytes = N * K * 9 // 32
    log(f"workload {args.workload}: N={N} K={K} B={B} weight bytes {wbytes}")
    codes, s, b = tb.tb_pack(p.t, p.scales)
    dev = torch.device("cuda:0")
    c0 = torch.from_numpy(codes.view(np.int32)).to(dev)
    s0 = torch.from_numpy(s).to(dev)
    b0 = torch.from_numpy(b).to(dev)
    R = args.replicas or max(1, math.ceil((1 << 30) / wbytes))
    reps = [(c0, s0, b0)] + [(c0.clone(), s0.clone(), b0.clone()) for _ in range(R - 1)]
    x = (torch.from_numpy(p.x_store.view(np.int16)).view(torch.bfloat16) if p.xdtype == "bf16"
         else torch.from_numpy(p.x_store)).to(dev)
    sg = torch.from_numpy(p.signs).to(dev)
    ws = torch.empty(tb.tb_ternary_gemv_workspace_size_n(B, K, N), dtype=torch.uint8, device=dev)
    y = torch.empty((B, N), dtype=torch.float32, device=dev)

    # parity of the exact configuration that is timed
    oc, osc, ob = oracle.pack(p.t, p.scales)
    want = oracle.packed_linear(p.x64, p.signs, p.block, oc, osc, ob)
    tb.tb_ternary_gemv(x, sg, p.block, *reps[R - 1], out=y, workspace=ws)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    mabs = float(np.abs(got - want).max() / np.abs(want).max())
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

    def time_graph(g, n_replays, n_steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n_steps  # us per step

    y_eager = y.clone()
    full, rem = divmod(args.steps, R)
    g_steps = capture(R, True)
    g_rem = capture(rem, True) if rem else None
    for _ in range(max(1, args.warmup // R)):
        g_steps.replay()
    torch.cuda.synchronize()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(full):
        g_steps.replay()
    if g_rem is not None:
        g_rem.replay()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    if not torch.equal(y, y_eager):
        raise SystemExit("graph replay result differs from the eager result")

    # Batch 1: one step is one launch of the single-launch band kernel, so
    # the kernel's average launch duration is the timed region over the
    # launches (the dispatch gap between back-to-back launches included).
    # Batches 2..8: a step is the K-split streaming kernel plus, when K is
    # split over several workgroups, the slice-sum kernel; the rate over the
    # whole step is then a lower bound for the streaming kernel alone.
    ms_step = total_ms / args.steps
    main_us = ms_step * 1e3
    value = wbytes * args.steps / (total_ms * 1e-3) / 1e9
    achieved = wbytes / (main_us * 1e-6) / 1e9

    # context: the two-kernel path (prepare + run) on the same ring, and a
    # hot (cache-resident) repeat of one replica, labelled as such
    reps_k = max(1, min(20, args.steps // R))
    g_two = capture(R, False)
    g_two.replay()
    two_us = time_graph(g_two, reps_k, reps_k * R)
    g_hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_hot):
        for _ in range(100):
            tb.tb_ternary_gemv(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
    g_hot.replay()
    hot_us = time_graph(g_hot, 5, 500)

    cpu = None
    if not args.no_cpu_baseline:
        per, ncalls, thr = cpu_baseline_gemv(p, oc, osc, ob)
        cpu = {"value": round(wbytes / per / 1e9, 4), "unit": "GB/s", "cores": thr, "kind": "oracle",
               "sample": f"{ncalls} full {args.workload} calls (N={N}, K={K}, B={B}), "
                         f"{per * 1e3:.1f} ms each, numpy fp64 (decode single-threaded, BLAS {thr} threads)"}

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
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{args.workload} decode GEMV N={N} K={K} batch {B} {p.xdtype} activations, "
                               f"2.25 bpw packed weights, {R} rotating weight replicas",
                   "N": N, "K": K, "batch": B, "block": p.block, "replicas": R},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload)},
        "cpu_baseline": cpu,
        "detail": {"kernel": "gemv_band_kernel" if B == 1 else "batch_stream_kernel (+ batch_reduce_kernel)",
                   "kernel_us_mean": round(main_us, 3),
                   "timing": "HIP graph of back-to-back steps over the replica ring; " +
                             ("one step is one launch of the single-launch kernel" if B == 1 else
                              "one step is the streaming launch plus the slice-sum launch when K is split"),
                   "step_us": round(ms_step * 1e3, 3),
                   "two_kernel_path_step_us": round(two_us, 3),
                   "hot_step_us_same_replica": round(hot_us, 3),
                   "parity_rel_l2": rel, "parity_max_abs_rel": mabs},
    }
    print(json.dumps(out), flush=True)


def _time_graph(torch, g, n_replays):
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3  # seconds


def _parity(got, want):
    got = np.asarray(got, dtype=np.float64)
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    mabs = float(np.abs(got - want).max() / np.abs(want).max())
    return rel, mabs


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
    codes, s, b = tb.tb_pack(p.t, p.scales)
    c0 = torch.from_numpy(codes.view(np.int32)).to(dev)
    s0 = torch.from_numpy(s).to(dev)
    b0 = torch.from_numpy(b).to(dev)
    x = torch.from_numpy(p.x_store.view(np.int16)).view(torch.bfloat16).to(dev)
    sg = torch.from_numpy(p.signs).to(dev)
    ws = torch.empty(tb.tb_ternary_gemm_workspace_size_n(M, K, N), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    tb.tb_ternary_gemm(x, sg, p.block, c0, s0, b0, out=y, workspace=ws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 1023, M - 1],
                                     np.random.default_rng(44).integers(0, M, 26)]))
    oc, osc, ob = oracle.pack(p.t, p.scales)
    want = oracle.packed_linear(p.x64[rows], p.signs, p.block, oc, osc, ob)
    rel, mabs = _parity(y[torch.from_numpy(rows).to(dev)].cpu().numpy(), want)
    log(f"parity (sampled rows) rel L2 {rel:.2e} max-abs {mabs:.2e}")
    if not (rel <= 1e-4 and mabs <= 1e-3):
        raise SystemExit("parity check failed; refusing to report a number")

    steps = max(1, min(args.steps, 200))
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
    torch.cuda.synchronize()
    nrep = max(1, steps // 10)
    t = _time_graph(torch, g, nrep) / (nrep * 10)
    t_run = _time_graph(torch, g2, nrep) / (nrep * 10)
    tflops = flops / t / 1e12
    run_tflops = flops / t_run / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        sample = 16
        t0 = time.perf_counter()
        oracle.packed_linear(p.x64[:sample], p.signs, p.block, oc, osc, ob)
        per = time.perf_counter() - t0
        cpu = {"value": round(2.0 * sample * N * K / per / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(),
               "kind": "oracle",
               "sample": f"{sample} of the {M} activation rows against the whole {N}x{K} pack, {per:.1f} s, numpy fp64"}

    out = {
        "metric": "algorithmic TFLOP/s of the prefill Packed linear (2 M N K per call)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": nrep * 10, "warmup": warm,
        "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp6 x fp4 (block-scaled MFMA, fp32 accumulate)", "data": "synthetic",
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


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def run_sweep(args):
    """The full decode sweep at batch 1: the 401 packed linears of the
    64-layer model (3:1 linear:full attention layers, MLP 17408, lm_head
    248320) and one embedding row with the inverse transform.  Every module
    has its own synthetic pack and input (modules are not chained).  One step
    = all 402 calls, captured once as a HIP graph."""
    import torch

    import hadamard_rotated_quantized_amd as tb
    import oracle
    from hadamard_rotated_quantized_amd import synth

    dev = torch.device("cuda:0")
    mods = synth.sweep_modules()
    signs_h = synth.sweep_signs()
    signs = {k: torch.from_numpy(v).to(dev) for k, v in signs_h.items()}
    packs, xs, ys = [], [], []
    t0 = time.perf_counter()
    for i, (name, N, K, kind) in enumerate(mods):
        t, sc, x = synth.device_module_draw(i, N, K, 1, dev)
        codes, so, bo = tb.tb_pack_device(t, sc, check=False)
        del t, sc
        packs.append((codes, so, bo))
        xs.append(x)
        ys.append(torch.empty((1, N) if kind == "linear" else (1, K), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    log(f"drew and packed {len(mods)} modules in {time.perf_counter() - t0:.1f} s")
    embed_id = torch.tensor([int(np.random.default_rng(synth.SWEEP_SEED).integers(0, synth.VOCAB))],
                            dtype=torch.int32, device=dev)
    wsz = tb.tb_ternary_gemv_workspace_size(1, max(m[2] for m in mods))
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)

    def call(i):
        name, N, K, kind = mods[i]
        c, sc, bi = packs[i]
        if kind == "linear":
            tb.tb_ternary_gemv(xs[i], signs[K], 1024, c, sc, bi, out=ys[i], workspace=ws)
        else:
            tb.tb_embed_inverse(embed_id, c, sc, bi, signs[K], 1024, out=ys[i])

    for i in range(len(mods)):
        call(i)
    torch.cuda.synchronize()
    # parity on one module of every shape (lm_head on sampled rows) and the embedding row
    checked, worst = [], 0.0
    seen = set()
    for i, (name, N, K, kind) in enumerate(mods):
        key = (N, K, kind)
        if key in seen:
            continue
        seen.add(key)
        t, sc, _ = synth.device_module_draw(i, N, K, 1, dev)
        if kind == "linear":
            rows = np.arange(N) if N <= 20000 else np.unique(np.concatenate(
                [[0, N - 1], np.random.default_rng(i).integers(0, N, 2046)]))
        else:
            rows = np.array([int(embed_id.item())])
        rt = torch.from_numpy(rows).to(dev)
        oc, osc, ob = oracle.pack(t[rt].cpu().numpy(), sc[rt].cpu().numpy())
        del t, sc
        if kind == "linear":
            xh = xs[i].float().cpu().numpy().astype(np.float64)
            want = oracle.packed_linear(xh, signs_h[K], 1024, oc, osc, ob)
            got = ys[i][:, rt].cpu().numpy()
        else:
            want = oracle.embed_inverse([0], oc, osc, ob, signs_h[K], 1024)
            got = ys[i].cpu().numpy()
        rel, mabs = _parity(got, want)
        worst = max(worst, rel)
        checked.append(f"{name}:{rel:.1e}")
        if not (rel <= 1e-4 and mabs <= 1e-3):
            raise SystemExit(f"parity check failed on {name}: rel {rel:.2e} max-abs {mabs:.2e}")
    log("parity " + ", ".join(checked))

    # the step: all 401 linears through the multi-module path (one transform
    # launch, one persistent streaming launch) plus the embedding row
    lin = [i for i, m in enumerate(mods) if m[3] == "linear"]
    emb = [i for i, m in enumerate(mods) if m[3] == "embedding"]
    plan, wsb = tb.tb_gemv_multi_plan([(xs[i], signs[mods[i][2]], *packs[i], ys[i]) for i in lin], 1024)
    plan_dev = torch.from_numpy(plan).to(dev)
    mws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step():
        tb.tb_ternary_gemv_multi(plan, plan_dev, mws)
        for i in emb:
            call(i)

    # the multi path must reproduce the per-module calls' outputs (checked
    # against the oracle above) within the parity bar
    ref = [ys[i].clone() for i in lin]
    for i in lin:
        ys[i].fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    worst_multi = 0.0
    for r, i in zip(ref, lin):
        d = float((ys[i].double() - r.double()).norm() / r.double().norm())
        worst_multi = max(worst_multi, d)
    log(f"multi-module path vs per-module calls: worst rel L2 {worst_multi:.2e}")
    if not worst_multi <= 1e-4:
        raise SystemExit("multi-module path disagrees with the per-module calls")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    nrep = max(3, min(args.steps, 50))
    sec = _time_graph(torch, g, nrep) / nrep
    wbytes = sum(N * K * 9 // 32 for (_, N, K, kind) in mods if kind == "linear") + 5120 * 9 // 32
    value = wbytes / sec / 1e9

    # context: the same 402 modules as separate calls in one graph
    gsep = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gsep):
        for i in range(len(mods)):
            call(i)
    gsep.replay()
    torch.cuda.synchronize()
    sep_sec = _time_graph(torch, gsep, max(3, min(args.steps, 20))) / max(3, min(args.steps, 20))

    # per-shape timing: a graph of every module of one shape, back to back;
    # a shape with few modules (lm_head, the embedding row) is called again
    # in the graph until it holds at least 32 calls, so that the graph's own
    # launch cost is spread as it is for the other shapes
    per_shape = {}
    for key in sorted({(m[1], m[2], m[3]) for m in mods}):
        idx = [i for i, m in enumerate(mods) if (m[1], m[2], m[3]) == key]
        idx = idx * max(1, -(-32 // len(idx)))
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            for i in idx:
                call(i)
        gs.replay()
        torch.cuda.synchronize()
        r = max(3, min(20, 2000 // len(idx)))
        us = _time_graph(torch, gs, r) / (r * len(idx)) * 1e6
        N, K, kind = key
        b = N * K * 9 // 32 if kind == "linear" else 5120 * 9 // 32
        per_shape[f"{kind} {N}x{K}"] = {"count": sum(m[1:] == key for m in mods), "calls_timed": len(idx),
                                        "us_each": round(us, 3),
                                        "GB/s": round(b / (us * 1e-6) / 1e9, 1)}

    out = {
        "metric": "effective weight GB/s (2.25 bpw), full batch-1 decode sweep of 402 packed modules",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": nrep, "warmup": 1,
        "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": "decode sweep: 401 packed linears of a 64-layer hidden-5120 model (48 linear-"
                               "attention + 16 full-attention layers, MLP 17408, lm_head 248320) + 1 embedding "
                               "row, batch 1: multi-module path (transform launch + persistent streaming "
                               "launch) and the embedding call", "modules": len(mods),
                   "weight_bytes": wbytes},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
        "detail": {"separate_calls_ms": round(sep_sec * 1e3, 4),
                   "separate_calls_GBps": round(wbytes / sep_sec / 1e9, 2),
                   "multi_vs_separate_worst_rel_l2": worst_multi,
                   "per_shape_separate_calls": per_shape, "parity_worst_rel_l2": worst, "parity": checked},
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
    ap.add_argument("--counters-only", action="store_true",
                    help="eager launches without timing, for rocprofv3 --pmc passes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.counters_only:
        run_counter_pass(args)
    elif args.workload == "copy":
        raise SystemExit("--workload copy is a counter-calibration pass: use it with --counters-only")
    elif args.workload == "prefill_gate_up":
        run_prefill(args)
    elif args.workload == "sweep":
        run_sweep(args)
    else:
        if args.workload == "down_proj" and args.batch is None:
            args.batch = 1
        run_gemv(args)


if __name__ == "__main__":
    main()
