"""Helpers for the GPU tests: move a synthetic problem to the device through
the library's own packer, compute the oracle through the oracle's own packer,
and compare under the parity bar (relative L2 <= 1e-4, max |err| <= 1e-3 max |y|)."""
from __future__ import annotations

import numpy as np

import hadamard_rotated_quantized_amd as tb
import oracle

REL_L2 = 1e-4
MAX_ABS = 1e-3


def torch():
    import torch as _t
    return _t


def cuda_available():
    try:
        return torch().cuda.is_available()
    except Exception:
        return False


def x_to_device(p):
    T = torch()
    if p.xdtype == "f32":
        return T.from_numpy(np.ascontiguousarray(p.x_store)).cuda()
    return T.from_numpy(np.ascontiguousarray(p.x_store).view(np.int16)).view(T.bfloat16).cuda()


def pack_to_device(t, scales):
    """Pack with the library's host packer and upload (codes as int32 words)."""
    T = torch()
    codes, s, b = tb.tb_pack(t, scales)
    return (T.from_numpy(codes.view(np.int32)).cuda(), T.from_numpy(s.view(np.float16)).cuda(),
            T.from_numpy(b.view(np.float16)).cuda())


def signs_to_device(signs):
    if signs is None:
        return None
    return torch().from_numpy(np.ascontiguousarray(signs)).cuda()


def oracle_pack(p):
    return oracle.pack(p.t, p.scales)


def compare(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = got - want
    nw = np.linalg.norm(want)
    rel = np.linalg.norm(err) / nw if nw > 0 else np.linalg.norm(err)
    mw = np.abs(want).max()
    mabs = np.abs(err).max() / mw if mw > 0 else np.abs(err).max()
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert mabs <= MAX_ABS, f"{what}: max abs error {mabs:.3e} of max|y| > {MAX_ABS}"
    return rel, mabs


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
