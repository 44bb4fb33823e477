"""Seeded synthetic inputs for the Packed-linear path.

This module only draws random data; it holds none of the method's arithmetic
(no packing, no transform, no decoding).  Both the HIP library's tests and the
fp64 oracle consume exactly what it returns.

Distributions (the pages print no activation or scale statistics; the ternary
frequencies are the trained distribution quoted in trdm.cn/news/822023 section
2.3):

* sign vector: i.i.d. +-1 with probability 1/2 each, int8;
* ternary weight t in {-1, 0, 1} with p(-1) = p(1) = 0.38, p(0) = 0.24, int8;
* group scale: fp16(|N(0, 0.02)| + 1e-3), one per 128 weights of a row;
* activations: N(0, 1) as float32, rounded to bf16 (round-to-nearest-even)
  for the bf16 workloads.

Host draws use numpy's PCG64 (`numpy.random.default_rng(seed)`) in the fixed
order sign vector, ternary weights, scales, activations.  The full decode
sweep (25 G weights) is drawn on the device with torch's generator, module by
module, because a host draw of that size takes minutes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

P_NEG = 0.38
P_ZERO = 0.24
SCALE_STD = 0.02
SCALE_FLOOR = 1e-3
GROUP = 128
_CHUNK_ROWS = 1024


# ---------------------------------------------------------------------------
# elementary draws (host)
# ---------------------------------------------------------------------------
def draw_signs(rng: np.random.Generator, K: int) -> np.ndarray:
    return np.where(rng.random(K) < 0.5, -1, 1).astype(np.int8)


def draw_ternary(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    t = np.empty((N, K), dtype=np.int8)
    for r in range(0, N, _CHUNK_ROWS):
        u = rng.random((min(_CHUNK_ROWS, N - r), K))
        blk = np.ones(u.shape, dtype=np.int8)           # 1 where u >= P_NEG + P_ZERO
        blk[u < P_NEG + P_ZERO] = 0
        blk[u < P_NEG] = -1
        t[r:r + u.shape[0]] = blk
    return t


def draw_scales(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    s = np.abs(rng.normal(0.0, SCALE_STD, size=(N, K // GROUP))) + SCALE_FLOOR
    return s.astype(np.float16)


def draw_activations(rng: np.random.Generator, B: int, K: int, dtype: str):
    """Returns (values as float64 exactly, storage array).

    dtype "f32": storage float32.  dtype "bf16": storage uint16 bf16 bit
    patterns obtained by round-to-nearest-even of the float32 draw.
    """
    x = rng.standard_normal((B, K)).astype(np.float32)
    if dtype == "f32":
        return x.astype(np.float64), x
    if dtype == "bf16":
        import torch  # conversion only (RNE fp32 -> bf16)
        bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        return vals, bits.copy()
    raise ValueError(dtype)


@dataclass
class Problem:
    """One Packed-linear problem: raw draws before packing."""
    name: str
    N: int
    K: int
    B: int
    block: int
    xdtype: str
    signs: np.ndarray | None        # int8 (K,) or None (block 0)
    t: np.ndarray                   # int8 (N, K) ternary
    scales: np.ndarray              # float16 (N, K/128)
    x64: np.ndarray                 # float64 (B, K), exact values of x
    x_store: np.ndarray             # float32 or uint16 bf16 bits (B, K)
    meta: dict = field(default_factory=dict)


def make_problem(name: str, N: int, K: int, B: int, seed, xdtype: str = "bf16",
                 block: int = 1024) -> Problem:
    rng = np.random.default_rng(seed)
    sig = draw_signs(rng, K) if block else None
    t = draw_ternary(rng, N, K)
    sc = draw_scales(rng, N, K)
    x64, xs = draw_activations(rng, B, K, xdtype)
    return Problem(name, N, K, B, block, xdtype, sig, t, sc, x64, xs)


# ---------------------------------------------------------------------------
# the workloads (shapes from the pages: hidden 5120, MLP 17408, q 6144,
# k/v 1024, linear-attention qkv 10240 / z 6144, vocabulary 248320)
# ---------------------------------------------------------------------------
CONFIGS = {
    "tiny": dict(N=256, K=1024, B=1, seed=0, xdtype="f32"),
    "q_proj": dict(N=6144, K=5120, B=1, seed=2, xdtype="bf16"),
    "down_proj": dict(N=5120, K=17408, B=8, seed=3, xdtype="bf16"),
    "prefill_gate_up": dict(N=17408, K=5120, B=2048, seed=4, xdtype="bf16"),
}


def config_problem(name: str, B: int | None = None) -> Problem:
    """Draw a named workload.  For down_proj the activations are drawn as
    (8, K) and a batch of B uses the first B rows."""
    c = CONFIGS[name]
    p = make_problem(name, c["N"], c["K"], c["B"], c["seed"], c["xdtype"])
    if B is not None:
        if B > p.B:
            raise ValueError(f"{name}: batch {B} > drawn {p.B}")
        p.B = B
        p.x64 = p.x64[:B]
        p.x_store = p.x_store[:B]
    return p


# --- full decode sweep: 402 packed modules ---------------------------------
HIDDEN = 5120
N_LAYERS = 64
VOCAB = 248320


def sweep_modules():
    """The 401 packed linears plus the inverse-transform embedding of one
    decode token, in layer order.  Layer L is full attention iff L % 4 == 3
    (3:1 linear:full).  Each entry: (name, N_out, K_in, kind)."""
    mods = []
    for L in range(N_LAYERS):
        if L % 4 == 3:
            mods += [(f"layers.{L}.self_attn.q_proj", 6144, HIDDEN, "linear"),
                     (f"layers.{L}.self_attn.k_proj", 1024, HIDDEN, "linear"),
                     (f"layers.{L}.self_attn.v_proj", 1024, HIDDEN, "linear"),
                     (f"layers.{L}.self_attn.o_proj", HIDDEN, 6144, "linear")]
        else:
            mods += [(f"layers.{L}.linear_attn.in_proj_qkv", 10240, HIDDEN, "linear"),
                     (f"layers.{L}.linear_attn.in_proj_z", 6144, HIDDEN, "linear"),
                     (f"layers.{L}.linear_attn.out_proj", HIDDEN, 6144, "linear")]
        mods += [(f"layers.{L}.mlp.gate_proj", 17408, HIDDEN, "linear"),
                 (f"layers.{L}.mlp.up_proj", 17408, HIDDEN, "linear"),
                 (f"layers.{L}.mlp.down_proj", HIDDEN, 17408, "linear")]
    mods.append(("lm_head", VOCAB, HIDDEN, "linear"))
    mods.append(("embed_tokens", VOCAB, HIDDEN, "embedding"))
    return mods


SWEEP_SEED = 5


def sweep_signs():
    """One sign vector per input width (5120, 6144, 17408), shared by every
    module of that width, drawn on the host."""
    rng = np.random.default_rng(SWEEP_SEED)
    return {K: draw_signs(rng, K) for K in (5120, 6144, 17408)}


def sweep_input_sites():
    """Per sweep module, the index of the activation it reads, in the order
    of sweep_modules().  Modules of one layer that read the same hidden state
    share it, as a decode layer feeds them: q/k/v_proj (or in_proj_qkv and
    in_proj_z) read the attention input, o_proj (out_proj) the attention
    output, gate/up_proj the MLP input and down_proj the MLP's inner state;
    lm_head reads the final hidden state.  The embedding lookup reads none
    (-1)."""
    sites, index = [], {}
    for name, N, K, kind in sweep_modules():
        if kind != "linear":
            sites.append(-1)
            continue
        short = name.split(".")[-1]
        layer = name.split(".")[1] if name.startswith("layers.") else "final"
        role = {"q_proj": "attn_in", "k_proj": "attn_in", "v_proj": "attn_in", "in_proj_qkv": "attn_in",
                "in_proj_z": "attn_in", "o_proj": "attn_out", "out_proj": "attn_out", "gate_proj": "mlp_in",
                "up_proj": "mlp_in", "down_proj": "mlp_mid", "lm_head": "final"}[short]
        sites.append(index.setdefault((layer, role), len(index)))
    return sites


def device_site_x(site: int, K: int, device):
    """Activation of input site `site` of the sweep: (1, K) bf16, N(0, 1)
    rounded to nearest even, drawn on `device` with torch's generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(SWEEP_SEED * 1_000_003 + 700_001 + site)
    return torch.randn((1, K), generator=g, device=device).to(torch.bfloat16)


def device_module_draw(index: int, N: int, K: int, B: int, device):
    """Draw module `index` of the sweep on `device` with torch's generator:
    returns (t int8 (N,K), scales fp16 (N,K/128), x bf16 (B,K)) as tensors."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(SWEEP_SEED * 1_000_003 + index)
    t = torch.empty((N, K), dtype=torch.int8, device=device)
    step = max(1, (1 << 28) // K)
    for r in range(0, N, step):
        n = min(step, N - r)
        u = torch.rand((n, K), generator=g, device=device)
        blk = torch.ones((n, K), dtype=torch.int8, device=device)
        blk[u < P_NEG + P_ZERO] = 0
        blk[u < P_NEG] = -1
        t[r:r + n] = blk
        del u, blk
    sc = (torch.randn((N, K // GROUP), generator=g, device=device) * SCALE_STD).abs_() + SCALE_FLOOR
    sc = sc.to(torch.float16)
    x = torch.randn((B, K), generator=g, device=device).to(torch.bfloat16)
    return t, sc, x
