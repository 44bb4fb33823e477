"""The decode-sweep workload generator against the module inventory fixed in
tests/golden/sweep_inventory.json (counts, widths and head counts the pages
state, and the totals derived from them by hand there)."""
import json
import os
from collections import Counter

from hadamard_rotated_quantized_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sweep_inventory.json")


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_module_counts_and_kinds():
    g = _golden()
    mods = synth.sweep_modules()
    assert len(mods) == g["packed_modules"] == 402
    kinds = Counter(m[3] for m in mods)
    assert kinds["linear"] == g["linear_modules"]
    assert kinds["embedding"] == g["inverse_modules"]
    layers = {int(m[0].split(".")[1]) for m in mods if m[0].startswith("layers.")}
    assert layers == set(range(g["layers"]))
    full = {int(m[0].split(".")[1]) for m in mods if ".self_attn." in m[0]}
    lin = {int(m[0].split(".")[1]) for m in mods if ".linear_attn." in m[0]}
    assert len(full) == g["full_attention_layers"] and len(lin) == g["linear_attention_layers"]
    assert not (full & lin)


def test_every_module_has_the_golden_shape():
    g = _golden()["shapes_out_in"]
    mods = synth.sweep_modules()
    per_name = Counter()
    for name, N, K, kind in mods:
        short = name.split(".")[-1]
        assert [N, K] == g[short], name
        per_name[short] += 1
    assert per_name["down_proj"] == per_name["gate_proj"] == per_name["up_proj"] == 64
    assert per_name["q_proj"] == per_name["k_proj"] == per_name["v_proj"] == per_name["o_proj"] == 16
    assert per_name["in_proj_qkv"] == per_name["in_proj_z"] == per_name["out_proj"] == 48
    assert per_name["lm_head"] == per_name["embed_tokens"] == 1


def test_totals_and_sign_widths():
    g = _golden()
    mods = synth.sweep_modules()
    w = sum(N * K for _, N, K, kind in mods if kind == "linear")
    assert w == g["derived_totals"]["linear_weights"]
    assert w * 9 // 32 == g["derived_totals"]["linear_bytes_at_2_25_bpw"] == 7_057_981_440
    assert sorted({K for _, _, K, _ in mods}) == g["sign_widths"]
    assert sorted(synth.sweep_signs()) == g["sign_widths"]


def test_input_sites_follow_the_layer_structure():
    mods = synth.sweep_modules()
    sites = synth.sweep_input_sites()
    assert len(sites) == len(mods) and sites[-1] == -1
    by_site = {}
    for s, (name, N, K, kind) in zip(sites, mods):
        if s >= 0:
            by_site.setdefault(s, []).append((name.split(".")[-1], K))
    assert len(by_site) == 64 * 4 + 1
    groups = sorted(tuple(sorted(n for n, _ in v)) for v in by_site.values())
    assert groups.count(("in_proj_qkv", "in_proj_z")) == 48
    assert groups.count(("k_proj", "q_proj", "v_proj")) == 16
    assert groups.count(("gate_proj", "up_proj")) == 64
    assert groups.count(("down_proj",)) == 64 and groups.count(("lm_head",)) == 1
    assert all(len({K for _, K in v}) == 1 for v in by_site.values())
