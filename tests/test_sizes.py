"""Byte counts of the expert format against the sizes the pages print."""
import json
import os

import coli_synth as cs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sizes.json")


def test_expert_and_per_token_bytes_match_pages():
    g = json.load(open(GOLD))
    cfg = cs.CONFIGS[1]
    assert (cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k) == \
        (g["hidden"], g["inter"], g["n_experts"], g["top_k"])
    eb = cfg.expert_bytes()
    assert eb == 18_915_328
    assert abs(eb / 1e6 - g["expert_mb_approx"]) < 0.5              # "about 19 MB"
    per_tok = g["moe_layers_reading"] * cfg.top_k * eb
    assert abs(per_tok / 1e9 - g["gb_per_token_approx"]) < 0.5       # "about 11 GB / token"
    disk = g["moe_layers_reading"] * (cfg.n_experts + 1) * eb + 0    # routed + shared per layer
    assert abs(disk / 1e9 - g["disk_gb_approx"]) / g["disk_gb_approx"] < 0.05
