"""Test helpers: build seeded layers for the oracle (CPU) from coli_synth recipes."""
from __future__ import annotations

import numpy as np

import coli_synth as cs


def expert_fp32(cfg, layer, e):
    return (cs.expert_matrix(cfg, layer, e, "gate").numpy(),
            cs.expert_matrix(cfg, layer, e, "up").numpy(),
            cs.expert_matrix(cfg, layer, e, "down").numpy())


def layer_inputs(cfg, layer=0, n_tok=None, first_tok=0):
    """Raw activations (before any RMSNorm), router weight and bias as numpy."""
    x = cs.activations(cfg, layer, "cpu", n_tok=n_tok, first_tok=first_tok).numpy()
    wr, b = cs.router(cfg, layer, "cpu")
    return x, wr.numpy(), b.numpy()


def oracle_layer(ref, cfg, layer=0, experts=None, wr=None, b=None, bits=4):
    """OracleLayer with the given experts packed by the oracle (all when None)
    with bits-wide weight codes."""
    if wr is None:
        wr_t, b_t = cs.router(cfg, layer, "cpu")
        wr, b = wr_t.numpy(), b_t.numpy()
    L = ref.OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                        cfg.norm_topk, cfg.rho, wr, b, {}, weight_bits=bits)
    ids = range(cfg.n_experts + cfg.n_shared) if experts is None else experts
    for e in ids:
        L.add_expert(e, ref.pack_expert(*expert_fp32(cfg, layer, e), bits=bits))
    return L


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
