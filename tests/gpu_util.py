"""GPU-test helpers: device layers packed by the library, oracle layers packed
by the oracle from the same seeded fp32 draws, and layout conversions."""
from __future__ import annotations

import numpy as np
import torch

import coli_synth as cs


def unperm8(q: np.ndarray) -> np.ndarray:
    """Undo the library's 8-group order (e0,e2,e4,e6,e1,e3,e5,e7) along the last axis."""
    q = np.asarray(q)
    g = q.reshape(*q.shape[:-1], -1, 2, 4)          # [..., groups, (evens, odds), 4]
    out = np.stack([g[..., 0, :], g[..., 1, :]], axis=-1)  # [..., groups, 4, 2]
    return out.reshape(q.shape)


def unperm16(q: np.ndarray) -> np.ndarray:
    """Undo the int2 weights' 16-group order (e0,e4,e8,e12,e1,...,e15) along the last axis."""
    q = np.asarray(q)
    g = q.reshape(*q.shape[:-1], -1, 4, 4)          # [..., groups, a, b] holds element 4b + a
    return np.swapaxes(g, -1, -2).reshape(q.shape)


def unperm_for(bits):
    return {4: unperm8, 8: lambda q: np.asarray(q), 2: unperm16}[bits]


def lib_cfg(C, cfg, n_group=1, topk_group=1, bits=4):
    return C.make_cfg(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                      cfg.norm_topk, cfg.rho, n_group, topk_group, bits)


def gpu_layer(C, cfg, layer=0):
    """LayerWeights on cuda:0, every matrix packed by coli_pack_int4."""
    wr, b, q, s = cs.build_layer(cfg, layer, "cuda", lambda w, qv, sv: C.coli_pack_int4(w, qv, sv))
    return C.LayerWeights(lib_cfg(C, cfg), wr, b, q, s)


def layer_input(ref, cfg, layer=0, n_tok=None, first_tok=0):
    """Layer input on the host: the raw draw, RMS-normalised by the oracle when
    the workload says the input is normalised."""
    x = cs.activations(cfg, layer, "cpu", n_tok=n_tok, first_tok=first_tok).numpy()
    if cfg.rmsnorm_input:
        x = ref.rmsnorm(x, np.float32(1e-5))
    return np.ascontiguousarray(x, np.float32)


def oracle_layer_for(ref, cfg, layer, x, forced_idx=None, draw_device="cuda", n_group=1,
                     topk_group=1, bits=4):
    """OracleLayer holding only the experts that tokens x select (plus shared),
    each drawn as fp32 by coli_synth (on draw_device, bit-identical to the CPU
    draw) and packed by the oracle."""
    wr, b = cs.router(cfg, layer, "cpu")
    wr, b = wr.numpy(), b.numpy()
    if forced_idx is None:
        idx, _, _ = ref.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho, n_group, topk_group)
    else:
        idx = forced_idx
    need = sorted(set(int(e) for e in np.unique(idx)) | ({cfg.n_experts} if cfg.n_shared else set()))
    L = ref.OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                        cfg.norm_topk, cfg.rho, wr, b, {}, n_group, topk_group, bits)
    for e in need:
        mats = [cs.expert_matrix(cfg, layer, e, w, draw_device).cpu().numpy()
                for w in ("gate", "up", "down")]
        L.add_expert(e, ref.pack_expert(*mats, bits=bits))
    return L


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


TIE_TOL = 1e-6


def check_routing(ref, cfg, x, wr, b, gidx, gw, tol=TIE_TOL):
    """Router parity of the GPU's choice (gidx, gw) for the token rows x.

    Per token the index list equals the oracle's and the gate weights agree
    within 1e-6 relative; or the GPU took another correct choice: distinct
    experts in descending order of the oracle's selection score c = s + b
    (neighbours within `tol` in either order), every expert in one list but
    not the other with c within `tol` of the K-th largest c (the near-tie the
    parity bar allows), and gate weights equal to the oracle's gate values for
    that choice. Plain top-k only (no expert groups).

    Returns (rows that took another correct choice, the oracle's gate values
    for the GPU's choice, [rows, K])."""
    K = cfg.top_k
    x = np.ascontiguousarray(x, np.float32)
    gidx = np.ascontiguousarray(gidx, np.int32)
    ridx, rw, logits = ref.route(x, wr, b, K, cfg.norm_topk, cfg.rho)
    c = 1.0 / (1.0 + np.exp(-logits)) + np.asarray(b, np.float64)
    assert all(len(set(int(e) for e in row)) == K for row in gidx), "repeated expert"
    w_for = ref.gates(x, wr, b, gidx, cfg.norm_topk, cfg.rho)
    swaps = []
    for t in range(x.shape[0]):
        if list(gidx[t]) == list(ridx[t]):
            np.testing.assert_allclose(gw[t], rw[t], rtol=1e-6)
            continue
        ct = c[t]
        kth = np.sort(ct)[::-1][K - 1]
        diff = set(int(e) for e in gidx[t]) ^ set(int(e) for e in ridx[t])
        assert all(abs(ct[e] - kth) <= tol for e in diff), \
            (t, list(gidx[t]), list(ridx[t]), [float(ct[e] - kth) for e in diff])
        assert all(ct[gidx[t][k]] >= ct[gidx[t][k + 1]] - tol for k in range(K - 1)), \
            (t, list(gidx[t]), "not in descending score order")
        np.testing.assert_allclose(gw[t], w_for[t], rtol=1e-6)
        swaps.append(t)
    return swaps, w_for


def add_missing_experts(ref, cfg, layer, OL, ids, draw_device="cuda", bits=4):
    """Add (oracle-packed, from coli_synth's fp32 draw) the experts of ids that
    OL does not hold yet."""
    for e in sorted(set(int(v) for v in np.unique(ids)) - set(OL.experts)):
        mats = [cs.expert_matrix(cfg, layer, e, w, draw_device).cpu().numpy()
                for w in ("gate", "up", "down")]
        OL.add_expert(e, ref.pack_expert(*mats, bits=bits))
