"""Pins of the oracle's whole layer: special cases that reduce to dense
SwiGLU (a float64 matmul on dequantised operands), invariants of grouping and
permutation, and brute force on the tiny workload (CPU only)."""
import dataclasses
import itertools

import numpy as np

import coli_synth as cs
from layers import layer_inputs, oracle_layer, rel_l2


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def dense_expert(ref, ex, qx, dx, bits=4):
    """One expert on one Q8_0 token as dense float64 matmuls of dequantised operands."""
    H = qx.shape[0]
    I = ex["gate_s"].shape[0]
    xd = qx.astype(np.float64) * np.repeat(dx.astype(np.float64), 32)
    cg = ref.unpack(ex["gate_q"], H, bits).astype(np.float64)
    cu = ref.unpack(ex["up_q"], H, bits).astype(np.float64)
    cd = ref.unpack(ex["down_q"], I, bits).astype(np.float64)
    g = (ex["gate_s"].astype(np.float64) * (cg @ xd)).astype(np.float32)
    u = (ex["up_s"].astype(np.float64) * (cu @ xd)).astype(np.float32)
    g64 = g.astype(np.float64)
    h = (g64 / (1.0 + np.exp(-g64)) * u.astype(np.float64)).astype(np.float32)
    qh, dh = ref.quant_q8(h[None])
    hd = qh[0].astype(np.float64) * np.repeat(dh[0].astype(np.float64), 32)
    y = (ex["down_s"].astype(np.float64) * (cd @ hd)).astype(np.float32)
    return g, u, h, y


def test_single_expert_reduces_to_dense_swiglu(ref):
    cfg = dataclasses.replace(cs.CONFIGS[0], n_experts=4, top_k=1, n_shared=0)
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg)
    y, taps = L.forward(x, taps=True)
    np.testing.assert_array_equal(taps["w"], np.float32(cfg.rho))
    qx, dx = ref.quant_q8(x)
    for t in range(cfg.n_tok):
        e = int(taps["idx"][t, 0])
        g, u, h, ye = dense_expert(ref, L.experts[e], qx[t], dx[t])
        np.testing.assert_array_equal(taps["g"][t, 0], g)
        np.testing.assert_array_equal(taps["u"][t, 0], u)
        np.testing.assert_array_equal(taps["h"][t, 0], h)
        want = (np.float64(cfg.rho) * ye.astype(np.float64)).astype(np.float32)
        assert rel_l2(y[t], want) < 1e-12


def test_zero_routed_experts_leave_shared(ref):
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg)
    H, I = cfg.hidden, cfg.inter
    zero = ref.pack_expert(np.zeros((I, H), np.float32), np.zeros((I, H), np.float32),
                           np.zeros((H, I), np.float32))
    for e in range(cfg.n_experts):
        L.add_expert(e, zero)
    y, taps = L.forward(x, taps=True)
    qx, dx = ref.quant_q8(x)
    for t in range(cfg.n_tok):
        _, _, _, ys = dense_expert(ref, L.experts[cfg.n_experts], qx[t], dx[t])
        np.testing.assert_array_equal(y[t], ys)
        np.testing.assert_array_equal(taps["ye"][t, cfg.top_k], ys)


def test_grouped_equals_per_token(ref):
    cfg = cs.with_tokens(cs.CONFIGS[0], 12)
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg)
    y = L.forward(x)
    for t in range(cfg.n_tok):
        np.testing.assert_array_equal(L.forward(x[t:t + 1])[0], y[t])


def test_token_permutation_permutes_outputs(ref):
    cfg = cs.with_tokens(cs.CONFIGS[0], 10)
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg)
    y = L.forward(x)
    perm = np.random.RandomState(6).permutation(cfg.n_tok)
    np.testing.assert_array_equal(L.forward(x[perm]), y[perm])


def test_forced_routing_and_accumulate(ref):
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg)
    y, taps = L.forward(x, taps=True)
    y2 = L.forward(x, forced_idx=taps["idx"], forced_w=taps["w"])
    np.testing.assert_array_equal(y, y2)
    base = np.random.RandomState(7).standard_normal(y.shape).astype(np.float32)
    y3 = L.forward(x, y_in=base)
    np.testing.assert_array_equal(y3, base + y)


def test_brute_force_tiny_layer(ref):
    """Whole tiny layer from independent pieces: float64 matmul logits, subset
    enumeration for the top-k, dense SwiGLU experts, float64 combine."""
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg)
    y = L.forward(x)
    qx, dx = ref.quant_q8(x)
    logits = x.astype(np.float64) @ wr.astype(np.float64).T
    for t in range(cfg.n_tok):
        s = _sig(logits[t])
        c = s + b.astype(np.float64)
        best = max(itertools.combinations(range(cfg.n_experts), cfg.top_k),
                   key=lambda S: sum(c[list(S)]))
        best = sorted(best, key=lambda e: (-c[e], e))
        wts = (cfg.rho * s[best] / s[best].sum()).astype(np.float32)
        acc = np.zeros(cfg.hidden)
        for e, wk in zip(best, wts):
            acc += np.float64(wk) * dense_expert(ref, L.experts[e], qx[t], dx[t])[3]
        acc += dense_expert(ref, L.experts[cfg.n_experts], qx[t], dx[t])[3]
        assert rel_l2(y[t], acc.astype(np.float32)) < 1e-9


def test_rmsnorm_closed_form(ref):
    rng = np.random.RandomState(8)
    x = (rng.standard_normal((3, 256)) * 3).astype(np.float32)
    out = ref.rmsnorm(x, 1e-5)
    rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(out, (x / rms).astype(np.float32), rtol=1e-7)
    # unit gain: mean square of the output is 1 up to eps
    ms = (out.astype(np.float64) ** 2).mean(axis=1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-5)
    np.testing.assert_array_equal(ref.rmsnorm(np.zeros((1, 64), np.float32)), 0.0)
