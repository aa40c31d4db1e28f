"""Pins of the oracle's int8 and int2 weight formats (CPU only): hand-worked
codes and bytes, round-trip bounds, the most negative code, brute-force block
dots, and whole-layer reductions to dense SwiGLU on dequantised operands."""
import dataclasses
import itertools
import json
import os

import numpy as np
import pytest

import coli_synth as cs
from layers import layer_inputs, oracle_layer, rel_l2
from test_oracle_layer import dense_expert

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_bits_hand.json")


@pytest.mark.parametrize("i", range(3))
def test_pack_hand_cases(ref, i):
    case = json.load(open(GOLDEN))["cases"][i]
    bits, s = case["bits"], np.float32(case["scale"])
    w = (np.asarray(case["row_over_scale"], np.float32) * s)[None]
    q, sc = ref.pack_weights(w, bits)
    assert sc[0] == s
    assert [f"0x{b:02x}" for b in q[0]] == case["bytes"], case["name"]
    np.testing.assert_array_equal(ref.unpack(q, w.shape[1], bits)[0], case["codes"])


@pytest.mark.parametrize("bits", [2, 8])
def test_roundtrip_bound(ref, bits):
    rng = np.random.RandomState(bits)
    w = (rng.standard_normal((37, 256)) * rng.uniform(0.01, 3.0, (37, 1))).astype(np.float32)
    w[5] = 0.0
    q, s = ref.pack_weights(w, bits)
    c = ref.unpack(q, 256, bits)
    qmax = (1 << (bits - 1)) - 1
    assert np.abs(c).max() <= qmax
    err = np.abs(c.astype(np.float64) * s[:, None].astype(np.float64) - w.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-6))
    assert s[5] == 0.0 and np.all(c[5] == 0)
    # the largest magnitude of every row maps to +-qmax
    am = np.argmax(np.abs(w), axis=1)
    assert np.all(np.abs(c[np.arange(37), am])[np.arange(37) != 5] == qmax)


def test_most_negative_codes_decode(ref):
    # int8 0x80 -> -128; int2 0b10 -> -2 (never produced by the packer)
    assert ref.unpack(np.array([[0x80] * 4], np.uint8), 4, 8)[0, 0] == -128
    np.testing.assert_array_equal(ref.unpack(np.array([[0b10011110]], np.uint8), 4, 2)[0],
                                  [-2, -1, 1, -2])


@pytest.mark.parametrize("bits", [2, 8])
def test_block_dots_brute_force(ref, bits):
    rng = np.random.RandomState(3 + bits)
    w = rng.standard_normal((5, 96)).astype(np.float32)
    q, _ = ref.pack_weights(w, bits)
    qx = rng.randint(-127, 128, size=(3, 96)).astype(np.int8)
    dots = ref.block_dots(q, 96, qx, bits)
    c = ref.unpack(q, 96, bits).astype(np.int64)
    for t in range(3):
        for r in range(5):
            for b in range(3):
                want = int(np.dot(c[r, 32 * b:32 * b + 32], qx[t, 32 * b:32 * b + 32].astype(np.int64)))
                assert dots[t, r, b] == want


@pytest.mark.parametrize("bits", [2, 8])
def test_single_expert_reduces_to_dense_swiglu(ref, bits):
    cfg = dataclasses.replace(cs.CONFIGS[0], n_experts=4, top_k=1, n_shared=0)
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg, bits=bits)
    y, taps = L.forward(x, taps=True)
    qx, dx = ref.quant_q8(x)
    for t in range(cfg.n_tok):
        e = int(taps["idx"][t, 0])
        g, u, h, ye = dense_expert(ref, L.experts[e], qx[t], dx[t], bits)
        np.testing.assert_array_equal(taps["g"][t, 0], g)
        np.testing.assert_array_equal(taps["u"][t, 0], u)
        np.testing.assert_array_equal(taps["h"][t, 0], h)
        want = (np.float64(cfg.rho) * ye.astype(np.float64)).astype(np.float32)
        assert rel_l2(y[t], want) < 1e-12


@pytest.mark.parametrize("bits", [2, 8])
def test_brute_force_tiny_layer(ref, bits):
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg)
    L = oracle_layer(ref, cfg, bits=bits)
    y = L.forward(x)
    qx, dx = ref.quant_q8(x)
    logits = x.astype(np.float64) @ wr.astype(np.float64).T
    for t in range(cfg.n_tok):
        s = 1.0 / (1.0 + np.exp(-logits[t]))
        c = s + b.astype(np.float64)
        best = max(itertools.combinations(range(cfg.n_experts), cfg.top_k),
                   key=lambda S: sum(c[list(S)]))
        best = sorted(best, key=lambda e: (-c[e], e))
        wts = (cfg.rho * s[best] / s[best].sum()).astype(np.float32)
        acc = np.zeros(cfg.hidden)
        for e, wk in zip(best, wts):
            acc += np.float64(wk) * dense_expert(ref, L.experts[e], qx[t], dx[t], bits)[3]
        acc += dense_expert(ref, L.experts[cfg.n_experts], qx[t], dx[t], bits)[3]
        assert rel_l2(y[t], acc.astype(np.float32)) < 1e-9


def test_error_against_fp32_shrinks_with_width(ref):
    """Against the unquantised fp32 weights (dense float64 SwiGLU), the layer
    error falls as the codes widen: int2 > int4 > int8 (a swapped range or
    scale for one width would break the order)."""
    from layers import expert_fp32
    cfg = dataclasses.replace(cs.CONFIGS[0], n_experts=4, top_k=1, n_shared=0)
    x, _, _ = layer_inputs(cfg)
    errs = {}
    for bits in (2, 4, 8):
        L = oracle_layer(ref, cfg, bits=bits)
        y, taps = L.forward(x, taps=True)
        want = np.zeros_like(y, dtype=np.float64)
        for t in range(cfg.n_tok):
            gw, uw, dw = (m.astype(np.float64) for m in expert_fp32(cfg, 0, int(taps["idx"][t, 0])))
            xt = x[t].astype(np.float64)
            g, u = gw @ xt, uw @ xt
            want[t] = cfg.rho * (dw @ (g / (1.0 + np.exp(-g)) * u))
        errs[bits] = rel_l2(y, want)
    assert errs[8] < errs[4] < errs[2], errs


def test_rejects_bad_widths(ref):
    with pytest.raises(ValueError):
        ref.pack_weights(np.zeros((1, 32), np.float32), 3)
    with pytest.raises(ValueError):
        ref.pack_weights(np.zeros((1, 6), np.float32), 2)  # 6 x 2 bits is not whole bytes
