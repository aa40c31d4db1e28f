"""Pins of the oracle's sigmoid router (CPU only)."""
import itertools

import numpy as np
import pytest

import coli_synth as cs
from layers import layer_inputs


def _sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def test_weights_sum_to_rho(ref):
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg, n_tok=64)
    idx, w, _ = ref.route(x, wr, b, cfg.top_k, True, cfg.rho)
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), cfg.rho, rtol=1e-6)
    assert np.all(w > 0)


def test_zero_bias_no_norm_is_argsort_of_logits(ref):
    # with b = 0 and no normalisation the choice is the K largest logits
    # (sigmoid is increasing) and w = rho * sigmoid(logit)
    rng = np.random.RandomState(4)
    T, H, E, K = 32, 128, 24, 5
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    idx, w, logits = ref.route(x, wr, np.zeros(E, np.float32), K, False, 2.5)
    lg = x.astype(np.float64) @ wr.astype(np.float64).T
    np.testing.assert_allclose(logits, lg, rtol=1e-12, atol=1e-12)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :K]
    np.testing.assert_array_equal(idx, order)
    np.testing.assert_allclose(w, (2.5 * _sig(np.take_along_axis(lg, order, 1))).astype(np.float32),
                               rtol=1e-7)


def test_brute_force_subsets_tiny_config(ref):
    # the chosen set is the unique K-subset maximising sum(c); order is descending c
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg)
    idx, w, logits = ref.route(x, wr, b, cfg.top_k, True, cfg.rho)
    for t in range(cfg.n_tok):
        c = _sig(logits[t]) + b.astype(np.float64)
        best = max(itertools.combinations(range(cfg.n_experts), cfg.top_k),
                   key=lambda s: sum(c[list(s)]))
        assert set(idx[t]) == set(best)
        assert all(c[idx[t][k]] >= c[idx[t][k + 1]] for k in range(cfg.top_k - 1))
        s = _sig(logits[t][idx[t]])
        np.testing.assert_allclose(w[t], (cfg.rho * s / s.sum()).astype(np.float32), rtol=1e-7)


def test_bias_steers_selection_but_not_weight(ref):
    rng = np.random.RandomState(5)
    H, E, K = 64, 12, 3
    x = rng.standard_normal((1, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    lg = (x.astype(np.float64) @ wr.astype(np.float64).T)[0]
    loser = int(np.argmin(lg))
    b = np.zeros(E, np.float32)
    b[loser] = 10.0
    idx, w, _ = ref.route(x, wr, b, K, True, 1.0)
    assert idx[0, 0] == loser
    s = _sig(lg[idx[0]])
    np.testing.assert_allclose(w[0], (s / s.sum()).astype(np.float32), rtol=1e-7)
    # a plausible mistake (biased score as gate value) would give ~1 for the loser
    assert w[0, 0] < 0.5


def test_ties_go_to_lower_index(ref):
    H, E, K = 32, 8, 3
    x = np.ones((1, H), np.float32)
    wr = np.zeros((E, H), np.float32)
    wr[[2, 5, 6]] = 0.1    # three identical top rows
    idx, w, _ = ref.route(x, wr, np.zeros(E, np.float32), K, True, 2.5)
    assert list(idx[0]) == [2, 5, 6]
    wr[[1, 3]] = 0.05      # identical runners-up, only one fits
    idx, _, _ = ref.route(x, wr, np.zeros(E, np.float32), 4, True, 2.5)
    assert list(idx[0]) == [2, 5, 6, 1]


def test_rejects_bad_k(ref):
    with pytest.raises(ValueError):
        ref.route(np.zeros((1, 32), np.float32), np.zeros((4, 32), np.float32),
                  np.zeros(4, np.float32), 5)


def test_gates_of_the_router_choice_equal_its_weights(ref):
    # invariant: the gate values the oracle gives its own choice are the
    # router's weights, bit for bit, normalised and not
    cfg = cs.CONFIGS[0]
    x, wr, b = layer_inputs(cfg, n_tok=32)
    for norm in (True, False):
        idx, w, _ = ref.route(x, wr, b, cfg.top_k, norm, cfg.rho)
        np.testing.assert_array_equal(ref.gates(x, wr, b, idx, norm, cfg.rho), w)


def test_gates_of_another_choice(ref):
    # closed form on any set of distinct experts, in any order: w_k =
    # rho * s_k / sum s (k ascending) with s the sigmoid of the logits; the
    # values follow the order of the given indices
    rng = np.random.RandomState(12)
    T, H, E, K = 16, 64, 20, 4
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(E) * 0.01).astype(np.float32)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    lg = x.astype(np.float64) @ wr.astype(np.float64).T
    s = np.take_along_axis(_sig(lg), idx.astype(np.int64), 1)
    want = (2.5 * s / s.sum(axis=1, keepdims=True)).astype(np.float32)
    got = ref.gates(x, wr, b, idx, True, 2.5)
    np.testing.assert_allclose(got, want, rtol=2e-7)
    np.testing.assert_allclose(got.astype(np.float64).sum(1), 2.5, rtol=1e-6)
    # the bias plays no part in the gate value
    np.testing.assert_array_equal(ref.gates(x, wr, np.zeros(E, np.float32), idx, True, 2.5), got)
    rev = np.ascontiguousarray(idx[:, ::-1])
    np.testing.assert_allclose(ref.gates(x, wr, b, rev, True, 2.5), got[:, ::-1], rtol=2e-7)
    with pytest.raises(ValueError):
        bad = idx.copy()
        bad[0, 1] = bad[0, 0]
        ref.gates(x, wr, b, bad, True, 2.5)
