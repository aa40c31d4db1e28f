"""Pins of the oracle's group-limited expert selection (CPU only).

Hand-worked cases (tests/golden/route_groups_hand.json) fix the reading:
group score = sum of the two largest biased scores, ties to the lower group,
groups ranked by the biased score. Reductions: one group, or keeping every
group, is the plain selection; and keeping some groups equals the plain
selection with the other groups' experts pushed out by their bias.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_groups_hand.json")


def _identity_route(ref, case, grouped=True):
    l = np.asarray(case["logits"], np.float32)[None]
    E = l.shape[1]
    wr = np.eye(E, dtype=np.float32)  # logits = x exactly
    b = np.asarray(case["bias"], np.float32)
    if grouped:
        return ref.route(l, wr, b, case["top_k"], True, case["rho"], case["n_group"],
                         case["topk_group"])
    return ref.route(l, wr, b, case["top_k"], True, case["rho"])


@pytest.mark.parametrize("i", range(3))
def test_hand_worked_cases(ref, i):
    case = json.load(open(GOLDEN))["cases"][i]
    idx, w, _ = _identity_route(ref, case)
    assert list(idx[0]) == case["idx"], case["name"]
    np.testing.assert_array_equal(w[0], np.asarray(case["w"], np.float32))
    idx0, _, _ = _identity_route(ref, case, grouped=False)
    assert list(idx0[0]) == case["ungrouped_idx"]


def _inputs(seed, T, H, E):
    rng = np.random.RandomState(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.02).astype(np.float32)
    return x, wr, b


@pytest.mark.parametrize("n_group", [1, 4, 8])
def test_keeping_every_group_is_plain_selection(ref, n_group):
    x, wr, b = _inputs(1, 16, 64, 64)
    plain = ref.route(x, wr, b, 6, True, 2.5)
    grouped = ref.route(x, wr, b, 6, True, 2.5, n_group, n_group)
    np.testing.assert_array_equal(grouped[0], plain[0])
    np.testing.assert_array_equal(grouped[1], plain[1])


@pytest.mark.parametrize("E,G,TG,K", [(256, 8, 4, 8), (64, 16, 3, 5), (48, 48, 10, 4)])
def test_equals_plain_selection_inside_kept_groups(ref, E, G, TG, K):
    T = 24
    x, wr, b = _inputs(E + G, T, 96, E)
    idx, w, logits = ref.route(x, wr, b, K, True, 2.5, G, TG)
    gs = E // G
    c = 1.0 / (1.0 + np.exp(-logits)) + b.astype(np.float64)
    for t in range(T):
        cg = np.sort(c[t].reshape(G, gs), axis=1)[:, ::-1]
        score = cg[:, 0] + (cg[:, 1] if gs > 1 else 0.0)
        kept = np.argsort(-score, kind="stable")[:TG]  # stable: ties to the lower group
        assert {int(e) // gs for e in idx[t]} <= set(kept.tolist())
        # the plain selection with every other expert pushed out by its bias
        b2 = b.copy()
        mask = np.ones(E, bool)
        for g in kept:
            mask[g * gs:(g + 1) * gs] = False
        b2[mask] = -100.0
        i2, w2, _ = ref.route(x[t:t + 1], wr, b2, K, True, 2.5)
        np.testing.assert_array_equal(idx[t], i2[0])
        np.testing.assert_array_equal(w[t], w2[0])


def test_rejects_bad_groups(ref):
    x, wr, b = _inputs(2, 1, 32, 12)
    for G, TG, K in [(5, 1, 2), (4, 0, 2), (4, 5, 2), (4, 1, 4)]:
        with pytest.raises(ValueError):
            ref.route(x, wr, b, K, True, 2.5, G, TG)
