"""Pins of the oracle's int4 packing and Q8_0 quantisation (CPU only)."""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("pack_int4_hand.json")["cases"], ids=lambda c: c["name"])
def test_pack_hand_cases(ref, case):
    s = np.float32(case["scale"])
    row = (np.array(case["row_over_scale"], np.float32) * s)[None]
    q, sc = ref.pack_int4(row)
    assert sc[0] == np.float32(case["scale"])
    assert [int(v) for v in ref.unpack_int4(q, row.shape[1])[0]] == case["codes"]
    assert [int(b, 16) for b in case["bytes"]] == [int(v) for v in q[0]]


def test_pack_roundtrip_bound(ref):
    rng = np.random.RandomState(1)
    w = (rng.standard_normal((64, 256)) * rng.uniform(1e-3, 10, (64, 1))).astype(np.float32)
    w[3] = 0.0
    w[5, :] = 1e-30
    q, s = ref.pack_int4(w)
    codes = ref.unpack_int4(q, 256).astype(np.float64)
    s64 = s.astype(np.float64)[:, None]
    err = np.abs(w - codes * s64)
    # |w - s q| <= s/2, plus slack for the fp32 rounding of s and of w/s
    assert np.all(err <= s64 * (0.5 + 1e-6) + 1e-45)
    amax = np.abs(w).max(axis=1)
    np.testing.assert_array_equal(s, (amax / np.float32(7)).astype(np.float32))
    # the largest magnitude of each non-zero row lands on +-7, never -8
    nz = amax > 0
    assert np.all(np.abs(codes[nz]).max(axis=1) == 7)
    assert codes.min() >= -7 and codes.max() <= 7
    assert np.all(q[3] == 0) and s[3] == 0


def test_unpack_decodes_minus_eight(ref):
    q = np.array([[0x88, 0x7F]], np.uint8)
    assert list(ref.unpack_int4(q, 4)[0]) == [-8, -8, -1, 7]


@pytest.mark.parametrize("case", _load("quant_q8_hand.json")["cases"], ids=lambda c: c["name"])
def test_q8_hand_cases(ref, case):
    x = np.array(case["block"], np.float32)
    q, d = ref.quant_q8(x[None])
    assert d[0, 0] == np.float32(case["d"])
    assert [int(v) for v in q[0]] == case["q"]


def test_q8_roundtrip_bound_and_zero_block(ref):
    rng = np.random.RandomState(2)
    x = (rng.standard_normal((5, 320)) * rng.uniform(1e-4, 50, (5, 1))).astype(np.float32)
    x[1, 32:64] = 0.0
    q, d = ref.quant_q8(x)
    dd = np.repeat(d.astype(np.float64), 32, axis=1)
    err = np.abs(x - q.astype(np.float64) * dd)
    assert np.all(err <= dd * (0.5 + 1e-6))
    assert d[1, 1] == 0 and np.all(q[1, 32:64] == 0)
    blocks = np.abs(x.reshape(5, 10, 32)).max(axis=2)
    np.testing.assert_array_equal(d, (blocks / np.float32(127)).astype(np.float32))
    assert np.all(np.abs(q.reshape(5, 10, 32)).max(axis=2)[d > 0] == 127)


def test_block_dots_brute_force(ref):
    rng = np.random.RandomState(3)
    w = rng.standard_normal((6, 96)).astype(np.float32)
    x = rng.standard_normal((2, 96)).astype(np.float32)
    wq, _ = ref.pack_int4(w)
    codes = ref.unpack_int4(wq, 96).astype(np.int64)
    qx, _ = ref.quant_q8(x)
    dots = ref.block_dots(wq, 96, qx)
    for t in range(2):
        for r in range(6):
            for b in range(3):
                exp = sum(int(codes[r, 32 * b + i]) * int(qx[t, 32 * b + i]) for i in range(32))
                assert dots[t, r, b] == exp
