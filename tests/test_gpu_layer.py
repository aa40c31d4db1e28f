"""GPU parity of the whole layer (coli_moe_forward) against the oracle.

Checks, per workload:
  Q8_0 codes of x bit-exact; per-block int32 dots of gate rows bit-exact
  (debug tap); router index sets equal (ties within 1e-6 tolerated) and gate
  weights within 1e-6; q_h codes equal (0 flips expected); layer output within
  1e-4 relative L2 (observed ~1e-7). The full-size workloads run every token
  on the GPU and compare the tokens the oracle evaluates (per-token and
  batched oracle evaluation are identical, an invariant pinned on the CPU).
"""
import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import (add_missing_experts, check_routing, gpu_layer, layer_input, lib_cfg,
                      oracle_layer_for, rel_l2, unperm8)

pytestmark = pytest.mark.gpu

TOL_REL_L2 = 1e-4


@pytest.fixture(scope="module")
def C():
    import int4_quantized_moe_sigmoid_amd as C
    assert torch.cuda.is_available()
    return C


_LAYERS = {}


def _layer(C, cfg, layer=0):
    key = (cfg.seed, cfg.hidden, cfg.n_experts, cfg.inter, cfg.bias_kind, layer)
    if key not in _LAYERS:
        _LAYERS.clear()            # keep one full-size layer resident at a time
        torch.cuda.empty_cache()
        _LAYERS[key] = gpu_layer(C, cfg, layer)
    return _LAYERS[key]


def run_gpu(C, W, x, flags=0, y_in=None, taps=True):
    """The layer on the GPU. With taps (COLI_FWD_DEBUG_TAPS) returns (y, the
    intermediates read back from the workspace); else (y, None): the kernels
    without the debug stores, the ones the bench times."""
    T = x.shape[0]
    lc = W.cfg
    fl = flags | (C.COLI_FWD_DEBUG_TAPS if taps else 0)
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T, fl), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(x).cuda()
    y = torch.from_numpy(y_in).cuda() if y_in is not None else \
        torch.empty((T, lc.hidden), dtype=torch.float32, device="cuda")
    C.coli_moe_forward(W, xd, y, ws, fl)
    torch.cuda.synchronize()
    if not taps:
        return y.cpu().numpy(), None
    L = C.coli_moe_workspace_layout(lc, T, fl)
    wsn = ws.cpu().numpy()
    H, I, K, S = lc.hidden, lc.inter, lc.top_k, lc.n_shared

    def arr(off, dtype, shape):
        n = int(np.prod(shape))
        return np.frombuffer(wsn[off:off + n * np.dtype(dtype).itemsize].tobytes(),
                             dtype=dtype).reshape(shape)
    NS = int(L.n_slots)
    taps = {
        "qx": unperm8(arr(L.qx, np.int8, (T, H))), "dx": arr(L.dx, np.float32, (T, H // 32)),
        "idx": arr(L.topk_idx, np.int32, (T, K)), "w": arr(L.topk_w, np.float32, (T, K)),
        "slot_of": arr(L.slot_of, np.int32, (T, K + S)),
        "qh": unperm8(arr(L.qh, np.int8, (NS, I))), "dh": arr(L.dh, np.float32, (NS, I // 32)),
        "tap": arr(L.tap, np.int32, (NS, int(L.tap_rows), H // 32)),
        "tap_stride": int(L.tap_stride),
    }
    return y.cpu().numpy(), taps


def compare(ref, cfg, OL, x, y, taps, tokens, check_dots=True, layer=0):
    """Oracle on `tokens`; returns (rel_l2 over those tokens, q_h flips).

    Routing: index lists equal to the oracle's with weights within 1e-6, or
    another correct choice across a near-tie (check_routing); a token that
    took one is compared with the oracle run on that choice, with the
    oracle's own gate values for it. At most one token in 64 may do so."""
    xs = x[tokens]
    yo, to = OL.forward(xs, taps=True)
    np.testing.assert_array_equal(taps["qx"][tokens], to["qx"])
    np.testing.assert_array_equal(taps["dx"][tokens], to["dx"])
    K, S, H, I = cfg.top_k, cfg.n_shared, cfg.hidden, cfg.inter
    swaps, w_for = check_routing(ref, cfg, xs, OL.w_router, OL.bias, taps["idx"][tokens],
                                 taps["w"][tokens])
    flips = 0
    for j, t in enumerate(tokens):
        if j in swaps:
            continue
        np.testing.assert_array_equal(taps["idx"][t], to["idx"][j])
        for k in range(K + S):
            s = taps["slot_of"][t, k]
            flips += int(np.sum(taps["qh"][s] != to["qh"][j, k]))
            if check_dots:
                e = int(taps["idx"][t, k]) if k < K else cfg.n_experts
                rows = np.arange(0, I, taps["tap_stride"])
                want = ref.block_dots(OL.experts[e]["gate_q"][rows], H, to["qx"][j:j + 1])[0]
                np.testing.assert_array_equal(taps["tap"][s][:len(rows)], want)
    if swaps:
        _note("near-tie choices", len(swaps), "of", len(tokens))
        assert len(swaps) <= max(1, len(tokens) // 64), swaps
        gidx = np.ascontiguousarray(taps["idx"][tokens])
        add_missing_experts(ref, cfg, layer, OL, gidx)
        yo = OL.forward(xs, forced_idx=gidx, forced_w=w_for)
    return rel_l2(y[tokens], yo), flips


def _note(*a):
    print("[case]", *a, flush=True)


def test_tiny_layer_all_tokens(C, ref):
    cfg = cs.CONFIGS[0]
    _note(cfg.name)
    W = _layer(C, cfg)
    x = layer_input(ref, cfg)
    y, taps = run_gpu(C, W, x)
    OL = oracle_layer_for(ref, cfg, 0, x)
    err, flips = compare(ref, cfg, OL, x, y, taps, list(range(cfg.n_tok)))
    _note("rel_l2", err, "flips", flips)
    assert flips == 0
    assert err <= TOL_REL_L2


@pytest.mark.parametrize("n_tok", [1, 2, 5, 9, 33])
def test_tiny_layer_token_counts(C, ref, n_tok):
    """Token counts on both sides of the few-token limit (1, 2 on the fused
    few-token kernels; 5, 9, 33 on the grouped MFMA kernels: one and several
    16-token groups per 32-token item, ragged last groups)."""
    cfg = cs.with_tokens(cs.CONFIGS[0], n_tok)
    _note(cfg.name, n_tok)
    W = _layer(C, cfg)
    x = layer_input(ref, cfg)
    y, taps = run_gpu(C, W, x)
    OL = oracle_layer_for(ref, cfg, 0, x)
    err, flips = compare(ref, cfg, OL, x, y, taps, list(range(n_tok)))
    assert flips == 0 and err <= TOL_REL_L2


# every token at full size: decode (1 token), MTP verify at 2, 3 and 4
# correlated tokens (the few-token kernels at each of their token counts), at
# 5 and 6 (drafts of 4 and 5: the grouped MFMA kernels with the fp64 epilogue,
# below the 16 tokens from which integer block scales are used) and the
# 512-token prefill chunk (grouped MFMA kernels, every item tail)
@pytest.mark.parametrize("cid,n_tok", [(1, 1), (2, 2), (2, 3), (2, 4), (2, 5), (2, 6), (3, 512)])
def test_full_size_layers(C, ref, cid, n_tok):
    cfg = cs.with_tokens(cs.CONFIGS[cid], n_tok)
    _note(cfg.name, n_tok)
    W = _layer(C, cfg)
    x = layer_input(ref, cfg)
    # the kernels without debug stores (the ones the bench times) first: they
    # must give the tapped kernels' output bit for bit
    y_plain, _ = run_gpu(C, W, x, taps=False)
    y, taps = run_gpu(C, W, x)
    np.testing.assert_array_equal(y_plain, y)
    tokens = list(range(n_tok))
    OL = oracle_layer_for(ref, cfg, 0, x)
    err, flips = compare(ref, cfg, OL, x, y, taps, tokens)
    _note("rel_l2", err, "flips", flips)
    assert flips == 0
    assert err <= TOL_REL_L2


# decode at full size on many tokens: 24 one-token calls on consecutive tokens
# of the decode input stream, each routed to its own experts (well over a
# hundred of the 256 in all), through the kernels the bench times and the
# tapped ones, every call against the oracle
def test_decode_calls_on_many_tokens(C, ref):
    n = 24
    cfg1 = cs.with_tokens(cs.CONFIGS[1], 1)
    cfgn = cs.with_tokens(cs.CONFIGS[1], n)
    _note(cfgn.name, "one-token calls", n)
    W = _layer(C, cfg1)
    xs = layer_input(ref, cfgn)
    OL = oracle_layer_for(ref, cfgn, 0, xs)  # every expert the n tokens select
    used = set()
    for t in range(n):
        x = np.ascontiguousarray(xs[t:t + 1])
        y_plain, _ = run_gpu(C, W, x, taps=False)
        y, taps = run_gpu(C, W, x)
        np.testing.assert_array_equal(y_plain, y)
        err, flips = compare(ref, cfg1, OL, x, y, taps, [0])
        assert flips == 0, (t, flips)
        assert err <= TOL_REL_L2, (t, err)
        used |= set(int(e) for e in taps["idx"][0])
    _note("experts used", len(used))
    assert len(used) > 100


# the two ends of the several-token work split at full size (E256 K8, four
# tokens): one token repeated four times (8 experts, each holding every token:
# two work units each, one h-block per workgroup) and four independent tokens
# (about 32 experts of one token each: as many units as entries, the most the
# grid holds)
@pytest.mark.parametrize("kind", ["same", "independent"])
def test_several_token_work_units(C, ref, kind):
    if kind == "same":
        cfg = cs.with_tokens(cs.CONFIGS[2], 4)
        x1 = layer_input(ref, cs.with_tokens(cs.CONFIGS[2], 1))
        x = np.ascontiguousarray(np.repeat(x1, 4, axis=0))
    else:
        cfg = cs.with_tokens(cs.CONFIGS[1], 4)
        x = layer_input(ref, cfg)
    _note("work units", kind)
    W = _layer(C, cfg)
    y_plain, _ = run_gpu(C, W, x, taps=False)
    y, taps = run_gpu(C, W, x)
    np.testing.assert_array_equal(y_plain, y)
    if kind == "same":  # every token's output equals the others'
        for t in range(1, 4):
            np.testing.assert_array_equal(y[t], y[0])
    OL = oracle_layer_for(ref, cfg, 0, x)
    err, flips = compare(ref, cfg, OL, x, y, taps, list(range(4)))
    _note("rel_l2", err, "flips", flips)
    assert flips == 0
    assert err <= TOL_REL_L2


def test_accumulate_and_zero_tokens(C, ref):
    cfg = cs.CONFIGS[0]
    _note("accumulate")
    W = _layer(C, cfg)
    x = layer_input(ref, cfg)
    base = cs.normal(cs.stream_key(99, 0, cs.T_X), x.shape, 1.0).numpy()
    y0, _ = run_gpu(C, W, x)
    y1, _ = run_gpu(C, W, x, C.COLI_FWD_ACCUM, y_in=base)
    np.testing.assert_array_equal(y1, base + y0)
    lc = W.cfg
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, 1), dtype=torch.uint8, device="cuda")
    empty = torch.empty((0, lc.hidden), dtype=torch.float32, device="cuda")
    C.coli_moe_forward(W, empty, empty, ws)


def test_batching_and_permutation_are_exact(C, ref):
    cfg = cs.with_tokens(cs.CONFIGS[0], 12)
    _note("batching/permutation")
    W = _layer(C, cfg)
    x = layer_input(ref, cfg)
    y, _ = run_gpu(C, W, x)
    perm = np.random.RandomState(3).permutation(12)
    yp, _ = run_gpu(C, W, np.ascontiguousarray(x[perm]))
    np.testing.assert_array_equal(yp, y[perm])
    for t in (0, 7):
        y1, _ = run_gpu(C, W, np.ascontiguousarray(x[t:t + 1]))
        np.testing.assert_array_equal(y1[0], y[t])


@pytest.mark.parametrize("n_tok", [1, 2, 4])
def test_router_ties_on_the_few_token_path(C, ref, n_tok):
    """Router rows and biases repeat with period 37, so expert e and e + 37
    have bit-identical scores; the K-th and (K+1)-th choices tie. Both sides
    must break ties to the lower expert index: index sets equal exactly."""
    import dataclasses
    cfg = dataclasses.replace(cs.CONFIGS[0], name="ties E256 K8", n_tok=n_tok, n_experts=256,
                              top_k=8)
    _note(cfg.name, n_tok)
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda", lambda w, qv, sv: C.coli_pack_int4(w, qv, sv))
    rows = torch.arange(cfg.n_experts, device="cuda") % 37
    wr, b = wr[rows].contiguous(), b[rows].contiguous()
    W = C.LayerWeights(lib_cfg(C, cfg), wr, b, q, s)
    x = layer_input(ref, cfg)
    y, taps = run_gpu(C, W, x)
    wrn, bn = wr.cpu().numpy(), b.cpu().numpy()
    idx, w, _ = ref.route(x, wrn, bn, cfg.top_k, cfg.norm_topk, cfg.rho)
    # every token's choice contains tied pairs (same row, different expert)
    assert all(len(set(int(e) % 37 for e in row)) < cfg.top_k for row in idx)
    np.testing.assert_array_equal(taps["idx"], idx)
    np.testing.assert_allclose(taps["w"], w, rtol=1e-6)
    OL = ref.OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                         cfg.norm_topk, cfg.rho, wrn, bn, {})
    for e in sorted(set(int(v) for v in np.unique(idx)) | {cfg.n_experts}):
        mats = [cs.expert_matrix(cfg, 0, e, m, "cuda").cpu().numpy() for m in ("gate", "up", "down")]
        OL.add_expert(e, ref.pack_expert(*mats))
    yo = OL.forward(x)
    err = rel_l2(y, yo)
    _note("rel_l2", err)
    assert err <= TOL_REL_L2
