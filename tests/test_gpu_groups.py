"""GPU parity of group-limited expert selection (n_group groups of E/n_group
consecutive experts, the topk_group best kept) on every routing path: the
one-token and few-token fused kernels, and the many-token top-k kernel (also
behind coli_moe_route). Full decode shapes (H6144 E256 K8 I2048), 8 groups,
4 kept, as in DeepSeek-V3's configuration."""
import dataclasses

import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import layer_input, lib_cfg, oracle_layer_for, rel_l2
from test_gpu_layer import run_gpu

pytestmark = pytest.mark.gpu

NG, TG = 8, 4
TOL_REL_L2 = 1e-4


@pytest.fixture(scope="module")
def C():
    import int4_quantized_moe_sigmoid_amd as C
    assert torch.cuda.is_available()
    return C


@pytest.fixture(scope="module")
def layer(C):
    cfg = cs.CONFIGS[1]
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda", lambda w, qv, sv: C.coli_pack_int4(w, qv, sv))
    yield cfg, wr, b, q, s
    torch.cuda.empty_cache()


def _note(*a):
    print("[case]", *a, flush=True)


def _group_scores(c, gs):
    g = np.sort(c.reshape(-1, gs), axis=1)[:, ::-1]
    return g[:, 0] + g[:, 1]


def _check_choice(ref, cfg, x, wr, b, idx, w, tol=1e-6, ng=NG, tg=TG, must_differ=True):
    """Index sets equal to the oracle's, except a swap across a near-tie (of
    expert scores at the K-th place or of group scores at the kept boundary)."""
    ridx, rw, logits = ref.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho, ng, tg)
    plain, _, _ = ref.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho)
    if must_differ:
        assert np.any(np.sort(ridx, 1) != np.sort(plain, 1)), "groups never changed the choice"
    c = 1.0 / (1.0 + np.exp(-logits)) + b.astype(np.float64)
    gs = cfg.n_experts // ng
    NG, TG = ng, tg
    for t in range(x.shape[0]):
        if list(idx[t]) == list(ridx[t]):
            np.testing.assert_allclose(w[t], rw[t], rtol=1e-6)
            continue
        gsc = np.sort(_group_scores(c[t], gs))[::-1]
        near_group = gsc[TG - 1] - gsc[TG] <= tol
        kept = {int(e) // gs for e in ridx[t]}
        cand = np.sort(c[t][[e for e in range(cfg.n_experts) if e // gs in kept]])[::-1]
        near_kth = cand[cfg.top_k - 1] - cand[cfg.top_k] <= tol
        assert near_group or near_kth, (t, idx[t], ridx[t])
        if not near_group:
            # the same groups kept: the swapped experts sit at the K-th place
            diff = set(int(e) for e in idx[t]) ^ set(int(e) for e in ridx[t])
            assert all(abs(c[t][e] - cand[cfg.top_k - 1]) <= tol for e in diff), \
                (t, idx[t], ridx[t])


@pytest.mark.parametrize("n_tok", [1, 3, 300])
def test_grouped_route_matches_oracle(C, ref, layer, n_tok):
    cfg0, wr, b, _, _ = layer
    cfg = cs.with_tokens(cfg0, n_tok)
    _note("grouped route", n_tok)
    x = layer_input(ref, cfg)
    lc = lib_cfg(C, cfg, NG, TG)
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, n_tok), dtype=torch.uint8, device="cuda")
    idx = torch.empty((n_tok, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((n_tok, cfg.top_k), dtype=torch.float32, device="cuda")
    C.coli_moe_route(torch.from_numpy(x).cuda(), wr, b, lc, idx, w, ws)
    torch.cuda.synchronize()
    _check_choice(ref, cfg, x, wr.cpu().numpy(), b.cpu().numpy(), idx.cpu().numpy(),
                  w.cpu().numpy())


@pytest.mark.parametrize("n_tok,sample", [(1, None), (2, None), (3, None), (512, 5)])
def test_grouped_layer_matches_oracle(C, ref, layer, n_tok, sample):
    cfg0, wr, b, q, s = layer
    cfg = cs.with_tokens(cfg0, n_tok)
    _note("grouped layer", n_tok)
    W = C.LayerWeights(lib_cfg(C, cfg, NG, TG), wr, b, q, s)
    x = layer_input(ref, cfg)
    y, taps = run_gpu(C, W, x)
    _check_choice(ref, cfg, x, wr.cpu().numpy(), b.cpu().numpy(), taps["idx"], taps["w"])
    tokens = list(range(n_tok)) if sample is None else \
        sorted(set(np.random.RandomState(7).choice(n_tok, sample, replace=False).tolist()) |
               {0, n_tok - 1})
    # the GPU's choice (checked above: the oracle's, or another correct one
    # across a near-tie) with the oracle's own gate values for it
    gidx = np.ascontiguousarray(taps["idx"][tokens])
    OL = oracle_layer_for(ref, cfg, 0, x[tokens], forced_idx=gidx, n_group=NG, topk_group=TG)
    w_for = ref.gates(x[tokens], wr.cpu().numpy(), b.cpu().numpy(), gidx, cfg.norm_topk, cfg.rho)
    np.testing.assert_allclose(taps["w"][tokens], w_for, rtol=1e-6)
    yo = OL.forward(x[tokens], forced_idx=gidx, forced_w=w_for)
    err = rel_l2(y[tokens], yo)
    _note("rel_l2", err)
    assert err <= TOL_REL_L2


# (E, n_group, topk_group): group sizes 32, 4 and 64 take the lane-shuffle
# group scores on the few-token paths, 128 (one-token path only) and 30 the
# LDS path; 16 groups keeping 2 have 2 * topk_group < K
GROUP_CFGS = [(256, 8, 4), (256, 64, 4), (256, 4, 2), (256, 2, 1), (240, 8, 4), (256, 16, 2)]


def _tiny(n_tok, E):
    return dataclasses.replace(cs.CONFIGS[0], name=f"groups E{E} K8", n_tok=n_tok,
                               n_experts=E, top_k=8)


def _route_any_path(C, W_parts, lc, x, n_tok, K):
    """Routing from the fused few-token kernels (forward taps) for n_tok <= 3,
    else from coli_moe_route (many-token top-k kernel)."""
    wr, b, q, s = W_parts
    if n_tok <= 3:
        _, taps = run_gpu(C, C.LayerWeights(lc, wr, b, q, s), x)
        return taps["idx"], taps["w"]
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, n_tok), dtype=torch.uint8, device="cuda")
    idt = torch.empty((n_tok, K), dtype=torch.int32, device="cuda")
    wt = torch.empty((n_tok, K), dtype=torch.float32, device="cuda")
    C.coli_moe_route(torch.from_numpy(x).cuda(), wr, b, lc, idt, wt, ws)
    torch.cuda.synchronize()
    return idt.cpu().numpy(), wt.cpu().numpy()


@pytest.mark.parametrize("E,ng,tg", GROUP_CFGS)
@pytest.mark.parametrize("n_tok", [1, 2, 300])
def test_group_configs_match_oracle(C, ref, E, ng, tg, n_tok):
    cfg = _tiny(n_tok, E)
    _note(cfg.name, "groups", ng, tg, "tokens", n_tok)
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda", lambda w, qv, sv: C.coli_pack_int4(w, qv, sv))
    x = layer_input(ref, cfg)
    idx, w = _route_any_path(C, (wr, b, q, s), lib_cfg(C, cfg, ng, tg), x, n_tok, cfg.top_k)
    _check_choice(ref, cfg, x, wr.cpu().numpy(), b.cpu().numpy(), idx, w, ng=ng, tg=tg,
                  must_differ=n_tok > 1)


@pytest.mark.parametrize("E,ng,tg", GROUP_CFGS)
@pytest.mark.parametrize("n_tok", [1, 2, 300])
def test_group_and_expert_ties(C, ref, E, ng, tg, n_tok):
    """Every group holds the same router rows and biases, so all group scores
    tie (the lowest groups must be kept) and every chosen score appears in
    each kept group (ties to the lower expert index): index sets exactly equal."""
    cfg = _tiny(n_tok, E)
    _note(cfg.name, "ties, groups", ng, tg, "tokens", n_tok)
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda", lambda w, qv, sv: C.coli_pack_int4(w, qv, sv))
    gs = cfg.n_experts // ng
    rows = torch.arange(cfg.n_experts, device="cuda") % gs
    wr, b = wr[rows].contiguous(), b[rows].contiguous()
    x = layer_input(ref, cfg)
    wrn, bn = wr.cpu().numpy(), b.cpu().numpy()
    ridx, rw, _ = ref.route(x, wrn, bn, cfg.top_k, cfg.norm_topk, cfg.rho, ng, tg)
    assert np.all(ridx < tg * gs)  # only the lowest groups
    idx, w = _route_any_path(C, (wr, b, q, s), lib_cfg(C, cfg, ng, tg), x, n_tok, cfg.top_k)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_allclose(w, rw, rtol=1e-6)


def test_rejects_bad_groups(C):
    cfg = cs.CONFIGS[1]
    wr = torch.zeros((256, 6144), device="cuda")
    b = torch.zeros(256, device="cuda")
    x = torch.zeros((1, 6144), device="cuda")
    idx = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((1, 8), dtype=torch.float32, device="cuda")
    for ng, tg in [(6, 2), (8, 0), (8, 9), (64, 1), (128, 4)]:
        lc = lib_cfg(C, cfg, ng, tg)
        ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        with pytest.raises(C.ColiError):
            C.coli_moe_route(x, wr, b, lc, idx, w, ws)
