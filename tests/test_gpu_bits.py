"""GPU parity of the int8 and int2 weight formats (coli_pack_weights, and the
layer: the fused few-token kernels up to four tokens, the grouped MFMA
kernels above): packing bit-exact; Q8_0(x) codes in each width's element
order, per-block gate dots bit-exact through the debug tap; Q8_0(h) codes
equal; outputs within 1e-4 rel-L2 of the oracle (tiny workload on every
token; full decode, MTP-verify and prefill shapes on sampled tokens)."""
import dataclasses

import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import layer_input, lib_cfg, oracle_layer_for, rel_l2, unperm_for

pytestmark = pytest.mark.gpu

TOL_REL_L2 = 1e-4


@pytest.fixture(scope="module")
def C():
    import int4_quantized_moe_sigmoid_amd as C
    assert torch.cuda.is_available()
    return C


def _note(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 256), (2048, 6144), (6144, 2048)])
def test_pack_weights_bit_exact(C, ref, bits, rows, cols):
    _note("pack", bits, rows, cols)
    w = (cs.normal(cs.stream_key(31 + bits, rows, cs.T_X), (rows, cols), 0.02).numpy())
    w[rows // 2] = 0.0
    q = torch.empty((rows, cols * bits // 8), dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    C.coli_pack_weights(torch.from_numpy(w).cuda(), bits, q, s)
    torch.cuda.synchronize()
    rq, rs = ref.pack_weights(w, bits)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def _layer(C, cfg, bits):
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda",
                                 lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv), bits=bits)
    return C.LayerWeights(lib_cfg(C, cfg, bits=bits), wr, b, q, s)


def _run_plain(C, W, x):
    """The layer without debug stores (the kernels the bench times): y only."""
    T = x.shape[0]
    lc = W.cfg
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T, 0), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, lc.hidden), dtype=torch.float32, device="cuda")
    C.coli_moe_forward(W, torch.from_numpy(x).cuda(), y, ws, 0)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run(C, W, x):
    T = x.shape[0]
    lc = W.cfg
    fl = C.COLI_FWD_DEBUG_TAPS
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, T, fl), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, lc.hidden), dtype=torch.float32, device="cuda")
    C.coli_moe_forward(W, torch.from_numpy(x).cuda(), y, ws, fl)
    torch.cuda.synchronize()
    L = C.coli_moe_workspace_layout(lc, T, fl)
    wsn = ws.cpu().numpy()
    H, I, K, S = lc.hidden, lc.inter, lc.top_k, lc.n_shared

    def arr(off, dtype, shape):
        n = int(np.prod(shape))
        return np.frombuffer(wsn[off:off + n * np.dtype(dtype).itemsize].tobytes(),
                             dtype=dtype).reshape(shape)
    NS = int(L.n_slots)
    un = unperm_for(lc.weight_bits)
    return y.cpu().numpy(), {
        "qx": un(arr(L.qx, np.int8, (T, H))), "dx": arr(L.dx, np.float32, (T, H // 32)),
        "idx": arr(L.topk_idx, np.int32, (T, K)), "w": arr(L.topk_w, np.float32, (T, K)),
        "slot_of": arr(L.slot_of, np.int32, (T, K + S)),
        "qh": un(arr(L.qh, np.int8, (NS, I))), "dh": arr(L.dh, np.float32, (NS, I // 32)),
        "tap": arr(L.tap, np.int32, (NS, int(L.tap_rows), H // 32)),
        "tap_stride": int(L.tap_stride)}


def _compare(ref, cfg, bits, x, y, taps, tokens):
    OL = oracle_layer_for(ref, cfg, 0, x[tokens], bits=bits)
    xs = x[tokens]
    yo, to = OL.forward(xs, taps=True)
    np.testing.assert_array_equal(taps["qx"][tokens], to["qx"])
    np.testing.assert_array_equal(taps["dx"][tokens], to["dx"])
    K, S, H, I = cfg.top_k, cfg.n_shared, cfg.hidden, cfg.inter
    flips = 0
    for j, t in enumerate(tokens):
        assert list(taps["idx"][t]) == list(to["idx"][j])
        np.testing.assert_allclose(taps["w"][t], to["w"][j], rtol=1e-6)
        for k in range(K + S):
            sl = taps["slot_of"][t, k]
            flips += int(np.sum(taps["qh"][sl] != to["qh"][j, k]))
            e = int(taps["idx"][t, k]) if k < K else cfg.n_experts
            rows = np.arange(0, I, taps["tap_stride"])
            want = ref.block_dots(OL.experts[e]["gate_q"][rows], H, to["qx"][j:j + 1], bits)[0]
            np.testing.assert_array_equal(taps["tap"][sl][:len(rows)], want)
    err = rel_l2(y[tokens], yo)
    _note("rel_l2", err, "q_h flips", flips)
    assert err <= TOL_REL_L2


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("n_tok", [1, 2, 3, 4, 5, 33])
def test_tiny_layer_every_token(C, ref, bits, n_tok):
    cfg = cs.with_tokens(cs.CONFIGS[0], n_tok)
    _note("tiny", bits, n_tok)
    W = _layer(C, cfg, bits)
    x = layer_input(ref, cfg)
    y, taps = _run(C, W, x)
    _compare(ref, cfg, bits, x, y, taps, list(range(n_tok)))


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("cid,n_tok,sample", [(1, 1, None), (2, 3, None), (3, 512, 16)])
def test_full_size_layers(C, ref, bits, cid, n_tok, sample):
    cfg = cs.with_tokens(cs.CONFIGS[cid], n_tok)
    _note("full", bits, cfg.name, n_tok)
    W = _layer(C, cfg, bits)
    x = layer_input(ref, cfg)
    y_plain = _run_plain(C, W, x)
    y, taps = _run(C, W, x)
    # the kernels without debug stores give the tapped kernels' output bit for bit
    np.testing.assert_array_equal(y_plain, y)
    tokens = list(range(n_tok)) if sample is None else \
        sorted(set(np.random.RandomState(9).choice(n_tok, sample, replace=False).tolist()) |
               {0, n_tok - 1})
    _compare(ref, cfg, bits, x, y, taps, tokens)
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits,n_tok", [(2, 1), (2, 2), (8, 1), (8, 3), (8, 4)])
def test_few_token_ragged_hidden(C, ref, bits, n_tok):
    # hidden 288 = 9 blocks of 32: most lanes of a row hold no block (the
    # fused kernels take up to four tokens, two with int2 weights)
    cfg = dataclasses.replace(cs.CONFIGS[0], hidden=288, n_tok=n_tok)
    _note("ragged hidden", bits, n_tok)
    W = _layer(C, cfg, bits)
    x = layer_input(ref, cfg)
    y, taps = _run(C, W, x)
    _compare(ref, cfg, bits, x, y, taps, list(range(n_tok)))


def test_rejects_unsupported_widths(C):
    # five tokens leave the fused kernels; hidden 288 = 9 x 32 is no multiple
    # of the MFMA row tile (64), and the GEMV kernels take int4 only
    cfg = dataclasses.replace(cs.CONFIGS[0], hidden=288, n_tok=5)
    for bits, code in [(8, C.COLI_E_UNSUPPORTED), (3, C.COLI_E_INVAL)]:
        lc = lib_cfg(C, cfg, bits=bits)
        n = cfg.n_experts + cfg.n_shared
        wb = 8 if bits == 3 else bits
        q = torch.zeros(n * 3 * cfg.inter * cfg.hidden * wb // 8, dtype=torch.uint8, device="cuda")
        s = torch.zeros(n * (2 * cfg.inter + cfg.hidden), dtype=torch.float32, device="cuda")
        wr = torch.zeros((cfg.n_experts, cfg.hidden), device="cuda")
        b = torch.zeros(cfg.n_experts, device="cuda")
        if bits == 3:
            with pytest.raises(Exception):
                C.LayerWeights(lc, wr, b, q, s)
            continue
        W = C.LayerWeights(lc, wr, b, q, s)
        ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
        y = torch.empty((5, cfg.hidden), device="cuda")
        with pytest.raises(C.ColiError) as ei:
            C.coli_moe_forward(W, torch.zeros((5, cfg.hidden), device="cuda"), y, ws)
        assert ei.value.code == code
    w = torch.zeros((2, 64), device="cuda")
    with pytest.raises(C.ColiError):
        C.coli_pack_weights(w, 3, torch.empty((2, 32), dtype=torch.uint8, device="cuda"),
                            torch.empty(2, device="cuda"))


@pytest.mark.parametrize("bits,n_tok,shared,norm", [(8, 1, 0, False), (8, 3, 1, False),
                                                     (2, 2, 0, True), (2, 7, 1, False),
                                                     (8, 9, 0, True)])
def test_widths_with_groups_and_degenerate_settings(C, ref, bits, n_tok, shared, norm):
    # int8 / int2 weights together with group-limited selection (8 groups of
    # 8 experts, 4 kept), no shared expert, gates not normalised; the fused
    # kernels (up to four tokens, int2 two) and the MFMA kernels
    cfg = dataclasses.replace(cs.CONFIGS[0], name=f"E64 K4 groups int{bits}", n_experts=64,
                              top_k=4, n_shared=shared, norm_topk=norm, n_tok=n_tok)
    _note("widths+groups", bits, n_tok, shared, norm)
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda",
                                 lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv), bits=bits)
    W = C.LayerWeights(lib_cfg(C, cfg, n_group=8, topk_group=4, bits=bits), wr, b, q, s)
    x = layer_input(ref, cfg)
    y, taps = _run(C, W, x)
    OL = oracle_layer_for(ref, cfg, 0, x, n_group=8, topk_group=4, bits=bits)
    yo, to = OL.forward(x, taps=True)
    np.testing.assert_array_equal(taps["qx"], to["qx"])
    np.testing.assert_array_equal(taps["idx"], to["idx"])
    np.testing.assert_allclose(taps["w"], to["w"], rtol=1e-6)
    err = rel_l2(y, yo)
    _note("rel_l2", err)
    assert err <= TOL_REL_L2
