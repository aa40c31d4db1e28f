"""GPU parity of the int8 and int2 weight formats (coli_pack_weights, and the
layer: the fused few-token kernels up to four tokens, the grouped MFMA
kernels above): packing bit-exact; Q8_0(x) codes in each width's element
order, per-block gate dots bit-exact through the debug tap; Q8_0(h) codes
equal; outputs within 1e-4 rel-L2 of the oracle (tiny workload on every
token, and on every token of layers whose experts take 64-token items; full
decode, MTP-verify and 512-token prefill shapes on every token)."""
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


def _compare(ref, cfg, bits, x, y, taps, tokens, OL=None, max_flips=None):
    if OL is None:
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
    if max_flips is not None:
        assert flips <= max_flips


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
@pytest.mark.parametrize("shape", ["tiny T400", "mid T800"])
def test_64_token_items_every_token(C, ref, bits, shape):
    # routed experts averaging 48 tokens or more take 64-token items (the
    # grouped kernels' KT = 64 instances at this width): every token against
    # the oracle, and the untapped kernels bit for bit against the tapped ones
    if shape == "tiny T400":  # 50 tokens per routed expert, 16-token tails
        cfg = cs.with_tokens(cs.CONFIGS[0], 400)
    else:  # zipf-skewed bias, 100 tokens per routed expert on average
        cfg = dataclasses.replace(cs.CONFIGS[3], name="mid T800 H1024 E32 K4 I512", n_tok=800,
                                  hidden=1024, n_experts=32, top_k=4, inter=512)
    _note("items64", bits, cfg.name)
    W = _layer(C, cfg, bits)
    x = layer_input(ref, cfg)
    y_plain = _run_plain(C, W, x)
    y, taps = _run(C, W, x)
    np.testing.assert_array_equal(y_plain, y)
    _compare(ref, cfg, bits, x, y, taps, list(range(cfg.n_tok)))
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("n_tok", [40, 400])  # 32- and 64-token items
def test_wide_scale_rows_take_the_fp64_epilogue(C, ref, bits, n_tok):
    # Q8_0 block scales of one row spanning more than 2^7 have no 31-bit
    # integer form, so such items take the fp64 epilogue: one block of input
    # token 3 scaled by 1e-4 (x side), the shared expert's first 32 gate rows
    # by 1e-5 (its h rows, down side); parity with the oracle on every token,
    # with taps and without
    cfg = dataclasses.replace(cs.CONFIGS[0], name=f"wide scales T{n_tok} H256 E16 K2 I128",
                              n_tok=n_tok)
    _note("wide", bits, cfg.name)
    calls = [0]
    shared_gate = 3 * cfg.n_experts  # build_layer packs gate, up, down of expert 0, 1, ...

    def pack(w, qv, sv):
        if calls[0] == shared_gate:
            w[:32] *= np.float32(1e-5)
        calls[0] += 1
        C.coli_pack_weights(w, bits, qv, sv)
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda", pack, bits=bits)
    W = C.LayerWeights(lib_cfg(C, cfg, bits=bits), wr, b, q, s)
    x = layer_input(ref, cfg)
    x[3, :32] *= np.float32(1e-4)
    wro, bo = cs.router(cfg, 0, "cpu")
    wro, bo = wro.numpy(), bo.numpy()
    idx, _, _ = ref.route(x, wro, bo, cfg.top_k, cfg.norm_topk, cfg.rho)
    OL = ref.OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                         cfg.norm_topk, cfg.rho, wro, bo, {}, 1, 1, bits)
    for e in sorted(set(int(v) for v in np.unique(idx)) | {cfg.n_experts}):
        mats = [cs.expert_matrix(cfg, 0, e, m, "cpu").numpy().copy() for m in ("gate", "up", "down")]
        if e == cfg.n_experts:
            mats[0][:32] *= np.float32(1e-5)
        OL.add_expert(e, ref.pack_expert(*mats, bits=bits))
    y_plain = _run_plain(C, W, x)
    y, taps = _run(C, W, x)
    np.testing.assert_array_equal(y_plain, y)
    # the scales really are wide: x of token 3, h of every shared slot
    dx3 = taps["dx"][3]
    assert dx3.max() / dx3[dx3 > 0].min() > 2.0 ** 8
    dh = taps["dh"][taps["slot_of"][:, cfg.top_k]]
    assert all(r.max() / r[r > 0].min() > 2.0 ** 8 for r in dh)
    _compare(ref, cfg, bits, x, y, taps, list(range(n_tok)), OL=OL, max_flips=0)


@pytest.mark.parametrize("bits", [2, 8])
@pytest.mark.parametrize("cid,n_tok,sample", [(1, 1, None), (2, 3, None), (3, 512, None)])
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
