"""GPU checks specific to the grouped MFMA (many-token) kernels.

- The kernels without debug taps (the ones a caller runs) give the same
  output, bit for bit, as the tapped kernels the parity tests compare with the
  oracle: full-size prefill (T = 512, int4) and mid-size layers of every
  weight width, with 32-token items and with 64-token items (taken once the
  routed experts average 48 tokens or more).
- 64-token items (1, 2 or 4 groups of 16) at parity with the oracle on every
  token of a small layer.
- Rows whose Q8_0 block scales span more than 2^7 have no 31-bit integer form
  (the exact int64 sum of the K loop needs one), so their items take the fp64
  epilogue: an input token with one block scaled by 1e-4 (x side) and a shared
  expert whose first 32 gate rows are scaled by 1e-5 (its h rows, down side)
  both stay at parity with the oracle (q_h codes equal, output within 1e-4
  rel-L2), with taps and without.
"""
import dataclasses

import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import gpu_layer, layer_input, lib_cfg, oracle_layer_for
from test_gpu_layer import compare, run_gpu

pytestmark = pytest.mark.gpu

TOL_REL_L2 = 1e-4


@pytest.fixture(scope="module")
def C():
    import int4_quantized_moe_sigmoid_amd as C
    assert torch.cuda.is_available()
    return C


def _note(*a):
    print("[case]", *a, flush=True)


def _forward(C, W, x, flags):
    T = x.shape[0]
    ws = torch.empty(C.coli_moe_workspace_bytes(W.cfg, T, flags), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((T, W.cfg.hidden), dtype=torch.float32, device="cuda")
    C.coli_moe_forward(W, torch.from_numpy(x).cuda(), y, ws, flags)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _bits_layer(C, cfg, bits):
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda",
                                 lambda w, qv, sv: C.coli_pack_weights(w, bits, qv, sv), bits=bits)
    return C.LayerWeights(lib_cfg(C, cfg, bits=bits), wr, b, q, s)


def test_untapped_kernels_match_tapped_full_prefill(C, ref):
    cfg = cs.CONFIGS[3]
    _note(cfg.name, "tapped vs untapped")
    W = gpu_layer(C, cfg)
    x = layer_input(ref, cfg)
    y0 = _forward(C, W, x, 0)
    y1 = _forward(C, W, x, C.COLI_FWD_DEBUG_TAPS)
    assert np.isfinite(y0).all()
    np.testing.assert_array_equal(y0, y1)
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bits,n_tok", [(8, 200), (4, 200), (2, 200), (8, 800), (4, 800), (2, 800)])
def test_untapped_kernels_match_tapped_widths(C, ref, bits, n_tok):
    # 200 tokens: 25 per routed expert (32-token items); 800: 100 (64-token items)
    cfg = dataclasses.replace(cs.CONFIGS[3], name=f"mid T{n_tok} H1024 E32 K4 I512", n_tok=n_tok,
                              hidden=1024, n_experts=32, top_k=4, inter=512)
    _note(cfg.name, "bits", bits)
    W = _bits_layer(C, cfg, bits)
    x = layer_input(ref, cfg)
    y0 = _forward(C, W, x, 0)
    y1 = _forward(C, W, x, C.COLI_FWD_DEBUG_TAPS)
    assert np.isfinite(y0).all()
    np.testing.assert_array_equal(y0, y1)


def _wide_cfg(n_tok=40):
    return dataclasses.replace(cs.CONFIGS[0], name=f"wide scales T{n_tok} H256 E16 K2 I128",
                               n_tok=n_tok)


def _wide_layer(C, cfg):
    """GPU layer with the shared expert's gate rows 0..31 scaled by 1e-5."""
    calls = [0]
    shared_gate = 3 * cfg.n_experts  # build_layer packs gate, up, down of expert 0, 1, ...

    def pack(w, qv, sv):
        if calls[0] == shared_gate:
            w[:32] *= np.float32(1e-5)
        calls[0] += 1
        C.coli_pack_int4(w, qv, sv)
    wr, b, q, s = cs.build_layer(cfg, 0, "cuda", pack)
    return C.LayerWeights(lib_cfg(C, cfg), wr, b, q, s)


def _wide_oracle(ref, cfg, x):
    wr, b = cs.router(cfg, 0, "cpu")
    wr, b = wr.numpy(), b.numpy()
    idx, _, _ = ref.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho)
    need = sorted(set(int(e) for e in np.unique(idx)) | {cfg.n_experts})
    L = ref.OracleLayer(cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k, cfg.n_shared,
                        cfg.norm_topk, cfg.rho, wr, b, {})
    for e in need:
        mats = [cs.expert_matrix(cfg, 0, e, m, "cpu").numpy().copy() for m in ("gate", "up", "down")]
        if e == cfg.n_experts:
            mats[0][:32] *= np.float32(1e-5)
        L.add_expert(e, ref.pack_expert(*mats))
    return L


@pytest.mark.parametrize("n_tok", [40, 400])  # 32- and 64-token items
def test_wide_scale_rows_take_the_fp64_epilogue(C, ref, n_tok):
    cfg = _wide_cfg(n_tok)
    _note(cfg.name)
    W = _wide_layer(C, cfg)
    x = layer_input(ref, cfg)
    x[3, :32] *= np.float32(1e-4)  # token 3: one block 1e4 below the others
    OL = _wide_oracle(ref, cfg, x)
    tokens = list(range(cfg.n_tok))
    y, taps = run_gpu(C, W, x)
    # the scales really are wide: x of token 3, h of every shared slot
    dx3 = taps["dx"][3]
    assert dx3.max() / dx3[dx3 > 0].min() > 2.0 ** 8
    sh = taps["slot_of"][:, cfg.top_k]
    dh = taps["dh"][sh]
    assert all(r.max() / r[r > 0].min() > 2.0 ** 8 for r in dh)
    err, flips = compare(ref, cfg, OL, x, y, taps, tokens)
    _note("rel_l2", err, "flips", flips)
    assert flips == 0
    assert err <= TOL_REL_L2
    y0 = _forward(C, W, x, 0)
    np.testing.assert_array_equal(y0, y)


def test_64_token_items_at_oracle_parity(C, ref):
    # 400 tokens x 2 of 16 experts: 50 per expert, items of 50 and 64 tokens
    # (four groups of 16), 64-token items of the shared expert and a 16-token tail
    cfg = dataclasses.replace(cs.CONFIGS[0], name="items64 T400 H256 E16 K2 I128", n_tok=400)
    _note(cfg.name)
    W = gpu_layer(C, cfg)
    x = layer_input(ref, cfg)
    y, taps = run_gpu(C, W, x)
    tokens = list(range(cfg.n_tok))
    OL = oracle_layer_for(ref, cfg, 0, x)
    err, flips = compare(ref, cfg, OL, x, y, taps, tokens)
    _note("rel_l2", err, "flips", flips)
    assert flips == 0
    assert err <= TOL_REL_L2
    np.testing.assert_array_equal(_forward(C, W, x, 0), y)
