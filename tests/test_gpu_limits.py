"""GPU parity at the edges of the configuration space, against the oracle:
the most routed experts and the largest top-k the boundary accepts (E = 1024,
K = 16; K = 16 also on the few-token path at E = 256), the largest hidden and
intermediate sizes (8192) on the grouped MFMA kernels and a hidden size that
sends the layer to the GEMV kernels, and the method's degenerate settings:
gates not normalised, no shared expert, one expert per token, every expert
chosen. Index sets exact (ties tolerated as in the layer tests), Q8_0 codes
and block dots bit-exact, output within 1e-4 rel-L2."""
import dataclasses

import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import gpu_layer, layer_input, oracle_layer_for
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


def _check(C, ref, cfg, tokens=None):
    W = gpu_layer(C, cfg)
    x = layer_input(ref, cfg)
    y, taps = run_gpu(C, W, x)
    tokens = list(range(cfg.n_tok)) if tokens is None else tokens
    OL = oracle_layer_for(ref, cfg, 0, x[tokens])
    err, flips = compare(ref, cfg, OL, x, y, taps, tokens)
    _note("rel_l2", err, "flips", flips)
    assert np.isfinite(y).all()
    assert err <= TOL_REL_L2
    del W
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,K,n_tok", [(1024, 16, 1), (1024, 16, 6), (256, 16, 1), (256, 16, 4)])
def test_most_experts_largest_topk(C, ref, E, K, n_tok):
    cfg = dataclasses.replace(cs.CONFIGS[0], name=f"E{E} K{K}", n_experts=E, top_k=K,
                              n_tok=n_tok)
    _note(cfg.name, n_tok)
    _check(C, ref, cfg)


@pytest.mark.parametrize("H,I,n_tok", [(8192, 8192, 1), (8192, 8192, 5), (8160, 8192, 2)])
def test_largest_hidden_and_inter(C, ref, H, I, n_tok):
    # 8160 = 255 x 32 is no multiple of the MFMA row tile: the GEMV kernels
    cfg = dataclasses.replace(cs.CONFIGS[0], name=f"H{H} I{I}", hidden=H, inter=I, n_experts=4,
                              top_k=2, n_tok=n_tok)
    _note(cfg.name, n_tok)
    _check(C, ref, cfg)


@pytest.mark.parametrize("n_tok", [1, 3, 9])
def test_gates_not_normalised(C, ref, n_tok):
    cfg = dataclasses.replace(cs.CONFIGS[0], name="norm off", norm_topk=False, n_tok=n_tok)
    _note(cfg.name, n_tok)
    _check(C, ref, cfg)


@pytest.mark.parametrize("K,n_tok", [(2, 1), (2, 2), (2, 9), (1, 1), (1, 5)])
def test_no_shared_expert(C, ref, K, n_tok):
    cfg = dataclasses.replace(cs.CONFIGS[0], name=f"no shared K{K}", n_shared=0, top_k=K,
                              n_tok=n_tok)
    _note(cfg.name, n_tok)
    _check(C, ref, cfg)


@pytest.mark.parametrize("n_tok", [1, 4, 7])
def test_every_expert_chosen(C, ref, n_tok):
    cfg = dataclasses.replace(cs.CONFIGS[0], name="E4 K4", n_experts=4, top_k=4, n_tok=n_tok)
    _note(cfg.name, n_tok)
    _check(C, ref, cfg)


# shapes the grouped MFMA kernels do not tile (I or H not a multiple of 64)
# and the few-token kernels do not take (I % 64 != 0, or H > 6144): the GEMV
# kernels with items of up to 4 tokens — one, two and four token slots per
# item (NT = 1, 2, 4), experts split over several items, ragged last items
@pytest.mark.parametrize("H,I,n_tok", [(8160, 256, 1), (256, 96, 1), (256, 96, 2),
                                       (256, 96, 3), (256, 96, 5), (256, 96, 9),
                                       (256, 96, 33)])
def test_gemv_path(C, ref, H, I, n_tok):
    cfg = dataclasses.replace(cs.CONFIGS[0], name=f"gemv H{H} I{I}", hidden=H, inter=I,
                              n_experts=4, top_k=2, n_tok=n_tok)
    _note(cfg.name, n_tok)
    _check(C, ref, cfg)
