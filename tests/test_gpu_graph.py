"""The layer forward captured in a HIP graph: coli_moe_forward (caller
workspace) and coli_moe_forward_static (the library's scratch array) are
captured once and replayed several times, with other eager forwards on the
same workspace or scratch, and synchronisations, between the replays; every
replay equals the eager forward of the same input bit for bit. Covers the
few-token kernels (one token at the GLM-5.2 shape, three tokens) and the
grouped MFMA path with integer block scales (33 tokens of the tiny layer)."""
import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import gpu_layer, layer_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    import int4_quantized_moe_sigmoid_amd as C
    assert torch.cuda.is_available()
    return C


def _eager(C, W, x, ws):
    y = torch.empty((x.shape[0], W.cfg.hidden), dtype=torch.float32, device="cuda")
    if ws is None:
        C.coli_moe_forward_static(W, x, y)
    else:
        C.coli_moe_forward(W, x, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check_graph(C, W, x, x_other, static):
    T = x.shape[0]
    ws = None
    if not static:
        ws = torch.empty(C.coli_moe_workspace_bytes(W.cfg, T), dtype=torch.uint8, device="cuda")
    want = _eager(C, W, x, ws)
    y = torch.empty((T, W.cfg.hidden), dtype=torch.float32, device="cuda")

    def fwd():
        if static:
            C.coli_moe_forward_static(W, x, y)
        else:
            C.coli_moe_forward(W, x, y, ws)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fwd()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        fwd()
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.isfinite(got).all(), f"replay {rep}"
        np.testing.assert_array_equal(got, want, err_msg=f"replay {rep}")
        # an eager forward of another input on the same workspace / scratch
        # between replays: the graph must not rely on what a call left there
        _eager(C, W, x_other, ws)


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("cid,n", [(1, 1), (2, 3), (0, 33)])
def test_forward_in_a_graph_matches_eager(C, ref, cid, n, static):
    cfg = cs.with_tokens(cs.CONFIGS[cid], n)
    print("[case] graph", cfg.name, n, "static" if static else "workspace", flush=True)
    W = gpu_layer(C, cfg)
    x = torch.from_numpy(layer_input(ref, cfg)).cuda()
    x_other = torch.from_numpy(layer_input(ref, cfg, first_tok=n)).cuda()
    _check_graph(C, W, x, x_other, static)
