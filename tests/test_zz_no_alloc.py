"""coli_moe_forward_static (no workspace argument, the library's fixed per-GPU
scratch array) against coli_moe_forward with a caller workspace: identical
outputs, bit for bit, on two calls in a row with the second smaller (the
scratch keeps the first call's contents), on the few-token kernels and on
the grouped MFMA kernels; a token count beyond the array is rejected before
anything is launched."""
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


def _with_ws(C, W, x, flags=0):
    T = x.shape[0]
    ws = torch.empty(C.coli_moe_workspace_bytes(W.cfg, T, flags), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((T, W.cfg.hidden), dtype=torch.float32, device="cuda")
    C.coli_moe_forward(W, x, y, ws, flags)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _static(C, W, x, flags=0):
    y = torch.full((x.shape[0], W.cfg.hidden), float("nan"), dtype=torch.float32,
                   device="cuda")
    C.coli_moe_forward_static(W, x, y, flags)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("cid,counts", [(2, (3, 1)), (0, (33, 5))])
def test_static_scratch_matches_workspace(C, ref, cid, counts):
    cfg = cs.with_tokens(cs.CONFIGS[cid], max(counts))
    print("[case] static scratch", cfg.name, counts, flush=True)
    W = gpu_layer(C, cfg)
    xall = torch.from_numpy(layer_input(ref, cfg)).cuda()
    for n in counts:                       # the second call is the smaller one
        x = xall[:n].contiguous()
        got = _static(C, W, x)
        want = _with_ws(C, W, x)
        assert np.isfinite(got).all()
        np.testing.assert_array_equal(got, want)
    # accumulate into y, as the stacked layers do
    x = xall[:counts[1]].contiguous()
    base = torch.randn((counts[1], cfg.hidden), generator=torch.Generator().manual_seed(5))
    y = base.cuda()
    C.coli_moe_forward_static(W, x, y, C.COLI_FWD_ACCUM)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), base.numpy() + _with_ws(C, W, x))
    del W
    torch.cuda.empty_cache()


def test_static_scratch_rejects_too_many_tokens(C):
    cfg = C.make_cfg(6144, 2048, 256, 8)
    n = 4096
    need = C.coli_moe_workspace_bytes(cfg, n)
    assert need > (32 << 20)
    wr = torch.zeros((256, 6144), dtype=torch.float32, device="cuda")
    b = torch.zeros(256, dtype=torch.float32, device="cuda")
    q = torch.zeros(257 * 3 * 2048 * 3072, dtype=torch.uint8, device="cuda")
    s = torch.zeros(257 * (2 * 2048 + 6144), dtype=torch.float32, device="cuda")
    W = C.LayerWeights(cfg, wr, b, q, s)
    x = torch.zeros((n, 6144), dtype=torch.float32, device="cuda")
    y = torch.full((n, 6144), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(C.ColiError) as e:
        C.coli_moe_forward_static(W, x, y)
    assert e.value.code == C.COLI_E_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())          # nothing was launched
    empty = torch.empty((0, 6144), dtype=torch.float32, device="cuda")
    C.coli_moe_forward_static(W, empty, empty)
