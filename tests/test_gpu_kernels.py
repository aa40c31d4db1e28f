"""GPU parity of the single-purpose entry points against the oracle:
int4 packing and Q8_0 codes bit-exact, RMSNorm, router index sets and gates."""
import numpy as np
import pytest
import torch

import coli_synth as cs
from gpu_util import layer_input, lib_cfg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    import int4_quantized_moe_sigmoid_amd as C
    assert torch.cuda.is_available()
    return C


def _note(*a):
    print("[case]", *a, flush=True)


def _tie_rows(rows, cols, seed):
    """Rows whose values sit exactly on int4 rounding ties, plus a zero row."""
    rng = np.random.RandomState(seed)
    w = (rng.randint(-14, 15, (rows, cols)) * 0.5).astype(np.float32)   # k/2 multiples of s=0.5
    w[:, 0] = 3.5                                                        # max |w| = 3.5 -> s = 0.5
    w[1] = 0.0
    return w


@pytest.mark.parametrize("rows,cols", [(1, 32), (5, 96), (37, 256), (2048, 6144), (6144, 2048)])
def test_pack_int4_bit_exact(C, ref, rows, cols):
    _note("pack", rows, cols)
    key = cs.stream_key(11, rows, cs.T_GATE, cols)
    w = cs.normal(key, (rows, cols), 0.02).numpy()
    if rows >= 5:
        w[:5] = _tie_rows(5, cols, rows)
    wd = torch.from_numpy(w).cuda()
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    C.coli_pack_int4(wd, q, s)
    torch.cuda.synchronize()
    rq, rs = ref.pack_int4(w)
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("n,dim", [(1, 32), (3, 256), (7, 6144), (512, 2048)])
def test_quant_q8_bit_exact(C, ref, n, dim):
    _note("quant_q8", n, dim)
    x = cs.normal(cs.stream_key(12, n, cs.T_X, dim), (n, dim), 1.0).numpy()
    # block 0 of token 0 has scale exactly 1 and values on rounding ties
    x[0, :10] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 3.5]
    if dim >= 64:
        x[-1, 32:64] = 0.0                                    # an all-zero block
    xd = torch.from_numpy(x).cuda()
    q = torch.empty((n, dim), dtype=torch.int8, device="cuda")
    d = torch.empty((n, dim // 32), dtype=torch.float32, device="cuda")
    C.coli_quant_q8(xd, q, d)
    torch.cuda.synchronize()
    rq, rd = ref.quant_q8(x)
    np.testing.assert_array_equal(d.cpu().numpy(), rd)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_rmsnorm_matches_oracle(C, ref):
    _note("rmsnorm")
    x = (cs.normal(cs.stream_key(13, 0, cs.T_X), (33, 6144), 1.0).numpy() * 3).astype(np.float32)
    x[5] = 0.0
    out = torch.empty_like(torch.from_numpy(x)).cuda()
    C.coli_rmsnorm(torch.from_numpy(x).cuda(), out, 1e-5)
    torch.cuda.synchronize()
    want = ref.rmsnorm(x, np.float32(1e-5))
    got = out.cpu().numpy()
    # fp64 sums in another order: equal except where the exact value is within
    # ~1e-16 of an fp32 rounding boundary
    assert np.mean(got == want) > 0.9999
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=0)


def _check_route(ref, cfg, x, wr, b, idx, w, tol_tie=1e-6):
    ridx, rw, logits = ref.route(x, wr, b, cfg.top_k, cfg.norm_topk, cfg.rho)
    c = 1.0 / (1.0 + np.exp(-logits)) + b.astype(np.float64)
    for t in range(x.shape[0]):
        if set(idx[t]) != set(ridx[t]):
            # accept only a swap across a (near-)tie at the k-th boundary
            kth = np.sort(c[t])[::-1][cfg.top_k - 1]
            diff = set(idx[t]) ^ set(ridx[t])
            assert all(abs(c[t, e] - kth) <= tol_tie for e in diff), (t, idx[t], ridx[t])
        else:
            np.testing.assert_array_equal(idx[t], ridx[t])
            np.testing.assert_allclose(w[t], rw[t], rtol=1e-6)


@pytest.mark.parametrize("cid,n_tok", [(0, 4), (1, 1), (2, 3), (3, 512), (4, 300)])
def test_route_matches_oracle(C, ref, cid, n_tok):
    cfg = cs.with_tokens(cs.CONFIGS[cid], n_tok)
    _note("route", cfg.name, n_tok)
    x = layer_input(ref, cfg)
    wr, b = cs.router(cfg, 0, "cpu")
    wr, b = wr.numpy(), b.numpy()
    lc = lib_cfg(C, cfg)
    ws = torch.empty(C.coli_moe_workspace_bytes(lc, n_tok), dtype=torch.uint8, device="cuda")
    idx = torch.empty((n_tok, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((n_tok, cfg.top_k), dtype=torch.float32, device="cuda")
    C.coli_moe_route(torch.from_numpy(x).cuda(), torch.from_numpy(wr).cuda(),
                     torch.from_numpy(b).cuda(), lc, idx, w, ws)
    torch.cuda.synchronize()
    _check_route(ref, cfg, x, wr, b, idx.cpu().numpy(), w.cpu().numpy())


def test_generator_identical_on_gpu():
    _note("generator")
    key = cs.stream_key(1, 0, cs.T_DOWN, 77)
    a = cs.normal(key, (1000, 333), 0.02, "cpu")
    g = cs.normal(key, (1000, 333), 0.02, "cuda").cpu()
    assert torch.equal(a, g)


def test_rejects_bad_arguments(C):
    _note("errors")
    x = torch.zeros((2, 48), dtype=torch.float32, device="cuda")
    q = torch.empty((2, 48), dtype=torch.int8, device="cuda")
    d = torch.empty((2, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(C.ColiError) as e:
        C.coli_quant_q8(x, q, d)
    assert e.value.code == C.COLI_E_INVAL
    x = torch.zeros(2 * 64 + 1, dtype=torch.float32, device="cuda")[1:].view(2, 64)
    q = torch.empty((2, 64), dtype=torch.int8, device="cuda")
    d = torch.empty((2, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(C.ColiError) as e:
        C.coli_quant_q8(x, q, d)
    assert e.value.code == C.COLI_E_ALIGN
    cfg = C.make_cfg(6144, 2048, 256, 8)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((1, 8), dtype=torch.float32, device="cuda")
    xr = torch.zeros((1, 6144), dtype=torch.float32, device="cuda")
    wr = torch.zeros((256, 6144), dtype=torch.float32, device="cuda")
    b = torch.zeros(256, dtype=torch.float32, device="cuda")
    with pytest.raises(C.ColiError) as e:
        C.coli_moe_route(xr, wr, b, cfg, idx, w, small)
    assert e.value.code == C.COLI_E_WORKSPACE
    bad = C.make_cfg(6144, 2048, 4, 8)
    assert C.lib().coli_moe_workspace_bytes(bad, 1, 0) == 0


def _fp8_weights(rows, cols, seed, nan_codes):
    """Seeded FP8 e4m3 codes of normally distributed weights with 128 x 128
    block scales of a few binades (a block-quantised checkpoint's shape)."""
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(rows, cols, generator=g) * 64.0
    q8 = w.to(torch.float8_e4m3fn).view(torch.uint8)
    if nan_codes:
        q8[0, :7] = 0x7F
        q8[-1, -5:] = 0xFF
        q8[rows // 2] = 0x80  # a row of negative zeros packs to scale 0
    nb = ((rows + 127) // 128, (cols + 127) // 128)
    bs = torch.exp2(torch.randint(-14, -6, nb, generator=g).float()) * \
        (1.0 + torch.rand(nb, generator=g))
    return q8.contiguous(), bs.float().contiguous()


@pytest.mark.parametrize("rows,cols,nan_codes", [(200, 352, True), (1, 32, False),
                                                 (130, 8192, True), (3, 8224, True),
                                                 (13, 2048, True), (5, 3072, False),
                                                 (9, 1024, True), (129, 4096, False),
                                                 (2048, 6144, True), (6144, 2048, False)])
def test_pack_fp8_int4_bit_exact(C, ref, rows, cols, nan_codes):
    print("[case] pack_fp8_int4", rows, cols, flush=True)
    q8, bs = _fp8_weights(rows, cols, rows + cols, nan_codes)
    q = torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    C.coli_pack_fp8_int4(q8.cuda(), bs.cuda(), q, s)
    torch.cuda.synchronize()
    rq, rs = ref.pack_fp8_int4(q8.numpy(), bs.numpy())
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("cols", [256, 1024])
def test_pack_fp8_int4_every_code(C, ref, cols):
    """Every e4m3 code (subnormals, both zeros, both NaN codes, +-448) in every
    position of a 16-code chunk, under unit and extreme block scales."""
    print("[case] pack_fp8_int4 every code", cols, flush=True)
    rows = 256
    q8 = ((torch.arange(rows)[:, None] + torch.arange(cols)[None, :]) % 256).to(torch.uint8)
    bs = torch.tensor([[1.0, 2.0 ** -120], [2.0 ** 100, 3.0]], dtype=torch.float32)
    bs = bs.repeat(1, cols // 256)
    q = torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    C.coli_pack_fp8_int4(q8.cuda(), bs.cuda(), q, s)
    torch.cuda.synchronize()
    rq, rs = ref.pack_fp8_int4(q8.numpy(), bs.numpy())
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("nbytes", [16, 4096 + 7 * 16, 64 << 20])
def test_stream_read_checksum(C, nbytes):
    # the read-ceiling probe touches every 16-byte word once: its XOR checksum
    # equals the XOR of all 32-bit words of the buffer
    _note("stream_read", nbytes)
    rng = np.random.RandomState(nbytes % 1000)
    host = rng.randint(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).copy()).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    C.coli_stream_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == want
    lib = C.lib()
    assert lib.coli_stream_read(buf.data_ptr(), 24, sink.data_ptr(), None) == C.COLI_E_INVAL
    assert lib.coli_stream_read(buf.data_ptr() + 4, 16, sink.data_ptr(), None) == C.COLI_E_ALIGN
