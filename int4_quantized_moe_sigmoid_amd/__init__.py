"""Python binding of libcoli_moe.so (include/coli_moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Tensors are torch tensors on the GPU (torch provides device memory
and streams); the default stream is torch's current stream. There is no
fallback: importing raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcoli_moe.so")

COLI_OK = 0
COLI_E_INVAL = -1
COLI_E_ALIGN = -2
COLI_E_WORKSPACE = -3
COLI_E_HIP = -4
COLI_E_UNSUPPORTED = -5
COLI_FWD_ACCUM = 1
COLI_FWD_DEBUG_TAPS = 2

EXPORTS = ("coli_strerror", "coli_pack_weights", "coli_pack_int4", "coli_pack_fp8_int4",
           "coli_quant_q8", "coli_moe_workspace_bytes",
           "coli_moe_workspace_layout", "coli_moe_route", "coli_moe_forward",
           "coli_moe_forward_profiled", "coli_moe_forward_static", "coli_rmsnorm",
           "coli_stream_read", "coli_mfma_probe")


class ColiError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.coli_strerror(code).decode()} (code {code})")


class coli_moe_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("weight_bits", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class coli_moe_weights(ctypes.Structure):
    _fields_ = [("cfg", coli_moe_cfg), ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("experts_q", ctypes.c_void_p), ("experts_scale", ctypes.c_void_p)]


class coli_moe_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("total", "qx", "dx", "logits", "topk_idx", "topk_w", "counts", "offs",
                 "slot_of", "slot_tok", "qh", "dh", "ye", "tap")] + \
               [("n_slots", ctypes.c_int64), ("tap_rows", ctypes.c_int64),
                ("tap_stride", ctypes.c_int64), ("reserved", ctypes.c_size_t * 4)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'` "
                          "(or python int4_quantized_moe_sigmoid_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, u32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32, \
        ctypes.c_int
    L.coli_strerror.argtypes = [i32]
    L.coli_strerror.restype = ctypes.c_char_p
    L.coli_pack_int4.argtypes = [vp, i64, i64, vp, vp, vp]
    L.coli_pack_fp8_int4.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.coli_pack_weights.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    L.coli_quant_q8.argtypes = [vp, i64, i64, vp, vp, vp]
    L.coli_moe_workspace_bytes.argtypes = [ctypes.POINTER(coli_moe_cfg), i64, u32]
    L.coli_moe_workspace_bytes.restype = sz
    L.coli_moe_workspace_layout.argtypes = [ctypes.POINTER(coli_moe_cfg), i64, u32,
                                            ctypes.POINTER(coli_moe_ws_layout)]
    L.coli_moe_route.argtypes = [vp, vp, vp, i64, ctypes.POINTER(coli_moe_cfg), vp, vp, vp, sz,
                                 vp]
    L.coli_moe_forward.argtypes = [ctypes.POINTER(coli_moe_weights), vp, i64, vp, vp, sz, u32,
                                   vp]
    L.coli_moe_forward_profiled.argtypes = [ctypes.POINTER(coli_moe_weights), vp, i64, vp, vp,
                                            sz, u32, vp, ctypes.POINTER(vp), i32,
                                            ctypes.POINTER(i32),
                                            ctypes.POINTER(ctypes.c_char_p)]
    L.coli_moe_forward_static.argtypes = [ctypes.POINTER(coli_moe_weights), vp, i64, vp, u32, vp]
    L.coli_rmsnorm.argtypes = [vp, i64, i64, ctypes.c_float, vp, vp]
    L.coli_stream_read.argtypes = [vp, i64, vp, vp]
    L.coli_mfma_probe.argtypes = [i32, i64, i32, vp, vp]
    for name in EXPORTS:
        getattr(L, name)
    return L


_lib = _load()


def lib():
    return _lib


def _check(rc: int, where: str):
    if rc != COLI_OK:
        raise ColiError(rc, where)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def make_cfg(hidden: int, inter: int, n_experts: int, top_k: int, n_shared: int = 1,
             norm_topk: bool = True, routed_scale: float = 2.5, n_group: int = 1,
             topk_group: int = 1, weight_bits: int = 4) -> coli_moe_cfg:
    """n_group > 1 selects the experts among the topk_group best of n_group
    groups (group-limited top-k); 1 is the plain selection. weight_bits: width
    of the expert weight codes (4, 8 or 2)."""
    return coli_moe_cfg(hidden, inter, n_experts, top_k, n_shared, int(bool(norm_topk)),
                        routed_scale, int(n_group), int(topk_group), int(weight_bits), 0)


class LayerWeights:
    """Device weights of one layer in the boundary format (see coli_moe_weights)."""

    def __init__(self, cfg: coli_moe_cfg, w_router: torch.Tensor, bias: torch.Tensor,
                 experts_q: torch.Tensor, experts_scale: torch.Tensor):
        n = cfg.n_experts + cfg.n_shared
        H, I = cfg.hidden, cfg.inter
        bits = cfg.weight_bits or 4
        if tuple(w_router.shape) != (cfg.n_experts, H) or tuple(bias.shape) != (cfg.n_experts,):
            raise ValueError("router weight / bias shape mismatch")
        if experts_q.numel() != n * 3 * I * H * bits // 8 or \
                experts_scale.numel() != n * (2 * I + H):
            raise ValueError("expert blob sizes do not match the config")
        self.cfg = cfg
        self.w_router, self.bias = w_router, bias
        self.experts_q, self.experts_scale = experts_q, experts_scale
        self.struct = coli_moe_weights(
            cfg, _dev(w_router, "w_router", torch.float32), _dev(bias, "bias", torch.float32),
            _dev(experts_q, "experts_q", torch.uint8),
            _dev(experts_scale, "experts_scale", torch.float32))

    @staticmethod
    def blob_views(cfg: coli_moe_cfg, experts_q: torch.Tensor, experts_scale: torch.Tensor,
                   e: int):
        """(gate_q, up_q, down_q, gate_s, up_s, down_s) views of expert e's blobs."""
        H, I = cfg.hidden, cfg.inter
        bits = cfg.weight_bits or 4
        mb = I * H * bits // 8
        bq = 3 * mb
        q = experts_q.view(-1)[e * bq:(e + 1) * bq]
        bs = 2 * I + H
        s = experts_scale.view(-1)[e * bs:(e + 1) * bs]
        return (q[:mb].view(I, H * bits // 8), q[mb:2 * mb].view(I, H * bits // 8),
                q[2 * mb:].view(H, I * bits // 8), s[:I], s[I:2 * I], s[2 * I:])


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------

def coli_pack_int4(w: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None):
    rows, cols = w.shape
    _check(_lib.coli_pack_int4(_dev(w, "w", torch.float32), rows, cols,
                               _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
                               _stream(stream)), "coli_pack_int4")


def coli_pack_weights(w: torch.Tensor, bits: int, q: torch.Tensor, scale: torch.Tensor,
                      stream=None):
    rows, cols = w.shape
    _check(_lib.coli_pack_weights(_dev(w, "w", torch.float32), rows, cols, int(bits),
                                  _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
                                  _stream(stream)), "coli_pack_weights")


def coli_pack_fp8_int4(q8: torch.Tensor, block_scale: torch.Tensor, q: torch.Tensor,
                       scale: torch.Tensor, stream=None):
    rows, cols = q8.shape
    if tuple(block_scale.shape) != ((rows + 127) // 128, (cols + 127) // 128):
        raise ValueError("block_scale must be [ceil(rows/128), ceil(cols/128)]")
    _check(_lib.coli_pack_fp8_int4(_dev(q8, "q8", torch.uint8),
                                   _dev(block_scale, "block_scale", torch.float32), rows, cols,
                                   _dev(q, "q", torch.uint8), _dev(scale, "scale", torch.float32),
                                   _stream(stream)), "coli_pack_fp8_int4")


def coli_quant_q8(x: torch.Tensor, q: torch.Tensor, d: torch.Tensor, stream=None):
    n, dim = x.shape
    _check(_lib.coli_quant_q8(_dev(x, "x", torch.float32), n, dim, _dev(q, "q", torch.int8),
                              _dev(d, "d", torch.float32), _stream(stream)), "coli_quant_q8")


def coli_moe_workspace_bytes(cfg: coli_moe_cfg, max_tok: int, flags: int = 0) -> int:
    n = _lib.coli_moe_workspace_bytes(ctypes.byref(cfg), max_tok, flags)
    if n == 0:
        raise ColiError(COLI_E_INVAL, "coli_moe_workspace_bytes")
    return int(n)


def coli_moe_workspace_layout(cfg: coli_moe_cfg, n_tok: int, flags: int = 0):
    out = coli_moe_ws_layout()
    _check(_lib.coli_moe_workspace_layout(ctypes.byref(cfg), n_tok, flags, ctypes.byref(out)),
           "coli_moe_workspace_layout")
    return out


def coli_moe_route(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor,
                   cfg: coli_moe_cfg, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                   ws: torch.Tensor, stream=None):
    _check(_lib.coli_moe_route(_dev(x, "x", torch.float32),
                               _dev(w_router, "w_router", torch.float32),
                               _dev(bias, "bias", torch.float32), x.shape[0], ctypes.byref(cfg),
                               _dev(topk_idx, "topk_idx", torch.int32),
                               _dev(topk_w, "topk_w", torch.float32),
                               _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
           "coli_moe_route")


def coli_moe_forward(weights: LayerWeights, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                     flags: int = 0, stream=None):
    _check(_lib.coli_moe_forward(ctypes.byref(weights.struct), _dev(x, "x", torch.float32),
                                 x.shape[0], _dev(y, "y", torch.float32),
                                 _dev(ws, "ws", torch.uint8), ws.numel(), flags,
                                 _stream(stream)), "coli_moe_forward")


def coli_moe_forward_profiled(weights: LayerWeights, x: torch.Tensor, y: torch.Tensor,
                              ws: torch.Tensor, events: Sequence[int], flags: int = 0,
                              stream=None):
    """events: raw hipEvent_t handles, two per launch (start, stop of launch j at
    2j, 2j + 1). Returns the names of the launches timed."""
    n = len(events)
    arr = (ctypes.c_void_p * max(n, 1))(*events)
    names = (ctypes.c_char_p * max(n // 2, 1))()
    used = ctypes.c_int(0)
    _check(_lib.coli_moe_forward_profiled(ctypes.byref(weights.struct),
                                          _dev(x, "x", torch.float32), x.shape[0],
                                          _dev(y, "y", torch.float32),
                                          _dev(ws, "ws", torch.uint8), ws.numel(), flags,
                                          _stream(stream), arr, n, ctypes.byref(used), names),
           "coli_moe_forward_profiled")
    return [names[i].decode() for i in range(min(used.value, n // 2))]


def coli_moe_forward_static(weights: LayerWeights, x: torch.Tensor, y: torch.Tensor,
                            flags: int = 0, stream=None):
    """coli_moe_forward with the library's fixed per-GPU scratch array instead
    of a workspace (no allocation; calls on one GPU must not overlap)."""
    _check(_lib.coli_moe_forward_static(ctypes.byref(weights.struct),
                                        _dev(x, "x", torch.float32), x.shape[0],
                                        _dev(y, "y", torch.float32), flags, _stream(stream)),
           "coli_moe_forward_static")


def coli_rmsnorm(x: torch.Tensor, out: torch.Tensor, eps: float = 1e-5, stream=None):
    n, dim = x.shape
    _check(_lib.coli_rmsnorm(_dev(x, "x", torch.float32), n, dim, eps,
                             _dev(out, "out", torch.float32), _stream(stream)), "coli_rmsnorm")


def coli_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Streaming read of buf (uint8, device) into the XOR checksum sink (int32[1])."""
    _check(_lib.coli_stream_read(_dev(buf, "buf", torch.uint8), buf.numel(),
                                 _dev(sink, "sink", torch.int32), _stream(stream)),
           "coli_stream_read")


def coli_mfma_probe(kind: int, n_workgroups: int, iters: int, cycles: torch.Tensor, stream=None):
    """Issue-rate probe (see coli_moe.h): cycles is int64 [4 n_workgroups + 1]."""
    if cycles.numel() < 4 * n_workgroups + 1:
        raise ValueError("cycles must hold 4 * n_workgroups + 1 entries")
    _check(_lib.coli_mfma_probe(int(kind), int(n_workgroups), int(iters),
                                _dev(cycles, "cycles", torch.int64), _stream(stream)),
           "coli_mfma_probe")
