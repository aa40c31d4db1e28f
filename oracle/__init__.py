"""TEST INFRASTRUCTURE ONLY: ctypes wrapper of the plain C++ CPU oracle.

Only tests/, the smoke check and the bench's CPU-baseline leg import this
package. The HIP product path never imports, links or calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coli_oracle.cpp")
_LIB = os.path.join(_HERE, "libcoli_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", _LIB + ".tmp", _SRC]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.coli_ref_pack_int4.argtypes = [vp, i64, i64, vp, vp]
        L.coli_ref_unpack_int4.argtypes = [vp, i64, i64, vp]
        L.coli_ref_pack.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
        L.coli_ref_unpack.argtypes = [vp, i64, i64, ctypes.c_int, vp]
        L.coli_ref_block_dots_bits.argtypes = [vp, i64, i64, ctypes.c_int, vp, i64, vp]
        L.coli_ref_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.coli_ref_e4m3_to_f32.restype = ctypes.c_float
        L.coli_ref_fp8_to_f32.argtypes = [vp, vp, i64, i64, vp]
        L.coli_ref_pack_fp8_int4.argtypes = [vp, vp, i64, i64, vp, vp]
        L.coli_ref_quant_q8.argtypes = [vp, i64, i64, vp, vp]
        L.coli_ref_block_dots.argtypes = [vp, i64, i64, vp, i64, vp]
        L.coli_ref_route.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_double, i64, i64, vp, vp, vp]
        L.coli_ref_gates.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_double, vp, vp]
        L.coli_ref_rmsnorm.argtypes = [vp, i64, i64, ctypes.c_double, vp]
        L.coli_ref_moe_forward.argtypes = [vp, vp, i64, vp, vp, vp, ctypes.c_int, vp]
        L.coli_ref_set_threads.argtypes = [ctypes.c_int]
        L.coli_ref_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def set_threads(n: int):
    lib().coli_ref_set_threads(int(n))


def num_threads() -> int:
    return int(lib().coli_ref_num_threads())


def pack_int4(w) -> tuple[np.ndarray, np.ndarray]:
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols // 2), np.uint8)
    s = np.empty(rows, np.float32)
    _check(lib().coli_ref_pack_int4(_p(w), rows, cols, _p(q), _p(s)), "pack_int4")
    return q, s


def pack_weights(w, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric b-bit pack (b in 2, 4, 8): codes [rows, cols b/8] u8, scale [rows]."""
    w = _c(w, np.float32)
    rows, cols = w.shape
    q = np.empty((rows, cols * bits // 8), np.uint8)
    s = np.empty(rows, np.float32)
    _check(lib().coli_ref_pack(_p(w), rows, cols, int(bits), _p(q), _p(s)), "pack")
    return q, s


def unpack(q, cols: int, bits: int) -> np.ndarray:
    q = _c(q, np.uint8)
    rows = q.shape[0]
    out = np.empty((rows, cols), np.int8)
    _check(lib().coli_ref_unpack(_p(q), rows, cols, int(bits), _p(out)), "unpack")
    return out


def e4m3_to_f32(b: int) -> float:
    """Value of one FP8 e4m3 code (the NaN code converts to 0)."""
    return float(lib().coli_ref_e4m3_to_f32(int(b)))


def fp8_to_f32(q8, block_scale) -> np.ndarray:
    """FP8 e4m3 codes [rows, cols] (uint8) times their 128 x 128 block scale,
    in fp32."""
    q8 = _c(q8, np.uint8)
    bs = _c(block_scale, np.float32)
    rows, cols = q8.shape
    if bs.shape != ((rows + 127) // 128, (cols + 127) // 128):
        raise ValueError("block scale shape")
    w = np.empty((rows, cols), np.float32)
    _check(lib().coli_ref_fp8_to_f32(_p(q8), _p(bs), rows, cols, _p(w)), "fp8_to_f32")
    return w


def pack_fp8_int4(q8, block_scale) -> tuple[np.ndarray, np.ndarray]:
    """FP8 e4m3 + block scales -> fp32 -> int4 (pack_int4 format)."""
    q8 = _c(q8, np.uint8)
    bs = _c(block_scale, np.float32)
    rows, cols = q8.shape
    if bs.shape != ((rows + 127) // 128, (cols + 127) // 128):
        raise ValueError("block scale shape")
    q = np.empty((rows, cols // 2), np.uint8)
    s = np.empty(rows, np.float32)
    _check(lib().coli_ref_pack_fp8_int4(_p(q8), _p(bs), rows, cols, _p(q), _p(s)),
           "pack_fp8_int4")
    return q, s


def unpack_int4(q, cols: int) -> np.ndarray:
    q = _c(q, np.uint8)
    rows = q.shape[0]
    out = np.empty((rows, cols), np.int8)
    _check(lib().coli_ref_unpack_int4(_p(q), rows, cols, _p(out)), "unpack_int4")
    return out


def quant_q8(x) -> tuple[np.ndarray, np.ndarray]:
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None]
    n, dim = x.shape
    q = np.empty((n, dim), np.int8)
    d = np.empty((n, dim // 32), np.float32)
    _check(lib().coli_ref_quant_q8(_p(x), n, dim, _p(q), _p(d)), "quant_q8")
    return q, d


def block_dots(wq, cols: int, qx, bits: int = 4) -> np.ndarray:
    wq = _c(wq, np.uint8)
    qx = _c(qx, np.int8)
    if qx.ndim == 1:
        qx = qx[None]
    rows = wq.shape[0]
    out = np.empty((qx.shape[0], rows, cols // 32), np.int32)
    _check(lib().coli_ref_block_dots_bits(_p(wq), rows, cols, int(bits), _p(qx), qx.shape[0],
                                          _p(out)), "block_dots")
    return out


def route(x, wr, bias, top_k: int, norm: bool = True, rho: float = 2.5, n_group: int = 1,
          topk_group: int = 1):
    """Sigmoid router + top-k; n_group > 1 selects among the topk_group best
    groups only (group score: sum of its two largest biased scores)."""
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    idx = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    logits = np.empty((T, E), np.float64)
    _check(lib().coli_ref_route(_p(x), _p(wr), _p(bias), T, H, E, top_k, int(norm),
                                float(np.float32(rho)), int(n_group), int(topk_group), _p(idx),
                                _p(w), _p(logits)), "route")
    return idx, w, logits


def gates(x, wr, bias, idx, norm: bool = True, rho: float = 2.5) -> np.ndarray:
    """Gate values the router gives the expert choice idx [T, K] (distinct
    experts per token): w_k = s[idx_k] / sum_k s[idx_k] * rho (without the
    division when norm is off), s the sigmoid of the router logits."""
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    bias = _c(bias, np.float32)
    idx = _c(idx, np.int32)
    T, H = x.shape
    E = wr.shape[0]
    K = idx.shape[1]
    w = np.empty((T, K), np.float32)
    _check(lib().coli_ref_gates(_p(x), _p(wr), _p(bias), T, H, E, K, int(norm),
                                float(np.float32(rho)), _p(idx), _p(w)), "gates")
    return w


def rmsnorm(x, eps: float = 1e-5) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty_like(x)
    _check(lib().coli_ref_rmsnorm(_p(x), x.shape[0], x.shape[1], float(eps), _p(out)),
           "rmsnorm")
    return out


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int64),
                ("n_shared", ctypes.c_int64), ("norm_topk", ctypes.c_int64),
                ("rho", ctypes.c_double),
                ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("gate_q", ctypes.c_void_p), ("up_q", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("n_group", ctypes.c_int64), ("topk_group", ctypes.c_int64),
                ("weight_bits", ctypes.c_int64)]


class _Taps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("idx", "w", "logits", "qx", "dx", "g", "u", "h", "qh", "dh", "ye")]


class OracleLayer:
    """Host-side layer for the oracle.

    experts: mapping expert id (0..E-1 routed, E = shared) -> dict with numpy
    arrays gate_q [I,H/2] u8, gate_s [I] f32, up_q, up_s, down_q [H,I/2], down_s [H].
    Experts that are absent may not be selected (the oracle rejects the call).
    """

    def __init__(self, hidden, inter, n_experts, top_k, n_shared, norm_topk, rho,
                 w_router, bias, experts: dict, n_group: int = 1, topk_group: int = 1,
                 weight_bits: int = 4):
        self.hidden, self.inter = int(hidden), int(inter)
        self.n_group, self.topk_group = int(n_group), int(topk_group)
        self.weight_bits = int(weight_bits)
        self.n_experts, self.top_k, self.n_shared = int(n_experts), int(top_k), int(n_shared)
        self.norm_topk, self.rho = bool(norm_topk), float(np.float32(rho))
        self.w_router = None if w_router is None else _c(w_router, np.float32)
        self.bias = None if bias is None else _c(bias, np.float32)
        self.experts = {}
        for e, d in experts.items():
            self.add_expert(e, d)

    def add_expert(self, e: int, d: dict):
        self.experts[int(e)] = {
            "gate_q": _c(d["gate_q"], np.uint8), "gate_s": _c(d["gate_s"], np.float32),
            "up_q": _c(d["up_q"], np.uint8), "up_s": _c(d["up_s"], np.float32),
            "down_q": _c(d["down_q"], np.uint8), "down_s": _c(d["down_s"], np.float32)}

    def _struct(self):
        n = self.n_experts + self.n_shared
        arrs = {}
        for key in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s"):
            a = (ctypes.c_void_p * n)()
            for e in range(n):
                a[e] = self.experts[e][key].ctypes.data if e in self.experts else None
            arrs[key] = a
        s = _Layer(self.hidden, self.inter, self.n_experts, self.top_k, self.n_shared,
                   int(self.norm_topk), self.rho,
                   _p(self.w_router), _p(self.bias),
                   ctypes.cast(arrs["gate_q"], ctypes.c_void_p),
                   ctypes.cast(arrs["up_q"], ctypes.c_void_p),
                   ctypes.cast(arrs["down_q"], ctypes.c_void_p),
                   ctypes.cast(arrs["gate_s"], ctypes.c_void_p),
                   ctypes.cast(arrs["up_s"], ctypes.c_void_p),
                   ctypes.cast(arrs["down_s"], ctypes.c_void_p),
                   self.n_group, self.topk_group, self.weight_bits)
        return s, arrs

    def forward(self, x, forced_idx=None, forced_w=None, y_in=None, taps: bool = False):
        """Returns y [T,H] (and a dict of intermediates when taps=True)."""
        x = _c(x, np.float32)
        T, H = x.shape
        K, KS, I, E = self.top_k, self.top_k + self.n_shared, self.inter, self.n_experts
        y = _c(y_in, np.float32).copy() if y_in is not None else np.zeros((T, H), np.float32)
        fi = None if forced_idx is None else _c(forced_idx, np.int32)
        fw = None if forced_w is None else _c(forced_w, np.float32)
        t = None
        tp = None
        if taps:
            t = {"idx": np.empty((T, K), np.int32), "w": np.empty((T, K), np.float32),
                 "logits": np.empty((T, E), np.float64),
                 "qx": np.empty((T, H), np.int8), "dx": np.empty((T, H // 32), np.float32),
                 "g": np.empty((T, KS, I), np.float32), "u": np.empty((T, KS, I), np.float32),
                 "h": np.empty((T, KS, I), np.float32), "qh": np.empty((T, KS, I), np.int8),
                 "dh": np.empty((T, KS, I // 32), np.float32),
                 "ye": np.empty((T, KS, H), np.float32)}
            tp = _Taps(**{k: v.ctypes.data for k, v in t.items()})
        s, keep = self._struct()
        rc = lib().coli_ref_moe_forward(ctypes.byref(s), _p(x), T, _p(fi), _p(fw), _p(y),
                                        int(y_in is not None),
                                        ctypes.byref(tp) if tp is not None else None)
        del keep
        _check(rc, "moe_forward")
        return (y, t) if taps else y


def pack_expert(gate: np.ndarray, up: np.ndarray, down: np.ndarray, bits: int = 4) -> dict:
    """Oracle-packed expert from fp32 matrices gate/up [I,H], down [H,I]."""
    gq, gs = pack_weights(gate, bits)
    uq, us = pack_weights(up, bits)
    dq, ds = pack_weights(down, bits)
    return {"gate_q": gq, "gate_s": gs, "up_q": uq, "up_s": us, "down_q": dq, "down_s": ds}
