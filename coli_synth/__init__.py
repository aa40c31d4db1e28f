"""Seeded synthetic inputs for the sigmoid-routed int4 MoE layer.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle. It holds none of the layer's arithmetic: it only draws numbers.

Generator (the same on every device, bit for bit):
  * a counter-based 64-bit hash, the SplitMix64 output function (Steele, Lea &
    Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014):
    element i of stream `key` is mix(key + (i+1) * 0x9E3779B97F4A7C15);
  * inverse-transform sampling of N(0,1) through a fixed table of 2^16 normal
    quantiles at the cell midpoints, Phi^-1((k + 0.5) / 65536), indexed by the
    top 16 bits of the hash, then one float32 multiply by sigma.
Integer ops wrap modulo 2^64 on CPU and GPU alike and the table is built once
on the host, so CPU and GPU draws are identical.

Streams are keyed by (config seed, layer, tensor id, expert); element index is
the row-major position inside the tensor, so any expert can be drawn alone.
"""
from __future__ import annotations

import dataclasses
import statistics
from typing import Optional

import numpy as np
import torch

_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_C1 = 0xBF58476D1CE4E5B9
_C2 = 0x94D049BB133111EB

# tensor ids inside a stream key
T_X = 1        # activations (independent part)
T_WR = 2       # router weight
T_BIAS = 3     # router correction bias
T_GATE = 4
T_UP = 5
T_DOWN = 6
T_XSHARED = 7  # shared component of correlated activations
T_RANK = 8     # Zipf rank permutation


def _s64(v: int) -> int:
    """Python int -> the int64 with the same low 64 bits."""
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_py(z: int) -> int:
    """SplitMix64 output function on a Python int (reference for tests)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * _C1) & _M64
    z = ((z ^ (z >> 27)) * _C2) & _M64
    return z ^ (z >> 31)


def stream_key(seed: int, layer: int, tensor: int, expert: int = 0) -> int:
    """64-bit key of one tensor's stream (chained SplitMix64 over the tuple)."""
    k = 0
    for part in (seed, layer, tensor, expert):
        k = mix64_py((k + _GOLDEN + (part & _M64)) & _M64)
    return k


def hash_py(key: int, i: int) -> int:
    """Element i of stream `key`, pure Python."""
    return mix64_py(key + (i + 1) * _GOLDEN)


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of an int64 tensor."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def hash_t(key: int, idx: torch.Tensor) -> torch.Tensor:
    """Element idx (int64 tensor) of stream `key`, as int64 bit patterns."""
    z = (idx + 1) * _s64(_GOLDEN) + _s64(key)
    z = (z ^ _srl(z, 30)) * _s64(_C1)
    z = (z ^ _srl(z, 27)) * _s64(_C2)
    return z ^ _srl(z, 31)


_TABLE_CACHE: dict = {}


def normal_table(device="cpu") -> torch.Tensor:
    """2^16 float32 quantiles of N(0,1) at cell midpoints."""
    dev = torch.device(device)
    key = str(dev)
    if key not in _TABLE_CACHE:
        if "cpu" not in _TABLE_CACHE:
            nd = statistics.NormalDist()
            vals = np.array([nd.inv_cdf((k + 0.5) / 65536.0) for k in range(65536)],
                            dtype=np.float64).astype(np.float32)
            _TABLE_CACHE["cpu"] = torch.from_numpy(vals)
        _TABLE_CACHE[key] = _TABLE_CACHE["cpu"].to(dev)
    return _TABLE_CACHE[key]


def normal(key: int, shape, sigma: float, device="cpu", out: Optional[torch.Tensor] = None,
           chunk: int = 1 << 24) -> torch.Tensor:
    """float32 tensor of N(0, sigma) draws from stream `key` (row-major element order)."""
    dev = torch.device(device)
    n = int(np.prod(shape)) if len(shape) else 1
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    flat = out.view(-1)
    table = normal_table(dev)
    sig = torch.tensor(sigma, dtype=torch.float32, device=dev)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(s, e, dtype=torch.int64, device=dev)
        h = hash_t(key, idx)
        flat[s:e] = table[_srl(h, 48)] * sig
    return out


def normal_py(key: int, i: int, sigma: float) -> float:
    """One draw, pure Python/numpy (reference for tests)."""
    tab = normal_table("cpu")
    v = np.float32(tab[hash_py(key, i) >> 48].item())
    return float(np.float32(v * np.float32(sigma)))


# --------------------------------------------------------------------------
# workload recipes
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int
    n_tok: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_shared: int = 1
    rho: float = 2.5
    norm_topk: bool = True
    rmsnorm_input: bool = True   # inputs are RMS-normalised before the layer
    bias_kind: str = "normal"    # "normal" N(0,.01) | "zipf" | "zero"
    correlated: bool = False     # x_t = 0.7 z + 0.3 eps_t
    n_layers: int = 1            # >1: pre-norm residual stack
    w_sigma: float = 0.02
    wr_sigma: float = 0.02
    b_sigma: float = 0.01

    @property
    def n_slots(self) -> int:
        return self.n_tok * (self.top_k + self.n_shared)

    def expert_bytes(self) -> int:
        """Packed bytes of one expert (gate, up, down) plus its row scales."""
        q = 3 * self.inter * self.hidden // 2
        s = 4 * (2 * self.inter + self.hidden)
        return q + s


CONFIGS = {
    0: MoEConfig("tiny T4 H256 E16 K2 I128", 0, 4, 256, 16, 2, 128, rmsnorm_input=False),
    1: MoEConfig("decode T1 H6144 E256 K8 I2048", 1, 1, 6144, 256, 8, 2048),
    2: MoEConfig("mtp-verify T3 correlated", 2, 3, 6144, 256, 8, 2048, correlated=True),
    3: MoEConfig("prefill T512 zipf-bias", 3, 512, 6144, 256, 8, 2048, bias_kind="zipf"),
    4: MoEConfig("stack8 T4096 uniform", 4, 4096, 6144, 256, 8, 2048, bias_kind="zero",
                 n_layers=8, rmsnorm_input=False),
}


def with_tokens(cfg: MoEConfig, n_tok: int) -> MoEConfig:
    return dataclasses.replace(cfg, n_tok=n_tok)


def zipf_ranks(cfg: MoEConfig, layer: int = 0) -> np.ndarray:
    """Seeded permutation r_e of 1..E (rank 1 = hottest expert)."""
    key = stream_key(cfg.seed, layer, T_RANK)
    h = hash_t(key, torch.arange(cfg.n_experts, dtype=torch.int64)).numpy()
    order = np.argsort(h, kind="stable")
    ranks = np.empty(cfg.n_experts, dtype=np.int64)
    ranks[order] = np.arange(1, cfg.n_experts + 1)
    return ranks


def router(cfg: MoEConfig, layer: int = 0, device="cpu"):
    """Router weight [E, H] N(0, .02) and correction bias [E] float32."""
    wr = normal(stream_key(cfg.seed, layer, T_WR), (cfg.n_experts, cfg.hidden), cfg.wr_sigma,
                device)
    if cfg.bias_kind == "zero":
        b = torch.zeros(cfg.n_experts, dtype=torch.float32)
    else:
        b = normal(stream_key(cfg.seed, layer, T_BIAS), (cfg.n_experts,), cfg.b_sigma, "cpu")
        if cfg.bias_kind == "zipf":
            # Zipf(s=1.1)-shaped skew over a seeded rank permutation, amplitude 0.6
            r = zipf_ranks(cfg, layer).astype(np.float64)
            b = torch.from_numpy((b.numpy().astype(np.float64) + 0.6 * r ** -1.1)
                                 .astype(np.float32))
    return wr, b.to(device)


def expert_matrix(cfg: MoEConfig, layer: int, expert: int, which: str, device="cpu",
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 weight of one expert matrix: gate/up [I, H], down [H, I] (out x in)."""
    tid = {"gate": T_GATE, "up": T_UP, "down": T_DOWN}[which]
    shape = (cfg.inter, cfg.hidden) if which != "down" else (cfg.hidden, cfg.inter)
    return normal(stream_key(cfg.seed, layer, tid, expert), shape, cfg.w_sigma, device, out)


def activations(cfg: MoEConfig, layer: int = 0, device="cpu", n_tok: Optional[int] = None,
                first_tok: int = 0) -> torch.Tensor:
    """Raw layer input [T, H] float32 (before any RMSNorm).

    Tokens are addressable: token t of the stream is row t, so a bench can draw
    many distinct tokens and a test can draw a window of them.
    """
    T = cfg.n_tok if n_tok is None else n_tok
    H = cfg.hidden
    dev = torch.device(device)
    idx0 = first_tok * H
    key = stream_key(cfg.seed, layer, T_X)
    x = torch.empty((T, H), dtype=torch.float32, device=dev)
    tab = normal_table(dev)
    idx = torch.arange(idx0, idx0 + T * H, dtype=torch.int64, device=dev)
    x.view(-1)[:] = tab[_srl(hash_t(key, idx), 48)]
    if cfg.correlated:
        # one shared component per token group, token-independent noise on top
        zkey = stream_key(cfg.seed, layer, T_XSHARED)
        zi = torch.arange(0, H, dtype=torch.int64, device=dev)
        z = tab[_srl(hash_t(zkey, zi), 48)]
        x = z.unsqueeze(0) * torch.tensor(0.7, dtype=torch.float32, device=dev) + \
            x * torch.tensor(0.3, dtype=torch.float32, device=dev)
    return x.contiguous()


def build_layer(cfg: MoEConfig, layer: int, device, pack_into, experts=None, bits: int = 4):
    """Draw a layer's expert weights matrix by matrix on `device` and hand each
    fp32 matrix to the caller's packer, pack_into(w, q_view, s_view), which
    fills the boundary blobs (q_view holds `bits`-wide codes: cols * bits / 8
    bytes per row). This module does no packing itself.

    Returns (w_router [E,H], bias [E], experts_q u8 [(E+S)*3*I*H*bits/8],
    experts_scale f32 [(E+S)*(2I+H)]). Experts not in `experts` stay unset.
    """
    dev = torch.device(device)
    H, I = cfg.hidden, cfg.inter
    n = cfg.n_experts + cfg.n_shared
    mb = I * H * bits // 8  # bytes of one packed matrix
    bq, bs = 3 * mb, 2 * I + H
    q = torch.empty(n * bq, dtype=torch.uint8, device=dev)
    s = torch.empty(n * bs, dtype=torch.float32, device=dev)
    buf_gu = torch.empty((I, H), dtype=torch.float32, device=dev)
    buf_d = torch.empty((H, I), dtype=torch.float32, device=dev)
    parts = (("gate", I, H, 0, 0, buf_gu), ("up", I, H, mb, I, buf_gu),
             ("down", H, I, 2 * mb, 2 * I, buf_d))
    for e in (range(n) if experts is None else experts):
        for which, rows, cols, qo, so, buf in parts:
            w = expert_matrix(cfg, layer, e, which, dev, out=buf)
            rb = cols * bits // 8
            qv = q[e * bq + qo:e * bq + qo + rows * rb].view(rows, rb)
            sv = s[e * bs + so:e * bs + so + rows]
            pack_into(w, qv, sv)
    wr, b = router(cfg, layer, dev)
    return wr, b, q, s
