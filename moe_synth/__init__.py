"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module only draws numbers: it holds none of the layer's arithmetic
(no routing, no capacity, no GEMM).  Both the CPU oracle and the HIP path
consume tensors made here; a tensor is generated once, on one device, and the
same bits are handed to both sides.

Generator (published definitions, implemented here from them):
  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014) used as a counter-based hash: draw i of a
    stream with key K is mix64(K + (i + 1) * GAMMA), GAMMA = 0x9E3779B97F4A7C15.
  * Stream key per tensor: K = mix64(seed * GAMMA + tag), one tag per tensor.
  * Normals: Box-Muller (1958) on pairs of draws, in float64:
      u1 = ((z0 >> 11) + 1) * 2^-53  in (0, 1],  u2 = (z1 >> 11) * 2^-53 in [0, 1)
      n0 = sqrt(-2 ln u1) cos(2 pi u2),  n1 = sqrt(-2 ln u1) sin(2 pi u2)
  * Scaled by the tensor's standard deviation, rounded to fp32, then (bf16
    tensors) rounded to bfloat16 with round-to-nearest-even.

All integer work is done in int64 torch tensors: multiplication wraps modulo
2^64 and right shifts are made logical with a mask, so the integer stream is
identical on every device.  The float64 transcendental functions may differ in
the last bit between devices, which is why a tensor is drawn once and shared.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# one substream per tensor
TAGS = {"x": 1, "x_prev": 2, "w_router": 3, "bias": 4, "w1": 5, "w3": 6, "w2": 7, "dy": 8}


def _s64(v: int) -> int:
    """Python int in [0, 2^64) -> the int64 with the same bits."""
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (reference for the tensor version)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bits."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(MIX1)
    z = (z ^ _lsr(z, 27)) * _s64(MIX2)
    return z ^ _lsr(z, 31)


def stream_key(seed: int, tag: int) -> int:
    return mix64_int((seed * GAMMA + tag) & MASK64)


def raw_draws(key: int, start: int, n: int, device) -> torch.Tensor:
    """Draws start .. start+n-1 of the stream as int64 bit patterns."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    return _mix64(i * _s64(GAMMA) + _s64(key))


def normals(seed: int, tag: int, n: int, device, chunk: int = 1 << 25) -> torch.Tensor:
    """n standard normals (float64) of substream (seed, tag)."""
    key = stream_key(seed, tag)
    out = torch.empty(n, dtype=torch.float64, device=device)
    npairs = (n + 1) // 2
    two_pi = 2.0 * math.pi
    for p0 in range(0, npairs, chunk):
        p1 = min(npairs, p0 + chunk)
        z = raw_draws(key, 2 * p0, 2 * (p1 - p0), device).view(-1, 2)
        u1 = (_lsr(z[:, 0], 11) + 1).to(torch.float64) * 2.0 ** -53
        u2 = _lsr(z[:, 1], 11).to(torch.float64) * 2.0 ** -53
        r = torch.sqrt(-2.0 * torch.log(u1))
        th = two_pi * u2
        pair = torch.stack((r * torch.cos(th), r * torch.sin(th)), dim=1).reshape(-1)
        lo = 2 * p0
        hi = min(n, 2 * p1)
        out[lo:hi] = pair[: hi - lo]
    return out


def normal_tensor(seed: int, name: str, shape, std: float, dtype: torch.dtype, device) -> torch.Tensor:
    n = 1
    for s in shape:
        n *= int(s)
    v = normals(seed, TAGS[name], n, device) * std
    return v.to(torch.float32).to(dtype).reshape(tuple(shape))


@dataclass
class MoEConfig:
    """Shape and routing parameters of one synthetic MoE layer."""
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    cf: float
    dtype: str                      # "f32" or "bf16"
    bias: str = "none"              # "none" | "normal" | "hot0"
    bias_std: float = 0.0
    bias_hot: float = 0.0
    lam: float = 0.0
    load_from_prev: bool = False    # load vector = previous batch's kept fraction
    reroute: int = 1
    aux_coef: float = 0.01
    tau: float = 0.0                # gate temperature (0: plain softmax)
    gap: float = 0.0                # top-2 gap threshold (0: off)
    dyn_cap: int = 0                # 1: capacity factor 1 + 0.01 log2(T) (cf ignored)
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads: shapes, value distributions and router extras.
CONFIGS = {
    "tiny": MoEConfig("tiny", T=64, d=128, E=8, k=2, d_ff=256, cf=1.0, dtype="f32",
                      note="tiny fp32 layer, no load penalty"),
    "mixtral": MoEConfig("mixtral", T=4096, d=4096, E=8, k=2, d_ff=14336, cf=1.25, dtype="bf16",
                         note="Mixtral-shape prefill, balanced routing"),
    "fine64": MoEConfig("fine64", T=8192, d=4096, E=64, k=2, d_ff=2048, cf=1.0, dtype="bf16",
                        bias="normal", bias_std=math.sqrt(0.5),
                        note="fine-grained many-expert layer, per-expert bias N(0, 0.5)"),
    "skew": MoEConfig("skew", T=2048, d=2048, E=16, k=2, d_ff=5632, cf=1.0, dtype="bf16",
                      bias="hot0", bias_hot=3.0, lam=0.3, load_from_prev=True,
                      note="skewed-load capping stress: expert 0 bias +3.0, lambda 0.3"),
    "decode": MoEConfig("decode", T=64, d=4096, E=8, k=2, d_ff=14336, cf=1.25, dtype="bf16",
                        note="decode-shape weight-streaming layer"),
}


def make_layer(cfg: MoEConfig, device="cpu", seed: int = 0, T: Optional[int] = None,
               want=("x", "w_router", "bias", "w1", "w3", "w2", "x_prev")) -> dict:
    """Draw the layer's tensors.

    x ~ N(0, 1); W_router, W1, W3 ~ N(0, 1/d); W2 ~ N(0, 1/d_ff); bias per the
    config (fp32).  Layouts: x [T, d], W_router [E, d], W1/W3 [E, d_ff, d],
    W2 [E, d, d_ff], bias [E].  `T` overrides the token count (x only).
    """
    T = cfg.T if T is None else T
    dt = cfg.torch_dtype
    out = {}
    sd = 1.0 / math.sqrt(cfg.d)
    sf = 1.0 / math.sqrt(cfg.d_ff)
    if "x" in want:
        out["x"] = normal_tensor(seed, "x", (T, cfg.d), 1.0, dt, device)
    if "x_prev" in want and cfg.load_from_prev:
        out["x_prev"] = normal_tensor(seed, "x_prev", (T, cfg.d), 1.0, dt, device)
    if "w_router" in want:
        out["w_router"] = normal_tensor(seed, "w_router", (cfg.E, cfg.d), sd, dt, device)
    if "bias" in want:
        if cfg.bias == "normal":
            out["bias"] = normal_tensor(seed, "bias", (cfg.E,), cfg.bias_std, torch.float32, device)
        elif cfg.bias == "hot0":
            b = torch.zeros(cfg.E, dtype=torch.float32, device=device)
            b[0] = cfg.bias_hot
            out["bias"] = b
        else:
            out["bias"] = None
    if "w1" in want:
        out["w1"] = normal_tensor(seed, "w1", (cfg.E, cfg.d_ff, cfg.d), sd, dt, device)
    if "w3" in want:
        out["w3"] = normal_tensor(seed, "w3", (cfg.E, cfg.d_ff, cfg.d), sd, dt, device)
    if "w2" in want:
        out["w2"] = normal_tensor(seed, "w2", (cfg.E, cfg.d, cfg.d_ff), sf, dt, device)
    return out


def quantize_rows_e4m3(w: torch.Tensor):
    """Synthetic one-byte weights from a weight tensor [..., rows, cols]: an
    fp32 scale per row, amax / 448 (448 is the largest E4M3 value; 1 for an
    all-zero row), and the E4M3 codes of w / scale by torch's round-to-nearest
    conversion.  Returns (codes uint8 [..., rows, cols], scales fp32 [..., rows]).
    """
    wf = w.float()
    amax = wf.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (wf / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.contiguous(), s.contiguous()


def quantize_rows_int8(w: torch.Tensor):
    """Synthetic INT8 weights from a weight tensor [..., rows, cols]: an fp32
    scale per row, amax / 127 (1 for an all-zero row), and the codes
    round-half-even(w / scale) in [-127, 127].  Returns (codes int8
    [..., rows, cols], scales fp32 [..., rows])."""
    wf = w.float()
    amax = wf.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax))
    q = torch.round(wf / s[..., None]).clamp_(-127, 127).to(torch.int8)
    return q.contiguous(), s.contiguous()


def quantize_rows_int4(w: torch.Tensor):
    """Synthetic INT4 weights from a weight tensor [..., rows, cols] (cols
    even): an fp32 scale per row, amax / 7 (1 for an all-zero row), the codes
    round-half-even(w / scale) in [-7, 7], packed two per byte, element 2j in
    the low nibble of byte j (two's complement nibbles).  Returns (packed
    uint8 [..., rows, cols / 2], scales fp32 [..., rows])."""
    wf = w.float()
    amax = wf.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax))
    q = torch.round(wf / s[..., None]).clamp_(-7, 7).to(torch.int32) & 15
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8)
    return packed.contiguous(), s.contiguous()


def upstream_grad(cfg: MoEConfig, device="cpu", seed: int = 0, T: Optional[int] = None) -> torch.Tensor:
    """Upstream gradient dy [T, d] of the layer output for the backward pass:
    N(0, 1) in the layer's dtype, substream "dy"."""
    T = cfg.T if T is None else T
    return normal_tensor(seed, "dy", (T, cfg.d), 1.0, cfg.torch_dtype, device)
