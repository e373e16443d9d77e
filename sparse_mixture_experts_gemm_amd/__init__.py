"""Python binding of the MI355X MoE FFN layer library (libmoe_hip.so).

Argument marshalling only: every stage runs in the library's HIP kernels.
torch provides device memory and streams.  The binding refuses to run when
the library is missing; there is no fallback.

Entry points mirror the C ABI in include/moe.h: route, dispatch, expert_ffn,
combine, forward (and forward_events), the one-byte-weight variants, plus
capacity / max_rows / workspace sizing.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch  # load torch's HIP runtime before the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_TOO_LARGE = 0, -1, -2, -3, -4
STATIC_SCRATCH_BYTES = 32 << 20  # MOE_STATIC_SCRATCH_BYTES: the array behind forward_noalloc
MOE_F32, MOE_BF16 = 0, 1


class MoEError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {code} ({strerror(code)})")
        self.code = code


class MoeParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float), ("reroute", ctypes.c_int32),
                ("lam", ctypes.c_float), ("aux_coef", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("gate_temperature", ctypes.c_float), ("top2_gap", ctypes.c_float),
                ("router_hidden", ctypes.c_int32), ("dynamic_capacity", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("cand", "cand_score", "eid", "pos", "row", "flag", "gate", "offsets",
                 "token_of_row", "demand", "kept", "totals", "aux_loss")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(MoeParams)
        PR = ctypes.POINTER(MoeRouting)
        L.moe_capacity.argtypes = [PP]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_max_rows.argtypes = [PP]
        L.moe_max_rows.restype = ctypes.c_int64
        L.moe_ffn_workspace_bytes.argtypes = [PP]
        L.moe_ffn_workspace_bytes.restype = ctypes.c_size_t
        L.moe_dispatch_workspace_bytes.argtypes = [PP]
        L.moe_dispatch_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [PP]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_route.argtypes = [PP, P, P, P, P, P, PR, P]
        L.moe_dispatch.argtypes = [PP, P, PR, P, P, ctypes.c_size_t, P]
        L.moe_expert_ffn.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_combine.argtypes = [PP, P, P, P, P, P]
        L.moe_forward.argtypes = [PP, P, P, P, P, P, P, P, P, P, PR, P, ctypes.c_size_t, P]
        L.moe_forward_events.argtypes = [PP, P, P, P, P, P, P, P, P, P, PR, P, ctypes.c_size_t, P,
                                         ctypes.POINTER(ctypes.c_void_p)]
        L.moe_forward_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, PR, P]
        L.moe_load_window_workspace_bytes.argtypes = [PP, ctypes.c_int32]
        L.moe_load_window_workspace_bytes.restype = ctypes.c_size_t
        L.moe_load_window.argtypes = [PP, P, ctypes.c_int32, ctypes.c_float, P, P, ctypes.c_size_t, P]
        L.moe_load_window.restype = ctypes.c_int
        L.moe_backward_workspace_bytes.argtypes = [PP]
        L.moe_backward_workspace_bytes.restype = ctypes.c_size_t
        L.moe_backward.argtypes = [PP, P, P, P, P, P, PR, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_expert_ffn_fp8.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P]
        L.moe_forward_fp8.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, PR, P, ctypes.c_size_t, P]
        L.moe_expert_ffn_i8.argtypes = L.moe_expert_ffn_fp8.argtypes
        L.moe_forward_i8.argtypes = L.moe_forward_fp8.argtypes
        L.moe_expert_ffn_i4.argtypes = L.moe_expert_ffn_fp8.argtypes
        L.moe_forward_i4.argtypes = L.moe_forward_fp8.argtypes
        for f in (L.moe_expert_ffn_i8, L.moe_forward_i8):
            f.restype = ctypes.c_int
        for f in (L.moe_route, L.moe_dispatch, L.moe_expert_ffn, L.moe_combine, L.moe_forward,
                  L.moe_forward_events, L.moe_forward_noalloc, L.moe_expert_ffn_fp8, L.moe_forward_fp8,
                  L.moe_backward):
            f.restype = ctypes.c_int
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


@dataclass
class Params:
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    capacity_factor: float = 1.0
    reroute: int = 1
    lam: float = 0.0
    aux_coef: float = 0.01
    dtype: int = MOE_BF16
    gate_temperature: float = 0.0  # 0: plain softmax gates
    top2_gap: float = 0.0          # 0: no top-2 gap threshold
    router_hidden: int = 0         # 0: linear router; H: two-layer router (w_router = W1 [H][d] then W2 [E][H])
    dynamic_capacity: int = 0      # 1: capacity factor 1 + 0.01 log2(T), capacity_factor ignored

    def c(self) -> MoeParams:
        return MoeParams(self.T, self.d, self.E, self.k, self.d_ff, self.capacity_factor,
                         self.reroute, self.lam, self.aux_coef, self.dtype, self.gate_temperature,
                         self.top2_gap, self.router_hidden, self.dynamic_capacity)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == MOE_BF16 else torch.float32


def capacity(p: Params) -> int:
    return int(lib().moe_capacity(ctypes.byref(p.c())))


def max_rows(p: Params) -> int:
    return int(lib().moe_max_rows(ctypes.byref(p.c())))


def ffn_workspace_bytes(p: Params) -> int:
    """Scratch bytes moe_expert_ffn needs (0: none)."""
    return int(lib().moe_ffn_workspace_bytes(ctypes.byref(p.c())))


def alloc_y_perm(p: Params, device="cuda"):
    """y_perm [R, d] fp32 for moe_expert_ffn / moe_combine."""
    return torch.empty((max(max_rows(p), 1), p.d), dtype=torch.float32, device=device)


def dispatch_workspace_bytes(p: Params) -> int:
    return int(lib().moe_dispatch_workspace_bytes(ctypes.byref(p.c())))


def workspace_bytes(p: Params) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(p.c())))


class Routing:
    """Device tensors of the routing arrays (layouts as in include/moe.h)."""

    NAMES = ("cand", "cand_score", "eid", "pos", "row", "flag", "gate", "offsets",
             "token_of_row", "demand", "kept", "totals", "aux_loss")

    def __init__(self, p: Params, device="cuda"):
        T, E, k = p.T, p.E, p.k
        R = max(max_rows(p), 0)
        i32, f32 = torch.int32, torch.float32
        self.cand = torch.empty((T, k + 1), dtype=i32, device=device)
        self.cand_score = torch.empty((T, k + 1), dtype=f32, device=device)
        self.eid = torch.empty((T, k), dtype=i32, device=device)
        self.pos = torch.empty((T, k), dtype=i32, device=device)
        self.row = torch.empty((T, k), dtype=i32, device=device)
        self.flag = torch.empty((T, k), dtype=torch.uint8, device=device)
        self.gate = torch.empty((T, k), dtype=f32, device=device)
        self.offsets = torch.empty(E + 1, dtype=i32, device=device)
        self.token_of_row = torch.empty(max(R, 1), dtype=i32, device=device)
        self.demand = torch.empty(E, dtype=i32, device=device)
        self.kept = torch.empty(E, dtype=i32, device=device)
        self.totals = torch.empty(3, dtype=i32, device=device)
        self.aux_loss = torch.empty(1, dtype=f32, device=device)
        self.R = R

    def c(self) -> MoeRouting:
        return MoeRouting(*[getattr(self, n).data_ptr() for n in self.NAMES])

    def cpu(self) -> dict:
        out = {n: getattr(self, n).cpu() for n in self.NAMES}
        out["token_of_row"] = out["token_of_row"][: self.R]
        return out


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoEError(rc, what)


def route(p: Params, x, w_router, bias, load, logits, r: Routing, stream=None):
    rc = lib().moe_route(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                         _ptr(logits), ctypes.byref(r.c()), _stream(stream))
    _check(rc, "moe_route")


def dispatch(p: Params, x, r: Routing, x_perm, workspace, stream=None):
    rc = lib().moe_dispatch(ctypes.byref(p.c()), _ptr(x), ctypes.byref(r.c()), _ptr(x_perm),
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_dispatch")


def expert_ffn(p: Params, x_perm, offsets, w1, w3, w2, h, y_perm, workspace=None, stream=None):
    """Stage 3.  workspace: a uint8 tensor of at least ffn_workspace_bytes(p)
    bytes (None when that is 0)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().moe_expert_ffn(ctypes.byref(p.c()), _ptr(x_perm), _ptr(offsets), _ptr(w1), _ptr(w3),
                              _ptr(w2), _ptr(h), _ptr(y_perm), _ptr(workspace), nbytes, _stream(stream))
    _check(rc, "moe_expert_ffn")


def combine(p: Params, y_perm, row, gate, y, stream=None):
    rc = lib().moe_combine(ctypes.byref(p.c()), _ptr(y_perm), _ptr(row), _ptr(gate), _ptr(y),
                           _stream(stream))
    _check(rc, "moe_combine")


def forward(p: Params, x, w_router, bias, load, w1, w3, w2, y, logits, r: Routing, workspace,
            stream=None):
    rc = lib().moe_forward(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                           _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y), _ptr(logits), ctypes.byref(r.c()),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(stream))
    _check(rc, "moe_forward")


def forward_noalloc(p: Params, x, w_router, bias, load, w1, w3, w2, y, logits, r: Routing, stream=None):
    """moe_forward on the library's static scratch array (no workspace, no allocation)."""
    rc = lib().moe_forward_noalloc(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                                   _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y), _ptr(logits), ctypes.byref(r.c()),
                                   _stream(stream))
    _check(rc, "moe_forward_noalloc")


def forward_events(p: Params, x, w_router, bias, load, w1, w3, w2, y, logits, r: Routing, workspace, events,
                   stream=None):
    """moe_forward with six timing events (torch.cuda.Event, enable_timing) recorded before the route,
    dispatch, gate-up GEMM, down GEMM and combine, and after the combine."""
    for e in events:
        if e is not None and not e.cuda_event:
            e.record()  # torch creates the HIP event on its first record
    ev = (ctypes.c_void_p * 6)(*[e.cuda_event if e is not None else None for e in events])
    rc = lib().moe_forward_events(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                                  _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y), _ptr(logits), ctypes.byref(r.c()),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream), ev)
    _check(rc, "moe_forward_events")


def expert_ffn_fp8(p: Params, x_perm, offsets, q1, s1, q3, s3, q2, s2, h, y_perm, stream=None):
    """Stage 3 with one-byte (E4M3) expert weights and fp32 row scales."""
    rc = lib().moe_expert_ffn_fp8(ctypes.byref(p.c()), _ptr(x_perm), _ptr(offsets), _ptr(q1), _ptr(s1),
                                  _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(h), _ptr(y_perm),
                                  _stream(stream))
    _check(rc, "moe_expert_ffn_fp8")


def forward_fp8(p: Params, x, w_router, bias, load, q1, s1, q3, s3, q2, s2, y, logits, r: Routing,
                workspace, stream=None):
    """The layer with one-byte (E4M3) expert weights and fp32 row scales."""
    rc = lib().moe_forward_fp8(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                               _ptr(q1), _ptr(s1), _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(y),
                               _ptr(logits), ctypes.byref(r.c()), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_forward_fp8")


def expert_ffn_i8(p: Params, x_perm, offsets, q1, s1, q3, s3, q2, s2, h, y_perm, stream=None):
    """Stage 3 with INT8 expert weights and fp32 row scales."""
    rc = lib().moe_expert_ffn_i8(ctypes.byref(p.c()), _ptr(x_perm), _ptr(offsets), _ptr(q1), _ptr(s1),
                                 _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(h), _ptr(y_perm), _stream(stream))
    _check(rc, "moe_expert_ffn_i8")


def forward_i8(p: Params, x, w_router, bias, load, q1, s1, q3, s3, q2, s2, y, logits, r: Routing,
               workspace, stream=None):
    """The layer with INT8 expert weights and fp32 row scales."""
    rc = lib().moe_forward_i8(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                              _ptr(q1), _ptr(s1), _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(y),
                              _ptr(logits), ctypes.byref(r.c()), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_forward_i8")


def expert_ffn_i4(p: Params, x_perm, offsets, q1, s1, q3, s3, q2, s2, h, y_perm, stream=None):
    """Stage 3 with INT4 expert weights (two codes per byte) and fp32 row
    scales."""
    rc = lib().moe_expert_ffn_i4(ctypes.byref(p.c()), _ptr(x_perm), _ptr(offsets), _ptr(q1), _ptr(s1),
                                 _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(h), _ptr(y_perm), _stream(stream))
    _check(rc, "moe_expert_ffn_i4")


def forward_i4(p: Params, x, w_router, bias, load, q1, s1, q3, s3, q2, s2, y, logits, r: Routing,
               workspace, stream=None):
    """The layer with INT4 expert weights (two codes per byte) and fp32 row
    scales."""
    rc = lib().moe_forward_i4(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(load),
                              _ptr(q1), _ptr(s1), _ptr(q3), _ptr(s3), _ptr(q2), _ptr(s2), _ptr(y),
                              _ptr(logits), ctypes.byref(r.c()), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_forward_i4")


def alloc_workspace(p: Params, device="cuda", dispatch_only: bool = False, ffn_only: bool = False) -> torch.Tensor:
    """Workspace of moe_forward, or of moe_dispatch / moe_expert_ffn alone."""
    n = dispatch_workspace_bytes(p) if dispatch_only else ffn_workspace_bytes(p) if ffn_only else workspace_bytes(p)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def backward_workspace_bytes(p: Params) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(p.c())))


class Grads:
    """fp32 gradient tensors of the backward pass (layouts as in include/moe.h)."""

    NAMES = ("dx", "dlogits", "dw_router", "dbias", "dw1", "dw3", "dw2")

    def __init__(self, p: Params, device="cuda"):
        f32 = torch.float32
        self.dx = torch.empty((p.T, p.d), dtype=f32, device=device)
        self.dlogits = torch.empty((p.T, p.E), dtype=f32, device=device)
        self.dw_router = torch.empty((p.E, p.d), dtype=f32, device=device)
        self.dbias = torch.empty(p.E, dtype=f32, device=device)
        self.dw1 = torch.empty((p.E, p.d_ff, p.d), dtype=f32, device=device)
        self.dw3 = torch.empty((p.E, p.d_ff, p.d), dtype=f32, device=device)
        self.dw2 = torch.empty((p.E, p.d, p.d_ff), dtype=f32, device=device)


def backward(p: Params, x, w_router, w1, w3, w2, r: Routing, dy, g: Grads, workspace, stream=None):
    """Gradients of the layer with the forward routing r held fixed (bf16 layers)."""
    rc = lib().moe_backward(ctypes.byref(p.c()), _ptr(x), _ptr(w_router), _ptr(w1), _ptr(w3), _ptr(w2),
                            ctypes.byref(r.c()), _ptr(dy), _ptr(g.dx), _ptr(g.dlogits), _ptr(g.dw_router),
                            _ptr(g.dbias), _ptr(g.dw1), _ptr(g.dw3), _ptr(g.dw2), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_backward")


def alloc_backward_workspace(p: Params, device="cuda") -> torch.Tensor:
    return torch.empty(max(backward_workspace_bytes(p), 256), dtype=torch.uint8, device=device)


def load_window_workspace_bytes(p: Params, window: int) -> int:
    return int(lib().moe_load_window_workspace_bytes(ctypes.byref(p.c()), int(window)))


def load_window(p: Params, cand, window: int, decay: float, load, workspace=None, stream=None):
    """Windowed load statistic: updates the fp32 [E] tensor `load` in place from the router's cand."""
    if workspace is None:
        workspace = torch.empty(max(load_window_workspace_bytes(p, window), 256), dtype=torch.uint8,
                                device=load.device)
    rc = lib().moe_load_window(ctypes.byref(p.c()), _ptr(cand), int(window), float(decay), _ptr(load),
                               _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "moe_load_window")
