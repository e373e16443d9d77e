"""CPU oracle of the sparse MoE FFN layer forward (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The arithmetic lives in ``moe_oracle.c`` (plain
C, double accumulation); this module only marshals numpy arrays through
ctypes.  It shares nothing with the HIP path.

Array conventions: fp32 arrays are ``np.float32``; bfloat16 arrays are the
raw bit patterns as ``np.uint16``.  torch CPU tensors are accepted and viewed
the same way.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_set_num_threads.restype = None
        L.oracle_capacity.argtypes = [i64, i64, i64, f64]
        L.oracle_capacity.restype = i64
        L.oracle_router_logits.argtypes = [i32, i32, i32, i32, P, P, P, P]
        L.oracle_scores.argtypes = [i32, i32, P, P, f32, P]
        L.oracle_topk.argtypes = [i32, i32, i32, P, P, P]
        L.oracle_gap_swap.argtypes = [i32, i32, f32, P, P]
        L.oracle_router_logits_glu.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_dispatch.argtypes = [i32, i32, i32, i64, i32, f32, ctypes.c_double, P, P] + [P] * 12
        L.oracle_ffn_rows.argtypes = [i32, P, P, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_layer_tokens.argtypes = [i32, P, i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_combine.argtypes = [i32, i32, i32, i32, P, P, P, P]
        L.oracle_dynamic_capacity_factor.argtypes = [i64]
        L.oracle_dynamic_capacity_factor.restype = f64
        L.oracle_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_e4m3_value.restype = f64
        L.oracle_fp8_e4m3_decode.argtypes = [i64, P, P]
        L.oracle_dequant_rows.argtypes = [i64, i64, P, P, P]
        L.oracle_dequant_rows_i8.argtypes = [i64, i64, P, P, P]
        L.oracle_dequant_rows_i8.restype = None
        L.oracle_dequant_rows_i4.argtypes = [i64, i64, P, P, P]
        L.oracle_dequant_rows_i4.restype = None
        L.oracle_backward_tokens.argtypes = [i32, P, i32, i32, i32, i32, i32, f64, P, P, P, P, P, P, P, P, P, P]
        L.oracle_backward_expert_units.argtypes = [i32, i32, P, i32, P, P, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.oracle_router_wgrad.argtypes = [i32, i32, i32, i32, P, P, P, P]
        L.oracle_load_window.argtypes = [i32, i32, i32, i32, P, i32, f64, P]
        L.oracle_load_window.restype = None
        for f in (L.oracle_backward_tokens, L.oracle_backward_expert_units, L.oracle_router_wgrad):
            f.restype = None
        for f in (L.oracle_router_logits, L.oracle_router_logits_glu, L.oracle_scores, L.oracle_topk, L.oracle_gap_swap, L.oracle_dispatch,
                  L.oracle_ffn_rows, L.oracle_layer_tokens, L.oracle_combine, L.oracle_fp8_e4m3_decode,
                  L.oracle_dequant_rows):
            f.restype = None
        _lib = L
    return _lib


def _np(a):
    """numpy view of an array-like; torch bf16 becomes its uint16 bits."""
    if a is None:
        return None
    if not isinstance(a, np.ndarray):
        import torch  # only for tensors handed in by a caller
        if isinstance(a, torch.Tensor):
            t = a.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        a = np.asarray(a)
    return np.ascontiguousarray(a)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"oracle element type must be float32, bf16 bits or float64, got {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))


def capacity(T: int, k: int, E: int, cf: float) -> int:
    return int(lib().oracle_capacity(T, k, E, float(np.float32(cf))))


def dynamic_capacity_factor(T: int) -> float:
    return float(lib().oracle_dynamic_capacity_factor(T))


def capacity_dynamic(T: int, k: int, E: int) -> int:
    """Capacity under the dynamic factor (double throughout)."""
    return int(lib().oracle_capacity(T, k, E, dynamic_capacity_factor(T)))


def router_logits(x, wr, bias=None) -> np.ndarray:
    x, wr = _np(x), _np(wr)
    bias = None if bias is None else _np(bias).astype(np.float32)
    T, d = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, d) and x.dtype == wr.dtype
    raw = np.empty((T, E), np.float32)
    lib().oracle_router_logits(T, d, E, _dt(x), _p(x), _p(wr), _p(bias), _p(raw))
    return raw


def router_logits_glu(x, w1, w2, bias=None, bias1=None) -> np.ndarray:
    """Two-layer router: raw = silu(x W1^T + bias1) W2^T + bias, W1 [H][d],
    W2 [E][H], bias1 [H] and bias [E] (either may be None)."""
    x, w1, w2 = _np(x), _np(w1), _np(w2)
    bias = None if bias is None else np.ascontiguousarray(_np(bias), dtype=np.float32)
    bias1 = None if bias1 is None else np.ascontiguousarray(_np(bias1), dtype=np.float32)
    T, d = x.shape
    H = w1.shape[0]
    E = w2.shape[0]
    assert w1.shape == (H, d) and w2.shape == (E, H) and x.dtype == w1.dtype == w2.dtype
    assert bias1 is None or bias1.shape == (H,)
    raw = np.empty((T, E), np.float32)
    lib().oracle_router_logits_glu(T, d, E, H, _dt(x), _p(x), _p(w1), _p(w2), _p(bias1), _p(bias), _p(raw))
    return raw


def scores(raw, load=None, lam: float = 0.0) -> np.ndarray:
    raw = _np(raw).astype(np.float32)
    load = None if load is None else _np(load).astype(np.float32)
    T, E = raw.shape
    s = np.empty_like(raw)
    lib().oracle_scores(T, E, _p(raw), _p(load), float(np.float32(lam)), _p(s))
    return s


def topk(s, K: int):
    s = _np(s).astype(np.float32)
    T, E = s.shape
    cand = np.empty((T, K), np.int32)
    cs = np.empty((T, K), np.float32)
    lib().oracle_topk(T, E, K, _p(s), _p(cand), _p(cs))
    return cand, cs


def gap_swap(cand, cand_score, delta: float):
    """Top-2 gap threshold: ranks 1 and 2 swapped where s[0] - s[1] < delta (fp32)."""
    cand = np.ascontiguousarray(_np(cand).astype(np.int32))
    cs = np.ascontiguousarray(_np(cand_score).astype(np.float32))
    T, K = cand.shape
    lib().oracle_gap_swap(T, K, float(np.float32(delta)), _p(cand), _p(cs))
    return cand, cs


def route(raw, k: int, load=None, lam: float = 0.0, gap: float = 0.0):
    """Scores and top-(k+1) candidates from fp32 router logits, then the
    top-2 gap threshold when gap > 0."""
    s = scores(raw, load, lam)
    cand, cs = topk(s, k + 1)
    if gap > 0:
        cand, cs = gap_swap(cand, cs, gap)
    return cand, cs


def dispatch(cand, cand_score, E: int, k: int, C: int, reroute: int = 1, aux_coef: float = 0.01,
             tau: float = 1.0) -> dict:
    """Capacity-capped dispatch; gates are the softmax of score / tau over the kept slots."""
    cand = _np(cand).astype(np.int32)
    cs = _np(cand_score).astype(np.float32)
    T = cand.shape[0]
    assert cand.shape == (T, k + 1) and cs.shape == (T, k + 1)
    cap_rows = min(T * k, E * C)
    o = dict(
        eid=np.empty((T, k), np.int32), pos=np.empty((T, k), np.int32),
        flag=np.empty((T, k), np.uint8), row=np.empty((T, k), np.int32),
        gate=np.empty((T, k), np.float32), gate64=np.empty((T, k), np.float64),
        offsets=np.empty(E + 1, np.int32), token_of_row=np.empty(max(cap_rows, 0), np.int32),
        demand=np.empty(E, np.int32), kept=np.empty(E, np.int32),
        totals=np.empty(3, np.int32), aux_loss=np.empty(1, np.float32),
    )
    lib().oracle_dispatch(T, E, k, C, int(reroute), float(np.float32(aux_coef)), float(tau), _p(cand), _p(cs),
                          _p(o["eid"]), _p(o["pos"]), _p(o["flag"]), _p(o["row"]), _p(o["gate"]),
                          _p(o["gate64"]), _p(o["offsets"]), _p(o["token_of_row"]),
                          _p(o["demand"]), _p(o["kept"]), _p(o["totals"]), _p(o["aux_loss"]))
    return o


def fp8_e4m3_value(byte: int) -> float:
    """Value of one OCP E4M3 byte."""
    return float(lib().oracle_fp8_e4m3_value(int(byte)))


def fp8_e4m3_decode(q) -> np.ndarray:
    """Values (double) of an array of E4M3 bytes, same shape."""
    q = np.ascontiguousarray(_np(q), dtype=np.uint8)
    out = np.empty(q.shape, np.float64)
    lib().oracle_fp8_e4m3_decode(q.size, _p(q), _p(out))
    return out


def dequant_rows(q, scale) -> np.ndarray:
    """w[..., r, c] = scale[..., r] * value(q[..., r, c]) in double."""
    q = np.ascontiguousarray(_np(q), dtype=np.uint8)
    scale = np.ascontiguousarray(_np(scale), dtype=np.float32)
    assert scale.shape == q.shape[:-1]
    w = np.empty(q.shape, np.float64)
    lib().oracle_dequant_rows(scale.size, q.shape[-1], _p(q), _p(scale), _p(w))
    return w


def dequant_rows_i8(q, scale) -> np.ndarray:
    """w[..., r, c] = scale[..., r] * q[..., r, c] in double, q INT8 codes."""
    q = np.ascontiguousarray(_np(q), dtype=np.int8)
    scale = np.ascontiguousarray(_np(scale), dtype=np.float32)
    assert scale.shape == q.shape[:-1]
    w = np.empty(q.shape, np.float64)
    lib().oracle_dequant_rows_i8(scale.size, q.shape[-1], _p(q), _p(scale), _p(w))
    return w


def dequant_rows_i4(q, scale) -> np.ndarray:
    """w[..., r, c] = scale[..., r] * q[..., r, c] in double, q INT4 codes
    packed two per byte (element 2j in the low nibble of byte j): q has
    cols / 2 bytes per row, w has cols elements."""
    q = np.ascontiguousarray(_np(q), dtype=np.uint8)
    scale = np.ascontiguousarray(_np(scale), dtype=np.float32)
    assert scale.shape == q.shape[:-1]
    cols = 2 * q.shape[-1]
    w = np.empty(q.shape[:-1] + (cols,), np.float64)
    lib().oracle_dequant_rows_i4(scale.size, cols, _p(q), _p(scale), _p(w))
    return w


def ffn_rows(expert, src, x, w1, w3, w2, want_h: bool = False):
    """y[i] = FFN_{expert[i]}(x[src[i]]) in double; optionally the SwiGLU h."""
    expert = _np(expert).astype(np.int32)
    src = _np(src).astype(np.int32)
    x, w1, w3, w2 = _np(x), _np(w1), _np(w3), _np(w2)
    E, d_ff, d = w1.shape
    assert w3.shape == w1.shape and w2.shape == (E, d, d_ff) and x.shape[1] == d
    assert x.dtype == w1.dtype == w3.dtype == w2.dtype
    n = expert.shape[0]
    y = np.empty((n, d), np.float64)
    h = np.empty((n, d_ff), np.float64) if want_h else None
    lib().oracle_ffn_rows(n, _p(expert), _p(src), d, d_ff, _dt(x), _p(x), _p(w1), _p(w3), _p(w2),
                          _p(y), _p(h))
    return (y, h) if want_h else y


def layer_tokens(tokens, x, w1, w3, w2, eid, gate64) -> np.ndarray:
    """Layer output rows (double) for the listed tokens, from a routing."""
    tokens = _np(tokens).astype(np.int32)
    x, w1, w3, w2 = _np(x), _np(w1), _np(w3), _np(w2)
    eid = _np(eid).astype(np.int32)
    gate64 = _np(gate64).astype(np.float64)
    E, d_ff, d = w1.shape
    k = eid.shape[1]
    n = tokens.shape[0]
    y = np.empty((n, d), np.float64)
    lib().oracle_layer_tokens(n, _p(tokens), k, d, d_ff, _dt(x), _p(x), _p(w1), _p(w3), _p(w2),
                              _p(eid), _p(gate64), _p(y))
    return y


def combine(row, gate, y_rows) -> np.ndarray:
    row = _np(row).astype(np.int32)
    gate = _np(gate).astype(np.float32)
    y_rows = _np(y_rows)
    T, k = row.shape
    d = y_rows.shape[1]
    y = np.empty((T, d), np.float64)
    lib().oracle_combine(T, k, d, _dt(y_rows), _p(row), _p(gate), _p(y_rows), _p(y))
    return y


def forward(x, wr, bias, w1, w3, w2, E: int, k: int, cf: float, load=None, lam: float = 0.0,
            reroute: int = 1, aux_coef: float = 0.01, raw=None) -> dict:
    """The whole layer.  `raw` replaces the oracle's own router logits (parity
    mode: the oracle routes from the same fp32 logits as the device)."""
    x = _np(x)
    T = x.shape[0]
    if raw is None:
        raw = router_logits(x, wr, bias)
    cand, cs = route(raw, k, load, lam)
    C = capacity(T, k, E, cf)
    disp = dispatch(cand, cs, E, k, C, reroute, aux_coef)
    y = layer_tokens(np.arange(T, dtype=np.int32), x, w1, w3, w2, disp["eid"], disp["gate64"])
    out = dict(raw=raw, cand=cand, cand_score=cs, C=C, y=y)
    out.update(disp)
    return out


# ---------------------------------------------------------------- backward --
def backward_tokens(tokens, x, wr, w1, w3, w2, eid, gate64, dy, tau: float = 1.0):
    """Router-logit gradient dlogits [n, E] and input gradient dx [n, d]
    (double) for the listed tokens, the routing held fixed."""
    tokens = _np(tokens).astype(np.int32)
    x, wr, w1, w3, w2 = _np(x), _np(wr), _np(w1), _np(w3), _np(w2)
    assert x.dtype == wr.dtype == w1.dtype == w3.dtype == w2.dtype
    eid = _np(eid).astype(np.int32)
    gate64 = _np(gate64).astype(np.float64)
    dy = np.ascontiguousarray(_np(dy), dtype=np.float64)
    E, d_ff, d = w1.shape
    k = eid.shape[1]
    assert k <= 64 and dy.shape == (x.shape[0], d)
    n = tokens.shape[0]
    dl = np.empty((n, E), np.float64)
    dx = np.empty((n, d), np.float64)
    lib().oracle_backward_tokens(n, _p(tokens), d, E, k, d_ff, _dt(x), float(tau), _p(x), _p(wr), _p(w1),
                                 _p(w3), _p(w2), _p(eid), _p(gate64), _p(dy), _p(dl), _p(dx))
    return dl, dx


def backward_expert_units(e: int, fs, tok, g, x, w1, w3, w2, dy):
    """Weight gradients of expert e for the intermediate units fs: rows
    dW1[e][f], dW3[e][f] ([nf, d] each) and columns dW2[e][:, f] ([d, nf]).
    The expert's kept slots are (tok[r], g[r]) in row order."""
    fs = _np(fs).astype(np.int32)
    tok = _np(tok).astype(np.int32)
    g = np.ascontiguousarray(_np(g), dtype=np.float64)
    x, w1, w3, w2 = _np(x), _np(w1), _np(w3), _np(w2)
    dy = np.ascontiguousarray(_np(dy), dtype=np.float64)
    E, d_ff, d = w1.shape
    nf = fs.shape[0]
    dw1 = np.empty((nf, d), np.float64)
    dw3 = np.empty((nf, d), np.float64)
    dw2 = np.empty((d, nf), np.float64)
    lib().oracle_backward_expert_units(e, nf, _p(fs), tok.shape[0], _p(tok), _p(g), d, d_ff, _dt(x), _p(x),
                                       _p(w1), _p(w3), _p(w2), _p(dy), _p(dw1), _p(dw3), _p(dw2))
    return dw1, dw3, dw2


def router_wgrad(x, dlogits):
    """dW_r [E, d] = dlogits^T x and dbias [E] = column sums of dlogits."""
    x = _np(x)
    dlogits = np.ascontiguousarray(_np(dlogits), dtype=np.float64)
    T, d = x.shape
    E = dlogits.shape[1]
    dwr = np.empty((E, d), np.float64)
    db = np.empty(E, np.float64)
    lib().oracle_router_wgrad(T, d, E, _dt(x), _p(x), _p(dlogits), _p(dwr), _p(db))
    return dwr, db


def expert_slots(eid, row, gate64, e: int):
    """The kept slots of expert e in row order: (tokens, gates)."""
    eid, row = _np(eid), _np(row)
    t, j = np.nonzero(eid == e)
    order = np.argsort(row[t, j], kind="stable")
    return t[order].astype(np.int32), np.asarray(gate64)[t[order], j[order]].astype(np.float64)


def backward(x, wr, w1, w3, w2, eid, row, gate64, dy, tau: float = 1.0) -> dict:
    """The whole backward pass (small layers): dlogits, dx, dW_r, dbias, dW1,
    dW3, dW2 in double, the routing (eid, row, gate64 of the forward) fixed."""
    x = _np(x)
    T = x.shape[0]
    E, d_ff, d = _np(w1).shape
    dl, dx = backward_tokens(np.arange(T, dtype=np.int32), x, wr, w1, w3, w2, eid, gate64, dy, tau)
    dwr, dbias = router_wgrad(x, dl)
    dw1 = np.empty((E, d_ff, d))
    dw3 = np.empty((E, d_ff, d))
    dw2 = np.empty((E, d, d_ff))
    fs = np.arange(d_ff, dtype=np.int32)
    for e in range(E):
        tok, g = expert_slots(eid, row, gate64, e)
        dw1[e], dw3[e], dw2[e] = backward_expert_units(e, fs, tok, g, x, w1, w3, w2, dy)
    return dict(dlogits=dl, dx=dx, dwr=dwr, dbias=dbias, dw1=dw1, dw3=dw3, dw2=dw2)


def load_window(cand, E: int, k: int, load, window: int = 1024, alpha: float = 0.99) -> np.ndarray:
    """Windowed load statistic: per window of `window` tokens (token order),
    load = alpha * load + (1 - alpha) * (the window's top-k selection
    frequency per expert).  Returns the updated fp32 [E] vector."""
    cand = np.ascontiguousarray(_np(cand), dtype=np.int32)
    T, K1 = cand.shape
    out = np.array(_np(load), dtype=np.float32, copy=True)
    assert out.shape == (E,) and k < K1 + 1
    lib().oracle_load_window(T, E, k, K1, _p(cand), int(window), float(alpha), _p(out))
    return out
