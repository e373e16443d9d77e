"""Pins of the oracle's backward pass (CPU).

The oracle's gradients are checked against references that share none of its
code:
  * torch float64 autograd of the layer written from its definition, the
    routing of the forward pass held fixed: y_t = sum over kept slots j of
    g_j * W2_e (silu(W1_e x_t) * (W3_e x_t)), g = softmax over the kept slots
    of (raw - lambda load)[t, e_j] / tau, raw = x W_r^T + bias
    ("MoE架构揭秘" §3.1 router and softmax, §3.3 the router trained through
    the experts; "GPT-4稀疏激活真相" §3.1 the expert FFN; "企业官网建设流程全解析"
    page §3 step 5 the weighted combine);
  * central finite differences of the oracle's own forward pass (a separate C
    path) with respect to expert weights and router logits;
  * invariants: the router-logit gradient of a token sums to zero over the
    experts (softmax is shift-invariant); identical experts give a zero
    router gradient; one expert with top-1 gives a zero router gradient and
    the textbook SwiGLU backward.
"""
import numpy as np
import pytest
import torch

import oracle


def f32_to_bf16_bits(a):
    """Round fp32 to bf16 (nearest even), as uint16 bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def make_case(T, d, E, k, d_ff, cf, dtype="f32", tau=1.0, lam=0.0, bias=False, seed=0, reroute=1,
              identical=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    w1 = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    w3 = (rng.standard_normal((E, d_ff, d)) / np.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32)
    if identical:
        w1[:], w3[:], w2[:] = w1[0], w3[0], w2[0]
    b = (rng.standard_normal(E) * 0.5).astype(np.float32) if bias else None
    load = (rng.random(E) / E).astype(np.float32) if lam else None
    if dtype == "bf16":
        x, wr, w1, w3, w2 = (f32_to_bf16_bits(v) for v in (x, wr, w1, w3, w2))
    raw = oracle.router_logits(x, wr, b)
    cand, cs = oracle.route(raw, k, load, lam)
    C = oracle.capacity(T, k, E, cf)
    disp = oracle.dispatch(cand, cs, E, k, C, reroute, 0.01, tau)
    dy = rng.standard_normal((T, d))
    return dict(x=x, wr=wr, w1=w1, w3=w3, w2=w2, b=b, load=load, lam=lam, tau=tau, disp=disp, dy=dy, E=E, k=k)


def torch_reference(c):
    """Gradients of L = sum(y * dy) by torch float64 autograd, routing fixed."""
    tt = lambda a: torch.tensor(as_f64(a), dtype=torch.float64, requires_grad=True)
    x, wr, w1, w3, w2 = (tt(c[n]) for n in ("x", "wr", "w1", "w3", "w2"))
    E = c["E"]
    b = tt(c["b"]) if c["b"] is not None else torch.zeros(E, dtype=torch.float64, requires_grad=True)
    raw = x @ wr.T + b
    raw.retain_grad()
    s = raw - (c["lam"] * torch.tensor(as_f64(c["load"]))) if c["load"] is not None else raw
    # the gates take the values of the fp32 scores the routing was decided on
    # (the oracle's own logits and penalty); the gradient flows through s
    s32 = oracle.scores(oracle.router_logits(c["x"], c["wr"], c["b"]), c["load"], c["lam"])
    s = torch.tensor(s32.astype(np.float64)) + (s - s.detach())
    eid = torch.tensor(c["disp"]["eid"].astype(np.int64))
    kept = eid >= 0
    sk = s.gather(1, eid.clamp(min=0)) / c["tau"]
    sk = torch.where(kept, sk, torch.full_like(sk, -float("inf")))
    any_kept = kept.any(dim=1, keepdim=True)
    g = torch.softmax(torch.where(any_kept, sk, torch.zeros_like(sk)), dim=1)
    g = torch.where(kept, g, torch.zeros_like(g))
    y = torch.zeros_like(x)
    for j in range(eid.shape[1]):
        for e in range(E):
            m = eid[:, j] == e
            if not m.any():
                continue
            xe = x[m]
            h = torch.nn.functional.silu(xe @ w1[e].T) * (xe @ w3[e].T)
            y = y.index_add(0, torch.nonzero(m)[:, 0], g[m, j:j + 1] * (h @ w2[e].T))
    (y * torch.tensor(c["dy"])).sum().backward()
    return dict(dlogits=raw.grad.numpy(), dx=x.grad.numpy(), dwr=wr.grad.numpy(), dbias=b.grad.numpy(),
                dw1=w1.grad.numpy(), dw3=w3.grad.numpy(), dw2=w2.grad.numpy())


def oracle_grads(o, c):
    d = c["disp"]
    return o.backward(c["x"], c["wr"], c["w1"], c["w3"], c["w2"], d["eid"], d["row"], d["gate64"], c["dy"],
                      c["tau"])


def close(a, b, what, rtol=1e-9):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= rtol, f"{what}: max rel err {err:.3e}"


CASES = {
    # drops and re-routes (capacity below demand), fp32 elements
    "capped_f32": dict(T=40, d=16, E=4, k=2, d_ff=24, cf=0.6),
    # bf16 elements, top-3, gate temperature, bias and load penalty
    "bf16_tau_bias_penalty": dict(T=30, d=32, E=6, k=3, d_ff=16, cf=1.0, dtype="bf16", tau=0.5, lam=0.3,
                                  bias=True, seed=3),
    # no re-route: overflowing slots dropped, some tokens with one kept slot
    "no_reroute": dict(T=36, d=16, E=3, k=2, d_ff=8, cf=0.5, reroute=0, seed=5),
    # uncapped top-1
    "top1_uncapped": dict(T=25, d=8, E=5, k=1, d_ff=12, cf=0.0, seed=7),
}


def check_backward_autograd(o):
    for name, kw in CASES.items():
        c = make_case(**kw)
        got, ref = oracle_grads(o, c), torch_reference(c)
        assert (c["disp"]["flag"] == 2).any() or kw["cf"] >= 1.0 or kw["cf"] == 0.0 or name == "capped_f32"
        for n in ("dlogits", "dx", "dwr", "dbias", "dw1", "dw3", "dw2"):
            close(got[n], ref[n], f"{name}: {n}")


def check_backward_finite_differences(o):
    """Central differences of the oracle's forward (oracle_layer_tokens, with
    the gates fixed) w.r.t. single expert-weight entries, and of the gate
    softmax w.r.t. router logits, against the oracle's backward."""
    c = make_case(T=24, d=8, E=3, k=2, d_ff=6, cf=0.8, seed=11)
    d = c["disp"]
    got = oracle_grads(o, c)
    T = c["x"].shape[0]
    toks = np.arange(T, dtype=np.int32)

    x64 = as_f64(c["x"])  # double elements throughout (the oracle takes one element type)

    def loss(w1, w3, w2):
        y = o.layer_tokens(toks, x64, w1, w3, w2, d["eid"], d["gate64"])
        return float((y * c["dy"]).sum())

    eps = 1e-3
    rng = np.random.default_rng(2)
    for name, idx_shape in (("w1", c["w1"].shape), ("w3", c["w3"].shape), ("w2", c["w2"].shape)):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in idx_shape)
            wp = {n: c[n].astype(np.float64) for n in ("w1", "w3", "w2")}
            wm = {n: v.copy() for n, v in wp.items()}
            wp[name][idx] += eps
            wm[name][idx] -= eps
            fd = (loss(wp["w1"], wp["w3"], wp["w2"]) - loss(wm["w1"], wm["w3"], wm["w2"])) / (2 * eps)
            g = got["d" + name][idx]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(g)), (name, idx, fd, g)
    # router logits: L as a function of the kept slots' scores through the gate softmax
    y_rows = {}
    for t in range(T):
        for j in range(c["k"]):
            e = d["eid"][t, j]
            if e >= 0:
                y_rows[t, j] = o.ffn_rows(np.array([e], np.int32), np.array([t], np.int32), c["x"], c["w1"],
                                          c["w3"], c["w2"])[0]
    raw = o.router_logits(c["x"], c["wr"], None).astype(np.float64)

    def loss_raw(r):
        tot = 0.0
        for t in range(T):
            js = [j for j in range(c["k"]) if d["eid"][t, j] >= 0]
            if not js:
                continue
            sc = np.array([r[t, d["eid"][t, j]] for j in js]) / c["tau"]
            g = np.exp(sc - sc.max())
            g /= g.sum()
            tot += sum(g[i] * float(y_rows[t, j] @ c["dy"][t]) for i, j in enumerate(js))
        return tot

    for _ in range(8):
        t, e = int(rng.integers(0, T)), int(rng.integers(0, c["E"]))
        rp, rm = raw.copy(), raw.copy()
        rp[t, e] += eps
        rm[t, e] -= eps
        fd = (loss_raw(rp) - loss_raw(rm)) / (2 * eps)
        assert abs(fd - got["dlogits"][t, e]) <= 1e-6 * max(1.0, abs(fd)), (t, e, fd, got["dlogits"][t, e])


def check_backward_invariants(o):
    # the router-logit gradient of every token sums to zero over the experts
    c = make_case(**CASES["bf16_tau_bias_penalty"])
    g = oracle_grads(o, c)
    assert np.abs(g["dlogits"].sum(axis=1)).max() <= 1e-12 * max(1.0, np.abs(g["dlogits"]).max())
    assert abs(g["dbias"].sum()) <= 1e-10 * max(1.0, np.abs(g["dbias"]).max())
    # identical experts: every kept slot's output is the same, so the gates get no gradient
    c = make_case(T=30, d=16, E=4, k=2, d_ff=8, cf=0.7, identical=True, seed=9)
    g = oracle_grads(o, c)
    assert np.abs(g["dlogits"]).max() <= 1e-12 and np.abs(g["dwr"]).max() <= 1e-12
    # one expert, top-1, uncapped: the dense SwiGLU FFN; gate 1, no router gradient
    c = make_case(T=20, d=12, E=1, k=1, d_ff=10, cf=0.0, seed=13)
    g = oracle_grads(o, c)
    assert np.abs(g["dlogits"]).max() == 0.0 and np.abs(g["dwr"]).max() == 0.0
    x, w1, w3, w2 = (torch.tensor(as_f64(c[n]), requires_grad=True) for n in ("x", "w1", "w3", "w2"))
    y = (torch.nn.functional.silu(x @ w1[0].T) * (x @ w3[0].T)) @ w2[0].T
    (y * torch.tensor(c["dy"])).sum().backward()
    for n, t in (("dx", x), ("dw1", w1), ("dw3", w3), ("dw2", w2)):
        close(g[n], t.grad.numpy(), f"dense {n}")


def check_backward_sampled_units(o):
    """The per-unit weight gradients equal the whole-matrix ones (the form the
    GPU parity tests sample at full size)."""
    c = make_case(**CASES["capped_f32"])
    d = c["disp"]
    full = oracle_grads(o, c)
    fs = np.array([0, 5, 23], np.int32)
    for e in range(c["E"]):
        tok, g = o.expert_slots(d["eid"], d["row"], d["gate64"], e)
        dw1, dw3, dw2 = o.backward_expert_units(e, fs, tok, g, c["x"], c["w1"], c["w3"], c["w2"], c["dy"])
        close(dw1, full["dw1"][e][fs], "units dw1", 1e-12)
        close(dw3, full["dw3"][e][fs], "units dw3", 1e-12)
        close(dw2, full["dw2"][e][:, fs], "units dw2", 1e-12)


def test_backward_matches_autograd(oracle_mod):
    check_backward_autograd(oracle_mod)


def test_backward_finite_differences(oracle_mod):
    check_backward_finite_differences(oracle_mod)


def test_backward_invariants(oracle_mod):
    check_backward_invariants(oracle_mod)


def test_backward_sampled_units(oracle_mod):
    check_backward_sampled_units(oracle_mod)
