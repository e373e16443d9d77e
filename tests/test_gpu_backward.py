"""GPU parity of the backward pass (moe_backward through the C ABI) against
the oracle's gradients, the forward routing held fixed.

The routing comes from moe_forward on the GPU and is checked bit-exact
against the oracle run on the GPU's logits; the oracle then differentiates
the layer in double with the same routing and double gates.  Every gradient
(dx, dlogits, dW_r, dbias, dW1, dW3, dW2; fp32 on the GPU) must satisfy
max|err| <= 2e-2 * RMS(ref), the bf16 layer's bound.  Small layers are
checked in full; the full-size workloads on sampled tokens (dx, dlogits) and
sampled intermediate units of two experts (rows of dW1 and dW3, columns of
dW2), with dW_r and dbias checked in full against the oracle's contraction
of the GPU's dlogits.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import sparse_mixture_experts_gemm_amd as moe
from tests.test_gpu_parity import DEV, Layer, np_of, params, rms, routing_vs_oracle, say, small_cfg

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    oracle.lib()


def close(got, ref, what):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if not ref.size:
        return 0.0
    r = rms(ref)
    err = float(np.abs(got - ref).max())
    assert err <= TOL * r + 1e-30, f"{what}: max|err| {err:.3e} > {TOL} * RMS {r:.3e}"
    return err / r if r > 0 else 0.0


def forward_and_backward(L, p):
    g = L.g
    r = moe.Routing(p, DEV)
    y = torch.empty((p.T, p.d), dtype=torch.bfloat16, device=DEV)
    logits = torch.empty((p.T, p.E), dtype=torch.float32, device=DEV)
    moe.forward(p, g["x"], g["w_router"], g["bias"], L.load_g, g["w1"], g["w3"], g["w2"], y, logits, r,
                moe.alloc_workspace(p, DEV))
    dy = moe_synth.upstream_grad(L.cfg, DEV, T=p.T)
    gr = moe.Grads(p, DEV)
    for n in moe.Grads.NAMES:  # poison: every element must be written
        getattr(gr, n).fill_(float("nan"))
    moe.backward(p, g["x"], g["w_router"], g["w1"], g["w3"], g["w2"], r, dy, gr, moe.alloc_backward_workspace(p, DEV))
    torch.cuda.synchronize()
    return r, logits, dy, gr


def run_backward(cfg, T=None, full=False, n_tok=12, n_units=6):
    L = Layer(cfg, T)
    p = params(cfg, T=L.T)
    say(f"[backward] {cfg.name} T={p.T} full={full}")
    r, logits, dy, gr = forward_and_backward(L, p)
    rc = r.cpu()
    ref = routing_vs_oracle(p, rc, logits.cpu().numpy(), L.load, p.lam)
    tau = p.gate_temperature if p.gate_temperature > 0 else 1.0
    dy64 = dy.double().cpu().numpy()
    G = {n: getattr(gr, n).double().cpu().numpy() for n in moe.Grads.NAMES}
    for n, v in G.items():
        assert np.isfinite(v).all(), f"{n} has unwritten or non-finite elements"
    # each token's router-logit gradient sums to zero (softmax shift invariance)
    assert np.abs(G["dlogits"].sum(axis=1)).max() <= 1e-4 * max(rms(G["dlogits"]), 1e-30) * p.k
    c = L.c
    if full:
        want = oracle.backward(c["x"], c["w_router"], c["w1"], c["w3"], c["w2"], ref["eid"], ref["row"], ref["gate64"],
                               dy64, tau)
        errs = {n: close(G[n if n != "dwr" else "dw_router"], want[n], n)
                for n in ("dx", "dlogits", "dwr", "dbias", "dw1", "dw3", "dw2")}
    else:
        rng = np.random.default_rng(17)
        toks = np.unique(np.r_[0, p.T - 1, rng.choice(p.T, n_tok, replace=False)]).astype(np.int32)
        dl, dx = oracle.backward_tokens(toks, c["x"], c["w_router"], c["w1"], c["w3"], c["w2"], ref["eid"],
                                        ref["gate64"], dy64, tau)
        errs = {"dx": close(G["dx"][toks], dx, "dx"), "dlogits": close(G["dlogits"][toks], dl, "dlogits")}
        kept = ref["kept"]
        experts = sorted({int(np.argmax(kept)), int(rng.choice(np.nonzero(kept)[0]))})
        fs = np.unique(np.r_[0, p.d_ff - 1, rng.choice(p.d_ff, n_units, replace=False)]).astype(np.int32)
        for e in experts:
            tok, gt = oracle.expert_slots(ref["eid"], ref["row"], ref["gate64"], e)
            w1r, w3r, w2c = oracle.backward_expert_units(e, fs, tok, gt, c["x"], c["w1"], c["w3"], c["w2"], dy64)
            errs[f"dw1[{e}]"] = close(G["dw1"][e][fs], w1r, f"dw1[{e}]")
            errs[f"dw3[{e}]"] = close(G["dw3"][e][fs], w3r, f"dw3[{e}]")
            errs[f"dw2[{e}]"] = close(G["dw2"][e][:, fs], w2c, f"dw2[{e}]")
        # router weights and bias: the oracle's contraction of the GPU's dlogits
        dwr, db = oracle.router_wgrad(c["x"], G["dlogits"])
        errs["dwr"] = close(G["dw_router"], dwr, "dw_router")
        errs["dbias"] = close(G["dbias"], db, "dbias")
    say(f"[ok] backward {cfg.name}: " + ", ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    return gr


BWD_SMALL = {
    "small_capped": dict(T=700, d=256, E=4, k=2, d_ff=384, cf=1.0),
    "top3_temperature": dict(T=500, d=128, E=8, k=3, d_ff=192, cf=0.8, tau=0.5),
    "bias_penalty": dict(T=400, d=128, E=16, k=2, d_ff=128, bias="hot0", bias_hot=3.0, lam=0.3,
                         load_from_prev=True),
    "dense_E1": dict(T=100, d=128, E=1, k=1, d_ff=256, cf=0.0),
    "one_token": dict(T=1, d=256, E=4, k=2, d_ff=128),
    "ragged": dict(T=333, d=192, E=5, k=2, d_ff=320, cf=1.3),
    # the forward's edge cases: every expert picked (k = E), capacity 1,
    # uncapped, dropping without re-route, 256 experts with top-8 (most
    # experts get a few rows or none: zero weight-gradient tiles), the
    # minimum dims (one partial 64-row tile), the top-2 gap threshold
    "k_equals_E": dict(E=2, k=2, T=300, cf=0.6),
    "capacity_one": dict(T=200, cf=1e-6),
    "uncapped": dict(T=300, cf=0.0),
    "no_reroute": dict(T=400, cf=0.5, reroute=0),
    "many_experts_top8": dict(E=256, k=8, T=512, d=64, d_ff=64, cf=1.0),
    "min_dims": dict(T=77, d=64, d_ff=64, E=3, k=1),
    "top2_gap": dict(T=600, E=8, k=2, cf=1.0, gap=0.1),
}


@pytest.mark.parametrize("case", sorted(BWD_SMALL))
def test_backward_small_full(case):
    run_backward(small_cfg(**BWD_SMALL[case]), full=True)


@pytest.mark.parametrize("name", ["skew", "decode", "fine64", "mixtral"])
def test_backward_workloads(name):
    run_backward(moe_synth.CONFIGS[name])


def test_backward_empty_batch_zero_weight_grads():
    cfg = small_cfg(T=0)
    p = params(cfg)
    g = moe_synth.make_layer(cfg, DEV, T=0)
    r = moe.Routing(p, DEV)
    moe.forward(p, g["x"], g["w_router"], None, None, g["w1"], g["w3"], g["w2"],
                torch.empty((0, cfg.d), dtype=torch.bfloat16, device=DEV),
                torch.empty((0, cfg.E), dtype=torch.float32, device=DEV), r, moe.alloc_workspace(p, DEV))
    gr = moe.Grads(p, DEV)
    for n in moe.Grads.NAMES:
        getattr(gr, n).fill_(float("nan"))
    moe.backward(p, g["x"], g["w_router"], g["w1"], g["w3"], g["w2"], r,
                 torch.empty((0, cfg.d), dtype=torch.bfloat16, device=DEV), gr, moe.alloc_backward_workspace(p, DEV))
    torch.cuda.synchronize()
    for n in ("dw_router", "dbias", "dw1", "dw3", "dw2"):
        assert (getattr(gr, n) == 0).all(), n


def test_backward_deterministic():
    cfg = moe_synth.CONFIGS["skew"]
    L = Layer(cfg, T=1024)
    p = params(cfg, T=1024)
    outs = [forward_and_backward(L, p)[3] for _ in range(2)]
    for n in moe.Grads.NAMES:
        a, b = getattr(outs[0], n), getattr(outs[1], n)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), n


def test_backward_stream_order():
    """moe_backward runs its weight-gradient half on a stream of its own and
    joins it back to the caller's stream: work enqueued after the call on
    that stream (here copies of every output, with no synchronisation in
    between) sees the finished gradients, on a non-default stream too."""
    cfg = moe_synth.CONFIGS["skew"]
    L = Layer(cfg, T=1024)
    p = params(cfg, T=1024)
    ref = forward_and_backward(L, p)
    g = L.g
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gr = moe.Grads(p, DEV)
        for n in moe.Grads.NAMES:
            getattr(gr, n).fill_(float("nan"))
        ws = moe.alloc_backward_workspace(p, DEV)
        copies = {}
        for _ in range(2):
            moe.backward(p, g["x"], g["w_router"], g["w1"], g["w3"], g["w2"], ref[0], ref[2], gr, ws, stream=s)
            copies = {n: getattr(gr, n).clone() for n in moe.Grads.NAMES}
            for n in moe.Grads.NAMES:  # the next call must overwrite every element again
                getattr(gr, n).fill_(float("nan"))
    torch.cuda.synchronize()
    for n in moe.Grads.NAMES:
        a, b = copies[n], getattr(ref[3], n)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), n


@pytest.mark.parametrize("over", [dict(dtype="f32"), dict(router_hidden=16)])
def test_backward_unsupported(over):
    cfg = small_cfg(T=64, dtype=over.get("dtype", "bf16"))
    p = params(cfg, router_hidden=over.get("router_hidden", 0))
    L = Layer(cfg)
    with pytest.raises(moe.MoEError) as ei:
        moe.backward(p, L.g["x"], L.g["w_router"], L.g["w1"], L.g["w3"], L.g["w2"], moe.Routing(p, DEV),
                     torch.zeros_like(L.g["x"]), moe.Grads(p, DEV), moe.alloc_backward_workspace(p, DEV))
    assert ei.value.code == moe.MOE_ERR_UNSUPPORTED
