"""GPU parity at the edges of what the C ABI accepts: every kernel
instantiation that moe.h's limits make reachable (0 <= T <= 2^20, E <= 256,
d <= 16384 for bf16 and 8192 for fp32) runs here against the oracle.

  * the vector-ALU router (fp32 layers, and bf16 layers with E > 64) at
    1, 2 and 4 tokens per wave (T >= 4096 gives 2, T >= 8192 gives 4) and
    at every hidden-size class (NX 1..32 chunks of 64 lanes: d up to 8192
    for fp32, 16384 for bf16);
  * the expert GEMM and combine at d = 16384;
  * moe_forward's fallback for x of 2 GiB and more (x_perm materialised in
    the workspace instead of the GEMM gathering rows from x);
  * routing and dispatch at T = 2^20 (1024 dispatch blocks).

Tolerances and routing exactness as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
import sparse_mixture_experts_gemm_amd as moe
from tests.test_gpu_parity import (DEV, Layer, assert_close, np_of, params, rms, routing_vs_oracle, run_stages,
                                   say, small_cfg)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    oracle.lib()


LIMIT_CASES = {
    # vector-ALU router, bf16 with E > 64: 4, 2 and 1 tokens per wave
    "valu_bf16_e96_tpw4": dict(T=8209, E=96, k=2, d=256, d_ff=64),
    "valu_bf16_e96_tpw2": dict(T=5000, E=96, k=3, d=256, d_ff=64),
    # vector-ALU router, fp32 with E > 32: 2 and 4 tokens per wave
    "valu_f32_e48_tpw2": dict(T=4099, E=48, k=2, d=128, d_ff=64, dtype="f32"),
    "valu_f32_e48_tpw4": dict(T=8300, E=48, k=2, d=128, d_ff=64, dtype="f32"),
    # hidden-size classes of the vector-ALU router: NX 16 and 32 (fp32 d 4096
    # and 8192, the fp32 limit), bf16 d 8192 and 16384 (the bf16 limit)
    "nx16_f32_d4096": dict(T=300, E=6, k=2, d=4096, d_ff=64, dtype="f32"),
    "nx32_f32_d8192": dict(T=200, E=5, k=2, d=8192, d_ff=64, dtype="f32"),
    "nx16_bf16_e96_d8192": dict(T=300, E=96, k=2, d=8192, d_ff=64),
    "nx32_bf16_e96_d16384": dict(T=300, E=96, k=2, d=16384, d_ff=64),
    # the expert GEMM (gate-up K = 16384; down N = 16384) and the MFMA router
    # at the bf16 limit
    "gemm_bf16_d16384": dict(T=600, E=2, k=1, d=16384, d_ff=128, cf=1.0),
}


@pytest.mark.parametrize("case", sorted(LIMIT_CASES))
def test_abi_limit_instantiations(case):
    cfg = small_cfg(**LIMIT_CASES[case])
    L = Layer(cfg)
    say(f"[case] {case}")
    run_stages(L, params(cfg), full_rows=cfg.T <= 600, stored=True)


def test_forward_x_of_2gib_materialises_x_perm():
    """T = 2^18, d = 4096 bf16: x spans exactly 2 GiB, so moe_forward copies
    the kept rows into x_perm in its workspace instead of gathering them in
    the GEMM.  Routing bit-exact over all tokens; the layer output of 32
    sampled tokens against the oracle."""
    cfg = small_cfg(T=1 << 18, E=4, k=2, d=4096, d_ff=64, cf=1.0)
    p = params(cfg)
    T, d = cfg.T, cfg.d
    assert T * d * 2 == 1 << 31
    say(f"[case] x of 2 GiB: T={T} d={d} workspace {moe.workspace_bytes(p) / 2**30:.1f} GiB")
    g = moe_synth.make_layer(cfg, DEV)
    r = moe.Routing(p, DEV)
    y = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device=DEV)
    ws = moe.alloc_workspace(p, DEV)
    moe.forward(p, g["x"], g["w_router"], g["bias"], None, g["w1"], g["w3"], g["w2"], y, logits, r, ws)
    torch.cuda.synchronize()
    del ws
    gl = logits.cpu().numpy()
    rc = r.cpu()
    ref = routing_vs_oracle(p, rc, gl, None, 0.0)
    rng = np.random.default_rng(5)
    toks = np.unique(np.r_[0, T - 1, rng.choice(T, 30, replace=False)]).astype(np.int64)
    tt = torch.from_numpy(toks).to(DEV)
    xs = np_of(g["x"].index_select(0, tt).cpu())
    own = oracle.router_logits(xs, np_of(g["w_router"].cpu()), None)
    assert np.abs(own - gl[toks]).max() <= 1e-3 * rms(own), "router logits"
    w = {n: np_of(g[n].cpu()) for n in ("w1", "w3", "w2")}
    yref = oracle.layer_tokens(np.arange(len(toks), dtype=np.int32), xs, w["w1"], w["w3"], w["w2"],
                               np.ascontiguousarray(ref["eid"][toks]), np.ascontiguousarray(ref["gate64"][toks]))
    got = y.index_select(0, tt).float().cpu().numpy()
    rel = assert_close(got, yref, p.dtype, "layer output", stored=True)
    say(f"[ok] x of 2 GiB: rows={int(ref['totals'][0])} max|err|/RMS={rel:.2e}")


@pytest.mark.parametrize("E", [8, 96])
def test_routing_at_the_token_limit(E):
    """T = 2^20 tokens (1024 dispatch blocks): the MFMA router (E 8) or the
    vector-ALU router at 4 tokens per wave (E 96), then the dispatch; every
    routing array bit-exact with the oracle run on the GPU's logits."""
    cfg = small_cfg(T=1 << 20, E=E, k=2, d=64, d_ff=64, cf=1.0)
    p = params(cfg)
    say(f"[case] T=2^20 E={E}")
    g = moe_synth.make_layer(cfg, DEV, want=("x", "w_router", "bias"))
    r = moe.Routing(p, DEV)
    logits = torch.empty((cfg.T, E), dtype=torch.float32, device=DEV)
    moe.route(p, g["x"], g["w_router"], g["bias"], None, logits, r)
    R = moe.max_rows(p)
    xp = torch.empty((R, cfg.d), dtype=torch.bfloat16, device=DEV)
    moe.dispatch(p, g["x"], r, xp, moe.alloc_workspace(p, DEV, dispatch_only=True))
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    rng = np.random.default_rng(9)
    toks = np.unique(np.r_[0, cfg.T - 1, rng.choice(cfg.T, 4096, replace=False)])
    own = oracle.router_logits(np_of(g["x"].cpu())[toks], np_of(g["w_router"].cpu()), None)
    assert np.abs(own - gl[toks]).max() <= 1e-3 * rms(own), "router logits"
    ref = routing_vs_oracle(p, r.cpu(), gl, None, 0.0)
    # x_perm rows are the token rows of token_of_row (sampled)
    rows = int(ref["totals"][0])
    sr = np.unique(np.r_[0, rows - 1, rng.choice(rows, 2048, replace=False)])
    tor = torch.from_numpy(ref["token_of_row"][sr].astype(np.int64)).to(DEV)
    assert torch.equal(xp[torch.from_numpy(sr).to(DEV)], g["x"].index_select(0, tor)), "x_perm"
    say(f"[ok] T=2^20 E={E}: rows={rows} dropped={int(ref['totals'][1])} rerouted={int(ref['totals'][2])}")


def test_fp16_intermediate_range():
    """A bf16 layer near the limits of its fp16 intermediates, inside the
    contract: x scaled by 40 so that h = silu(a) * b reaches 10^4 (fp16 tops
    out at 65504), and W2 scaled by 1e-3 so that a large share of its
    entries lie below 2^-14, where the fp16 narrowing keeps fewer bits.
    h within one fp16 ulp, y_perm and the layer output within 2e-2 * RMS."""
    cfg = small_cfg(T=300, E=4, k=2, d=256, d_ff=256, cf=1.0)
    L = Layer(cfg)
    L.g["x"].mul_(40.0)
    L.g["w2"].mul_(1e-3)
    torch.cuda.synchronize()
    L.c = {n: (np_of(v) if v is not None else None) for n, v in L.g.items()}
    # preconditions, in double on the host: |h| high in fp16's range but below
    # 65504; W2 partly below 2^-14 and nowhere near 65504
    x = L.g["x"].double().cpu().numpy()
    w1, w3 = L.g["w1"].double().cpu().numpy(), L.g["w3"].double().cpu().numpy()
    a, b = np.einsum("td,efd->etf", x, w1), np.einsum("td,efd->etf", x, w3)
    hmax = float(np.abs(a / (1.0 + np.exp(-a)) * b).max())
    w2 = np.abs(L.g["w2"].double().cpu().numpy())
    say(f"[case] fp16 range: max|h| {hmax:.0f}, W2 below 2^-14: {(w2 < 2.0 ** -14).mean():.2f}")
    assert 1e4 < hmax < 65504.0
    assert (w2 < 2.0 ** -14).mean() > 0.3 and w2.max() < 1.0
    run_stages(L, params(cfg), full_rows=True, stored=True)
