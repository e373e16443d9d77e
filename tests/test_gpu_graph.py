"""moe_forward and moe_forward_noalloc captured in a HIP graph (through
torch.cuda.graph) and replayed: every replay writes the same routing arrays,
logits and layer output, bit for bit, as the eager call.  The library
enqueues kernels only (no memset, copy or allocation), so a capture records
the whole forward pass.  Between replays the outputs are poisoned and other
eager work runs on the device, and every replay is checked."""
import sys

import pytest
import torch

import moe_synth
import sparse_mixture_experts_gemm_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def outputs(p, cfg):
    r = moe.Routing(p, DEV)
    y = torch.empty((p.T, cfg.d), dtype=torch.bfloat16, device=DEV)
    logits = torch.empty((p.T, cfg.E), dtype=torch.float32, device=DEV)
    return r, y, logits


def poison(r, y, logits):
    for n in moe.Routing.NAMES:
        getattr(r, n).fill_(-7)
    y.fill_(float("nan"))
    logits.fill_(float("nan"))


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else (t.view(torch.int16) if t.dtype == torch.bfloat16 else t)


def same(a, b, what):
    ra, ya, la = a
    rb, yb, lb = b
    assert torch.equal(bits(la), bits(lb)), f"{what}: logits"
    assert torch.equal(bits(ya), bits(yb)), f"{what}: layer output"
    for n in moe.Routing.NAMES:
        assert torch.equal(bits(ra[n]), bits(rb[n])), f"{what}: routing array {n}"


def snapshot(r, y, logits):
    torch.cuda.synchronize()
    return r.cpu(), y.cpu(), logits.cpu()


# skew: two uniform down slices; fine64: one; mixtral at T 2100: the
# device-side split plan (8 of 24 m tiles split in two)
@pytest.mark.parametrize("entry,name,T", [("forward", "skew", None), ("forward", "fine64", 2048),
                                          ("forward", "mixtral", 2100), ("noalloc", "mixtral", 128)])
def test_forward_graph_replay(entry, name, T):
    cfg = moe_synth.CONFIGS[name]
    T = cfg.T if T is None else T
    p = moe.Params(T=T, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff, capacity_factor=cfg.cf, reroute=cfg.reroute,
                   lam=cfg.lam, aux_coef=cfg.aux_coef, dtype=moe.MOE_BF16)
    L = moe_synth.make_layer(cfg, DEV, T=T)
    load = torch.full((cfg.E,), 1.0 / cfg.E, dtype=torch.float32, device=DEV) if cfg.lam else None
    ws = moe.alloc_workspace(p, DEV) if entry == "forward" else None
    if entry == "noalloc":
        assert moe.workspace_bytes(p) <= moe.STATIC_SCRATCH_BYTES

    def call(r, y, logits):
        if entry == "forward":
            moe.forward(p, L["x"], L["w_router"], L["bias"], load, L["w1"], L["w3"], L["w2"], y, logits, r, ws)
        else:
            moe.forward_noalloc(p, L["x"], L["w_router"], L["bias"], load, L["w1"], L["w3"], L["w2"], y, logits, r)

    say(f"[graph] {entry} {name} T={T}: eager reference")
    ref_bufs = outputs(p, cfg)
    call(*ref_bufs)
    ref = snapshot(*ref_bufs)

    # capture on a side stream after a warm-up there
    bufs = outputs(p, cfg)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(*bufs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say(f"[graph] {entry} {name} T={T}: capture")
    with torch.cuda.graph(g, stream=s):
        call(*bufs)
    torch.cuda.synchronize()
    other = outputs(p, cfg)
    for rep in range(4):
        poison(*bufs)
        torch.cuda.synchronize()
        g.replay()
        got = snapshot(*bufs)
        same(got, ref, f"replay {rep}")
        # eager work between replays, including the same entry point on other buffers
        call(*other)
        same(snapshot(*other), ref, f"eager call after replay {rep}")
    say(f"[ok] graph {entry} {name} T={T}: 4 replays bit-identical")
