"""moe_forward_noalloc (the variant for callers that cannot allocate: its
workspace is the library's static scratch array) through the C ABI against
moe_forward with a caller workspace: routing arrays, logits and the layer
output bit-identical (the same kernels in the same order), on two calls in a
row, the second with a smaller batch, so the array's leftover contents from
the first call must not matter."""
import ctypes
import sys

import pytest
import torch

import moe_synth
import sparse_mixture_experts_gemm_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def run_pair(cfg, T, L):
    """moe_forward_noalloc and moe_forward on the first T tokens of L."""
    p = moe.Params(T=T, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff, capacity_factor=cfg.cf, reroute=cfg.reroute,
                   lam=cfg.lam, aux_coef=cfg.aux_coef, dtype=moe.MOE_BF16)
    assert moe.workspace_bytes(p) <= moe.STATIC_SCRATCH_BYTES
    x = L["x"][:T].contiguous()
    outs = []
    for use_static in (True, False):
        say(f"[no_alloc] {cfg.name} T={T} static={use_static}")
        r = moe.Routing(p, DEV)
        for n in moe.Routing.NAMES:  # poison every output
            getattr(r, n).fill_(-3)
        y = torch.full((T, cfg.d), float("nan"), dtype=torch.bfloat16, device=DEV)
        logits = torch.full((T, cfg.E), float("nan"), dtype=torch.float32, device=DEV)
        if use_static:
            moe.forward_noalloc(p, x, L["w_router"], L["bias"], None, L["w1"], L["w3"], L["w2"], y, logits, r)
        else:
            moe.forward(p, x, L["w_router"], L["bias"], None, L["w1"], L["w3"], L["w2"], y, logits, r,
                        moe.alloc_workspace(p, DEV))
        torch.cuda.synchronize()
        outs.append((y.cpu(), logits.cpu(), r.cpu()))
    (ys, ls, rs), (yw, lw, rw) = outs
    assert torch.equal(ls.view(torch.int32), lw.view(torch.int32)), "logits"
    for n in moe.Routing.NAMES:
        a, b = rs[n], rw[n]
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), f"routing array {n} differs"
    assert torch.equal(ys.view(torch.int16), yw.view(torch.int16)), "layer output differs"
    assert int(rs["totals"][0]) > 0


def test_noalloc_matches_forward_two_calls():
    """Decode-shape layer (d 4096, E 8, top-2, d_ff 14336): 160 tokens, then 64."""
    cfg = moe_synth.CONFIGS["decode"]
    L = moe_synth.make_layer(cfg, DEV, T=160)
    run_pair(cfg, 160, L)
    run_pair(cfg, 64, L)


def test_noalloc_rejects_layers_beyond_the_array():
    """The Mixtral-shape prefill layer needs far more than the array: the call
    is refused before anything is enqueued."""
    cfg = moe_synth.CONFIGS["mixtral"]
    p = moe.Params(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff, capacity_factor=cfg.cf, dtype=moe.MOE_BF16)
    assert moe.workspace_bytes(p) > moe.STATIC_SCRATCH_BYTES
    r = moe.MoeRouting(*[256] * len(moe.Routing.NAMES))  # never dereferenced
    rc = moe.lib().moe_forward_noalloc(ctypes.byref(p.c()), 256, 256, None, None, 256, 256, 256, 256, 256,
                                       ctypes.byref(r), None)
    assert rc == moe.MOE_ERR_TOO_LARGE
    assert "scratch" in moe.strerror(rc)
