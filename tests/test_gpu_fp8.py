"""GPU parity of the quantised expert weights, OCP E4M3 codes
(moe_expert_ffn_fp8, moe_forward_fp8), INT8 codes (moe_expert_ffn_i8,
moe_forward_i8) and INT4 codes two per byte (moe_expert_ffn_i4,
moe_forward_i4), through the C ABI against the oracle, which dequantises the
same codes and scales exactly (double) and runs its plain SwiGLU FFN.

Groups of at most 32 rows per expert run the weight-streaming kernel, larger
ones the 256 x 256 MFMA tile; both are covered for the one-byte codes, the
weight-streaming kernel (the only one INT4 codes run on) for INT4.

Tolerances as for the bf16 layer: h (rounded once to fp16) within one fp16
ulp per element plus 1e-4 * RMS for fp32 accumulation; y_perm and the layer
output within 2e-2 * RMS (the output beyond one bf16 unit roundoff of |ref|
only where the storage rounding of the largest element alone would take half
of that budget).
Routing arrays bit-exact with the oracle run on the GPU's fp32 logits.
"""
import sys

import numpy as np
import pytest
import torch

import moe_synth
import oracle
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
    oracle.lib()


def rms(a):
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2)))


def bf16_as_double(t):
    return t.float().cpu().numpy().astype(np.float64)


class Fp8Layer:
    """A bf16 layer's inputs with the expert weights replaced by codes (E4M3,
    INT8 or INT4) and row scales; the oracle's copies are the exact
    dequantised weights."""

    def __init__(self, cfg, seed=0, fmt="e4m3"):
        self.cfg = cfg
        self.fmt = fmt
        say(f"[gen] {cfg.name} {fmt} T={cfg.T} d={cfg.d} E={cfg.E} d_ff={cfg.d_ff} cf={cfg.cf}")
        g = moe_synth.make_layer(cfg, DEV, seed=seed)
        self.x, self.wr, self.bias = g["x"], g["w_router"], g["bias"]
        self.q, self.s, self.wd = {}, {}, {}
        for n in ("w1", "w3", "w2"):
            if fmt == "int8":
                q, s = moe_synth.quantize_rows_int8(g[n])
                self.wd[n] = oracle.dequant_rows_i8(q.cpu().numpy(), s.cpu().numpy())
            elif fmt == "int4":
                q, s = moe_synth.quantize_rows_int4(g[n])
                self.wd[n] = oracle.dequant_rows_i4(q.cpu().numpy(), s.cpu().numpy())
            else:
                q, s = moe_synth.quantize_rows_e4m3(g[n])
                self.wd[n] = oracle.dequant_rows(q.cpu().numpy(), s.cpu().numpy())
            self.q[n], self.s[n] = q, s
        del g
        torch.cuda.synchronize()
        self.xd = bf16_as_double(self.x)
        self.p = moe.Params(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, d_ff=cfg.d_ff, capacity_factor=cfg.cf,
                            reroute=cfg.reroute, lam=cfg.lam, aux_coef=cfg.aux_coef, dtype=moe.MOE_BF16)

    def weights(self):
        return (self.q["w1"], self.s["w1"], self.q["w3"], self.s["w3"], self.q["w2"], self.s["w2"])

    def expert_ffn(self, *a):
        {"int8": moe.expert_ffn_i8, "int4": moe.expert_ffn_i4, "e4m3": moe.expert_ffn_fp8}[self.fmt](*a)

    def forward(self, *a):
        {"int8": moe.forward_i8, "int4": moe.forward_i4, "e4m3": moe.forward_fp8}[self.fmt](*a)


def routing_exact(p, rc, logits):
    cand, cs = oracle.route(logits, p.k)
    C = oracle.capacity(p.T, p.k, p.E, p.capacity_factor)
    ref = oracle.dispatch(cand, cs, p.E, p.k, C, p.reroute, p.aux_coef)
    assert np.array_equal(rc["cand"].numpy(), cand), "cand"
    for n in ("eid", "row", "flag", "offsets"):
        assert np.array_equal(rc[n].numpy(), ref[n]), n
    return ref


def check_layer(L, full=True, rows_sample=None):
    p, T, d, dff = L.p, L.p.T, L.p.d, L.p.d_ff
    R = moe.max_rows(p)
    # route + dispatch on the bf16 path, then the FP8 FFN stage by stage
    r = moe.Routing(p, DEV)
    logits = torch.empty((T, p.E), dtype=torch.float32, device=DEV)
    moe.route(p, L.x, L.wr, L.bias, None, logits, r)
    x_perm = torch.empty((max(R, 1), d), dtype=torch.bfloat16, device=DEV)
    moe.dispatch(p, L.x, r, x_perm, moe.alloc_workspace(p, DEV, dispatch_only=True))
    h = torch.empty((max(R, 1), dff), dtype=torch.float16, device=DEV)
    y_perm = moe.alloc_y_perm(p, DEV)
    say(f"[expert_ffn_fp8] T={T} R={R}")
    L.expert_ffn(p, x_perm, r.offsets, *L.weights(), h, y_perm)
    torch.cuda.synchronize()
    rc = r.cpu()
    gl = logits.cpu().numpy()
    ref = routing_exact(p, rc, gl)
    offs = ref["offsets"]
    rows = int(offs[-1])
    srows = np.arange(rows, dtype=np.int32) if rows_sample is None else rows_sample(offs)
    if len(srows):
        expert_of = np.searchsorted(offs, srows, side="right").astype(np.int32) - 1
        xp = bf16_as_double(x_perm[:rows])
        yo, ho = oracle.ffn_rows(expert_of, srows, xp, L.wd["w1"], L.wd["w3"], L.wd["w2"], want_h=True)
        hg = h.float().cpu().numpy()[srows].astype(np.float64)
        bad = np.abs(hg - ho) > 2.0 ** -10 * np.abs(ho) + 1e-4 * rms(ho)
        assert not bad.any(), f"h: {bad.sum()} elements beyond rounding bound"
        yg = y_perm.double().cpu().numpy()[srows]
        err = np.abs(yg - yo).max()
        assert err <= 2e-2 * rms(yo), f"y_perm: {err:.3e} > 2e-2 * {rms(yo):.3e}"
    # combine, then the whole layer through moe_forward_fp8 (gates folded into
    # the down projection, gated rows in fp16): within one bf16 ulp of the
    # staged output plus the fp16 roundings
    y = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    moe.combine(p, y_perm, r.row, r.gate, y)
    say(f"[forward_fp8] T={T}")
    r2 = moe.Routing(p, DEV)
    y2 = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    logits2 = torch.empty((T, p.E), dtype=torch.float32, device=DEV)
    L.forward(p, L.x, L.wr, L.bias, None, *L.weights(), y2, logits2, r2, moe.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    ys, y2f = y.float().cpu().numpy().astype(np.float64), y2.float().cpu().numpy().astype(np.float64)
    bad = np.abs(y2f - ys) > 2.0 ** -7 * np.abs(ys) + 2.0 ** -7 * rms(ys)
    assert not bad.any(), f"moe_forward_fp8 vs staged: {bad.sum()} elements beyond rounding bound"
    ref2 = routing_exact(p, r2.cpu(), logits2.cpu().numpy())
    toks = np.arange(T, dtype=np.int32) if full else np.unique(np.r_[0, T - 1, np.arange(0, T, 7)]).astype(np.int32)
    yref = oracle.layer_tokens(toks, L.xd, L.wd["w1"], L.wd["w3"], L.wd["w2"], ref2["eid"], ref2["gate64"])
    got = y2.float().cpu().numpy()[toks].astype(np.float64)
    dev = np.abs(got - yref)
    # the bf16 storage rounding of each element is allowed only where that of the
    # largest one alone would take half the 2e-2 * RMS budget (as in the bf16 parity tests)
    if dev.size and np.abs(yref).max() * 2.0 ** -9 >= 0.5 * 2e-2 * rms(yref):
        dev = dev - 2.0 ** -8 * np.abs(yref)
    err = float(dev.max()) if dev.size else 0.0
    assert err <= 2e-2 * rms(yref) + 1e-30, f"layer output: {err:.3e} > 2e-2 * {rms(yref):.3e}"
    say(f"[ok] T={T} rows={rows} dropped={int(ref2['totals'][1])} max|err|/RMS={err / max(rms(yref), 1e-30):.2e}")


def cfg(**kw):
    base = dict(name="fp8", T=64, d=512, E=8, k=2, d_ff=1024, cf=1.25, dtype="bf16")
    base.update(kw)
    return moe_synth.MoEConfig(**base)


CASES = {
    # C = 20: experts with up to 16 rows (one 16-row block) and 17-20 (two)
    "decode_small": dict(),
    # C = 32, the largest capacity of the weight-streaming kernel; several
    # 64-column gate-up tiles and 128-column down tiles, ragged N tails
    "cap32_ragged_n": dict(T=128, d=384, d_ff=640, cf=1.0),
    "one_token": dict(T=1),
    "top1_many_experts": dict(T=200, E=24, k=1, d=256, d_ff=256, cf=1.0),
    "long_k": dict(T=40, d=2048, d_ff=1536, E=4, k=2, cf=1.5),
    "drops": dict(T=96, E=8, k=2, cf=0.5, d=256, d_ff=512),
    # more than 32 rows per expert: the 256 x 256 MFMA tile with the codes
    # widened in registers.  C = 350: two m tiles per expert, the second
    # ragged; the forward's down projection in two K slices (d_ff 512)
    "mfma_two_mtiles_split": dict(T=700, E=4, k=2, d=256, d_ff=512, cf=1.0),
    # ragged N tiles: gate-up 1.5 tiles of 128 h columns, down 256 + 64
    # output columns; C = 334
    "mfma_ragged_n": dict(T=500, E=3, k=2, d=320, d_ff=192, cf=1.0),
    # long K (d 2048), one m tile of 150 rows per expert, top-1
    "mfma_long_k": dict(T=300, E=2, k=1, d=2048, d_ff=1024, cf=1.0),
    # dropping capacity (C = 75) with re-routes, eight experts
    "mfma_drops": dict(T=600, E=8, k=2, cf=0.5, d=256, d_ff=256),
}


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
@pytest.mark.parametrize("case", sorted(CASES))
def test_fp8_cases(case, fmt):
    check_layer(Fp8Layer(cfg(name=case, **CASES[case]), fmt=fmt))


@pytest.mark.parametrize("case", sorted(c for c in CASES if not c.startswith("mfma_")))
def test_int4_cases(case):
    """INT4 codes on the weight-streaming kernel (at most 32 rows per
    expert): the same cases as the one-byte codes there."""
    check_layer(Fp8Layer(cfg(name=case, **CASES[case]), fmt="int4"))


@pytest.mark.parametrize("fmt", ["e4m3", "int8", "int4"])
def test_fp8_decode_full_size(fmt):
    """The decode workload (T 64, d 4096, E 8, d_ff 14336) with one-byte
    weights, sampled rows at each expert's ends and middle."""
    c = moe_synth.CONFIGS["decode"]

    def sample(offs):
        rows = set()
        for e in range(len(offs) - 1):
            b, en = int(offs[e]), int(offs[e + 1])
            rows.update(r for r in (b, en - 1, (b + en) // 2) if b <= r < en)
        return np.array(sorted(rows), np.int32)

    check_layer(Fp8Layer(c, fmt=fmt), full=True, rows_sample=sample)


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
@pytest.mark.parametrize("name", ["skew", "mixtral"])
def test_fp8_prefill_full_size(name, fmt):
    """Prefill workloads with one-byte weights (the MFMA tile): sampled rows
    at each expert's ends, m-tile boundaries and middle; sampled tokens."""
    c = moe_synth.CONFIGS[name]

    def sample(offs):
        rows = set()
        for e in range(len(offs) - 1):
            b, en = int(offs[e]), int(offs[e + 1])
            rows.update(r for r in (b, en - 1, (b + en) // 2, b + 255, b + 256) if b <= r < en)
        return np.array(sorted(rows), np.int32)

    check_layer(Fp8Layer(c, fmt=fmt), full=False, rows_sample=sample)


def test_fp8_empty_batch():
    L = Fp8Layer(cfg(T=4))
    p = moe.Params(T=0, d=512, E=8, k=2, d_ff=1024, capacity_factor=1.25, dtype=moe.MOE_BF16)
    r = moe.Routing(p, DEV)
    y = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    logits = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    moe.forward_fp8(p, L.x[:0], L.wr, L.bias, None, *L.weights(), y, logits, r, moe.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    assert int(r.offsets.cpu()[-1]) == 0


def test_fp8_fp32_layer_unsupported():
    """One-byte weights serve bf16 layers only."""
    L = Fp8Layer(cfg(T=4))
    p = moe.Params(T=64, d=512, E=8, k=2, d_ff=1024, capacity_factor=1.0, dtype=moe.MOE_F32)
    x = torch.zeros((64, 512), dtype=torch.float32, device=DEV)
    r = moe.Routing(p, DEV)
    with pytest.raises(moe.MoEError) as ei:
        moe.forward_fp8(p, x, L.wr.float(), None, None, *L.weights(), torch.empty_like(x),
                        torch.empty((64, 8), device=DEV), r, moe.alloc_workspace(p, DEV))
    assert ei.value.code == moe.MOE_ERR_UNSUPPORTED
