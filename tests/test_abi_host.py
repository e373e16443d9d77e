"""Host-side checks of the C ABI library: it loads, exports what include/moe.h
declares, and its pure host functions and argument checks behave (no GPU)."""
import ctypes
import os
import re

import pytest

import sparse_mixture_experts_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward"} <= set(names)
    L = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/moe.h but not exported"


def P(**kw):
    base = dict(T=64, d=128, E=8, k=2, d_ff=256, capacity_factor=1.0, reroute=1, lam=0.0,
                aux_coef=0.01, dtype=moe.MOE_F32)
    base.update(kw)
    return moe.Params(**base)


def test_capacity_matches_oracle(oracle_mod):
    cases = [(64, 2, 8, 1.0), (4096, 2, 8, 1.25), (8192, 2, 64, 1.0), (2048, 2, 16, 1.0),
             (64, 2, 8, 1.25), (32, 2, 64, 1.3), (1000, 3, 7, 1.1), (5, 1, 8, 0.0), (7, 2, 3, 50.0),
             (0, 2, 8, 1.0), (1, 1, 1, 1.0)]
    for T, k, E, cf in cases:
        p = P(T=T, k=k, E=E, capacity_factor=cf)
        assert moe.capacity(p) == oracle_mod.capacity(T, k, E, cf), (T, k, E, cf)
        C = oracle_mod.capacity(T, k, E, cf)
        assert moe.max_rows(p) == min(T * k, E * C)


def splits_of(p):
    """Slices of the down projection, read back from moe_expert_ffn's scratch
    size: slices 1.. each take R x d fp32."""
    R = moe.max_rows(p)
    return 1 + moe.ffn_workspace_bytes(p) // (R * p.d * 4)


def down_split(p, R):
    """moe_forward's down-projection split on the 256-row GEMM (more than 32
    rows per expert), restated: the split plan for the bound on the m tiles
    (min(R / 256 + E, E ceil(C / 256))) of ntn = ceil(d / 256) n tiles: the
    tiles fill whole rounds of 256 -> one slice; else G = the last round's
    m tiles rounded up, S = min(256 / (G ntn), clamp(d_ff / 512, 1, 8));
    S = 1 -> one slice; G = every m tile -> S uniform slices; otherwise the
    device-side plan."""
    C = moe.capacity(p)
    if C <= 32:
        return "uniform", 1
    mt = min(R // 256 + p.E, p.E * -(-C // 256))
    ntn, nk = -(-p.d // 256), p.d_ff // 64
    rem = (mt * ntn) % 256
    if rem == 0:
        return "uniform", 1
    G = min(mt, -(-rem // ntn))
    S = min(256 // (G * ntn), min(8, max(1, nk // 8)))
    if S <= 1:
        return "uniform", 1
    if G == mt and nk % S == 0:
        return "uniform", S
    return "planned", 1


def gated_rows_bytes(p, R):
    """moe_forward's gated fp16 rows: slice 0 [R][d], plus (when the down
    projection is split) the further slices, at most min(2^24, (S_max - 1) R d)
    elements, S_max = clamp(d_ff / 512, 1, 8)."""
    extra = 0
    if down_split(p, R) != ("uniform", 1):
        smax = min(8, max(1, p.d_ff // 64 // 8))
        extra = min(1 << 24, (smax - 1) * R * p.d)
    return (R * p.d + extra) * 2


def test_workspace_sizes_cover_buffers():
    p = P(T=4096, d=4096, E=8, k=2, d_ff=14336, capacity_factor=1.25, dtype=moe.MOE_BF16)
    R = moe.max_rows(p)
    assert R == 8192
    ws = moe.workspace_bytes(p)
    S = splits_of(p)
    assert S == 2 and moe.ffn_workspace_bytes(p) == (S - 1) * R * 4096 * 4
    # h [R][d_ff] (fp16), the gated rows (slice 0 [R][d] fp16 and at most
    # 2^24 elements of the split rows' further slices) and the row gates [R];
    # x spans less than 2 GiB, so moe_forward reads the gate-up rows from x and
    # needs no x_perm
    assert down_split(p, R) == ("planned", 1)
    assert gated_rows_bytes(p, R) == (R * 4096 + (1 << 24)) * 2
    base = R * 14336 * 2 + gated_rows_bytes(p, R) + R * 4 + moe.dispatch_workspace_bytes(p)
    assert base <= ws < base + R * 4096 * 2
    assert moe.dispatch_workspace_bytes(p) > 0
    # an fp32 layer keeps y_perm [R][d] in fp32 and needs no row gates
    q = P(T=700, d=256, E=4, k=2, d_ff=384, capacity_factor=1.0, dtype=moe.MOE_F32)
    Rq = moe.max_rows(q)
    assert moe.ffn_workspace_bytes(q) == 0
    base = Rq * 384 * 4 + Rq * 256 * 4 + moe.dispatch_workspace_bytes(q)
    assert base <= moe.workspace_bytes(q) < base + 6 * 256
    # x of 2 GiB and more: moe_forward writes x_perm [R][d] into its workspace
    for T, has_xp in (((1 << 18) - 1, False), (1 << 18, True)):
        q = P(T=T, d=4096, E=8, k=2, d_ff=1024, capacity_factor=1.0, dtype=moe.MOE_BF16)
        Rq = moe.max_rows(q)
        base = Rq * 1024 * 2 + gated_rows_bytes(q, Rq) + Rq * 4 + moe.dispatch_workspace_bytes(q)
        wq = moe.workspace_bytes(q)
        assert (wq >= base + Rq * 4096 * 2) == has_xp and wq >= base, (T, wq, base)


def test_forward_down_split_choice():
    """Which down projection moe_forward runs, read back from its workspace
    size: the Mixtral-shape layer the planned split (the last round's m tiles
    split), the skewed layer two uniform slices (every tile split), the
    fine-grained layer one slice (the tiles fill whole rounds), decode the
    weight-streaming kernel's one slice."""
    mix = P(T=4096, d=4096, E=8, k=2, d_ff=14336, capacity_factor=1.25, dtype=moe.MOE_BF16)
    skew = P(T=2048, d=2048, E=16, k=2, d_ff=5632, capacity_factor=1.0, dtype=moe.MOE_BF16)
    fine = P(T=8192, d=4096, E=64, k=2, d_ff=2048, capacity_factor=1.0, dtype=moe.MOE_BF16)
    dec = P(T=64, d=4096, E=8, k=2, d_ff=14336, capacity_factor=1.25, dtype=moe.MOE_BF16)
    want = {"mix": ("planned", 1), "skew": ("uniform", 2), "fine": ("uniform", 1), "dec": ("uniform", 1)}
    for name, q in (("mix", mix), ("skew", skew), ("fine", fine), ("dec", dec)):
        R = moe.max_rows(q)
        assert down_split(q, R) == want[name], name
        # the workspace holds exactly the gated rows the choice needs
        rest = moe.workspace_bytes(q) - gated_rows_bytes(q, R)
        assert 0 < rest - q.d_ff * R * 2 - R * 4 - moe.dispatch_workspace_bytes(q) < 8 * 256, name


def test_ffn_workspace_only_for_split_down_projections():
    """The expert FFN needs scratch only where its down projection is split
    (few row tiles for the chip): the Mixtral-shape layer and the skewed
    layer (2 slices each), not the fine-grained layer, the decode shape or
    fp32."""
    mix = P(T=4096, d=4096, E=8, k=2, d_ff=14336, capacity_factor=1.25, dtype=moe.MOE_BF16)
    skew = P(T=2048, d=2048, E=16, k=2, d_ff=5632, capacity_factor=1.0, dtype=moe.MOE_BF16)
    fine = P(T=8192, d=4096, E=64, k=2, d_ff=2048, capacity_factor=1.0, dtype=moe.MOE_BF16)
    dec = P(T=64, d=4096, E=8, k=2, d_ff=14336, capacity_factor=1.25, dtype=moe.MOE_BF16)
    assert (splits_of(mix), splits_of(skew), splits_of(fine), splits_of(dec)) == (2, 2, 1, 1)
    assert moe.ffn_workspace_bytes(fine) == moe.ffn_workspace_bytes(dec) == 0


@pytest.mark.parametrize("cf", [float("inf"), 1e30, 3.0e38, 1e19])
def test_huge_capacity_factor_is_uncapped(cf, oracle_mod):
    """A capacity factor so large that T*k/E*cf exceeds the int64 range (or
    is infinite) still gives C = T: the clamp comes before the conversion."""
    for T, k, E in ((64, 2, 8), (4096, 2, 8), (1, 1, 1), (1000, 8, 256)):
        p = P(T=T, k=k, E=E, capacity_factor=cf)
        assert moe.capacity(p) == T, (T, k, E, cf)
        assert moe.max_rows(p) == T * k
        assert oracle_mod.capacity(T, k, E, cf) == T


def test_d_ff_bound_of_the_down_tile():
    """A 256-row tile of h must span less than 2 GiB: d_ff < 2^22."""
    assert moe.capacity(P(d=64, d_ff=(1 << 22) - 64)) == 16  # accepted: C = ceil(64 * 2 / 8)
    r = moe.MoeRouting()
    p = P(d=64, d_ff=1 << 22)
    rc = moe.lib().moe_forward(ctypes.byref(p.c()), None, None, None, None, None, None, None, None,
                               None, ctypes.byref(r), None, 0, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("bad", [dict(E=0), dict(E=257), dict(k=0), dict(k=9, E=16), dict(k=3, E=2),
                                 dict(T=-1), dict(T=(1 << 20) + 1), dict(d=0), dict(gate_temperature=-0.5),
                                 dict(gate_temperature=float("nan")), dict(gate_temperature=float("inf")),
                                 dict(top2_gap=-0.1), dict(top2_gap=float("nan")), dict(top2_gap=float("inf")),
                                 dict(router_hidden=-1)])
def test_invalid_sizes_rejected(bad):
    p = P(**bad)
    assert moe.capacity(p) == -1
    assert moe.workspace_bytes(p) == 0
    r = moe.MoeRouting()
    rc = moe.lib().moe_route(ctypes.byref(p.c()), None, None, None, None, None, ctypes.byref(r), None)
    assert rc == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [dict(d=100), dict(d_ff=96), dict(dtype=7), dict(d=16384 + 64),
                                 dict(d=16384, d_ff=131072, dtype=moe.MOE_BF16),  # one expert matrix of 4 GiB
                                 dict(d=8192, d_ff=131072, dtype=moe.MOE_F32),
                                 dict(router_hidden=257),  # two-layer router: at most 256 hidden units
                                 dict(router_hidden=257, dtype=moe.MOE_BF16)])
def test_unsupported_shapes_rejected(bad):
    p = P(**bad)
    r = moe.MoeRouting()
    rc = moe.lib().moe_forward(ctypes.byref(p.c()), None, None, None, None, None, None, None, None,
                               None, ctypes.byref(r), None, 0, None)
    assert rc == moe.MOE_ERR_UNSUPPORTED


def test_null_pointers_rejected():
    p = P()
    r = moe.MoeRouting()  # all members NULL
    assert moe.lib().moe_route(ctypes.byref(p.c()), 16, 16, None, None, 16, ctypes.byref(r), None) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_dispatch(ctypes.byref(p.c()), 16, ctypes.byref(r), 16, 16, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_expert_ffn(ctypes.byref(p.c()), 16, None, 16, 16, 16, 16, 16, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_combine(ctypes.byref(p.c()), 16, None, None, 16, None) == moe.MOE_ERR_INVALID_ARG


def test_workspace_too_small_rejected():
    p = P()
    names = moe.Routing.NAMES
    r = moe.MoeRouting(*[256] * len(names))  # non-null fake addresses; never dereferenced
    need = moe.workspace_bytes(p)
    rc = moe.lib().moe_forward(ctypes.byref(p.c()), 256, 256, None, None, 256, 256, 256, 256, 256,
                               ctypes.byref(r), 256, need - 1, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    rc = moe.lib().moe_dispatch(ctypes.byref(p.c()), 256, ctypes.byref(r), 256, 256,
                                moe.dispatch_workspace_bytes(p) - 1, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
    # a split down projection needs its scratch
    q = P(T=4096, d=4096, E=8, k=2, d_ff=14336, capacity_factor=1.25, dtype=moe.MOE_BF16)
    need = moe.ffn_workspace_bytes(q)
    assert need > 0
    for ws, nb in ((None, 0), (256, need - 1)):
        rc = moe.lib().moe_expert_ffn(ctypes.byref(q.c()), 256, 256, 256, 256, 256, 256, 256, ws, nb, None)
        assert rc == moe.MOE_ERR_INVALID_ARG


def test_misaligned_pointer_rejected():
    p = P()
    r = moe.MoeRouting(*[256] * len(moe.Routing.NAMES))
    rc = moe.lib().moe_route(ctypes.byref(p.c()), 258, 256, None, None, 256, ctypes.byref(r), None)
    assert rc == moe.MOE_ERR_UNSUPPORTED


def test_strerror():
    assert moe.strerror(0) == "ok"
    for c in (-1, -2, -3, 5):
        assert isinstance(moe.strerror(c), str) and moe.strerror(c)


def test_dynamic_capacity_matches_oracle(oracle_mod):
    for T, k, E in ((32, 2, 64), (1000, 2, 12), (4096, 2, 8), (1, 1, 1), (0, 2, 8), (8191, 4, 16), (3, 2, 2)):
        p = P(T=T, k=k, E=E, capacity_factor=-1.0, dynamic_capacity=1)
        assert moe.capacity(p) == oracle_mod.capacity_dynamic(T, k, E), (T, k, E)
    bad = P(dynamic_capacity=2)
    r = moe.MoeRouting()
    rc = moe.lib().moe_forward(ctypes.byref(bad.c()), None, None, None, None, None, None, None, None,
                               None, ctypes.byref(r), None, 0, None)
    assert rc == moe.MOE_ERR_INVALID_ARG


def i4_ffn_rc(p, s_ptr=256):
    return moe.lib().moe_expert_ffn_i4(ctypes.byref(p.c()), 256, 256, 256, s_ptr, 256, s_ptr, 256, s_ptr,
                                       256, 256, None)


def test_int4_weights_limits_rejected():
    """INT4 expert weights run on the weight-streaming kernel only: bf16
    layers whose experts hold at most 32 rows, d and d_ff multiples of 128;
    a layer with larger groups is unsupported (not an invalid argument) and
    missing scales are an invalid argument.  Every case is rejected before
    any launch (the fake addresses are never touched)."""
    ok = dict(T=64, d=512, E=8, k=2, d_ff=1024, capacity_factor=1.25, dtype=moe.MOE_BF16)
    assert moe.capacity(P(**ok)) == 20
    assert i4_ffn_rc(P(**ok), s_ptr=None) == moe.MOE_ERR_INVALID_ARG
    for bad in (dict(dtype=moe.MOE_F32), dict(d=448), dict(d_ff=960), dict(T=256, capacity_factor=1.0),
                dict(capacity_factor=-1.0)):
        kw = dict(ok)
        kw.update(bad)
        assert i4_ffn_rc(P(**kw)) == moe.MOE_ERR_UNSUPPORTED, bad
    r = moe.MoeRouting(*[256] * len(moe.Routing.NAMES))
    big = P(**dict(ok, T=256, capacity_factor=1.0))
    assert moe.capacity(big) == 64
    rc = moe.lib().moe_forward_i4(ctypes.byref(big.c()), 256, 256, None, None, 256, 256, 256, 256, 256, 256,
                                  256, 256, ctypes.byref(r), 256, moe.workspace_bytes(big), None)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    rc = moe.lib().moe_forward_i4(ctypes.byref(P(**ok).c()), 256, 256, None, None, 256, None, 256, 256, 256,
                                  256, 256, 256, ctypes.byref(r), 256, 1 << 30, None)
    assert rc == moe.MOE_ERR_INVALID_ARG


def fp8_ffn_rc(p, s_ptr=256):
    return moe.lib().moe_expert_ffn_fp8(ctypes.byref(p.c()), 256, 256, 256, s_ptr, 256, s_ptr, 256, s_ptr,
                                        256, 256, None)


def test_fp8_weights_limits_rejected():
    """One-byte expert weights: bf16 layers only; groups of at most 32 rows
    per expert (the weight-streaming kernel) need d and d_ff multiples of
    128, larger groups (the matrix-core tile) multiples of 64; missing scales
    are an invalid argument.  The checks come before any launch (the fake
    addresses are never touched)."""
    ok = dict(T=64, d=512, E=8, k=2, d_ff=1024, capacity_factor=1.25, dtype=moe.MOE_BF16)
    assert moe.capacity(P(**ok)) == 20
    assert fp8_ffn_rc(P(**ok), s_ptr=None) == moe.MOE_ERR_INVALID_ARG
    for bad in (dict(dtype=moe.MOE_F32), dict(d=448), dict(d_ff=960), dict(T=256, capacity_factor=1.0,
                                                                              dtype=moe.MOE_F32)):
        kw = dict(ok)
        kw.update(bad)
        assert fp8_ffn_rc(P(**kw)) == moe.MOE_ERR_UNSUPPORTED, bad
    # groups of more than 32 rows take d and d_ff multiples of 64: the missing
    # scale is then the first error found
    big = dict(ok, T=256, capacity_factor=1.0, d=448, d_ff=960)
    assert moe.capacity(P(**big)) == 64
    assert fp8_ffn_rc(P(**big), s_ptr=None) == moe.MOE_ERR_INVALID_ARG
    r = moe.MoeRouting(*[256] * len(moe.Routing.NAMES))
    p = P(**dict(ok, T=256, capacity_factor=1.0, dtype=moe.MOE_F32))
    rc = moe.lib().moe_forward_fp8(ctypes.byref(p.c()), 256, 256, None, None, 256, 256, 256, 256, 256, 256,
                                   256, 256, ctypes.byref(r), 256, moe.workspace_bytes(p), None)
    assert rc == moe.MOE_ERR_UNSUPPORTED
    rc = moe.lib().moe_forward_fp8(ctypes.byref(P(**ok).c()), 256, 256, None, None, 256, None, 256, 256, 256,
                                   256, 256, 256, ctypes.byref(r), 256, 1 << 30, None)
    assert rc == moe.MOE_ERR_INVALID_ARG
