"""Pins of the CPU oracle against things other than itself.

Each check ties one oracle step to what the pages print (tests/golden), to a
closed form, to exact arithmetic, to brute force on tiny inputs, or to a
special case that reduces to a textbook routine.  A plausible mistake in the
oracle (a dropped term, a wrong index, a transposed operand, ties to the wrong
side, a double rounding in the penalty, a token-major queue) fails at least
one of them; tests/test_oracle_mutations.py plants such mistakes and checks
that they are caught.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def rng(seed=0):
    return np.random.default_rng(seed)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits (test-side conversion)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- capacity --

def check_capacity(o):
    g = GOLD["capacity_worked"]
    assert o.capacity(g["T"], g["k"], g["E"], g["cf"]) == g["capacity"]
    # the five workloads' capacities: ceil(T*k/E*cf)
    for (T, k, E, cf), C in [((64, 2, 8, 1.0), 16), ((4096, 2, 8, 1.25), 1280),
                             ((8192, 2, 64, 1.0), 256), ((2048, 2, 16, 1.0), 256),
                             ((64, 2, 8, 1.25), 20)]:
        assert o.capacity(T, k, E, cf) == C
    # ceiling, not floor: 10 tokens, top-1, 4 experts, cf 1 -> 2.5 -> 3
    assert o.capacity(10, 1, 4, 1.0) == 3
    # uncapped and clamped to T
    assert o.capacity(7, 2, 3, 0.0) == 7
    assert o.capacity(7, 2, 3, 100.0) == 7


def test_capacity_pins(oracle_mod):
    check_capacity(oracle_mod)


def check_dynamic_capacity(o):
    """The dynamic factor against the page's worked value (1.05 at a batch of
    32), its exact values at powers of two, its floor at one token, and the
    capacity it gives (ceil(T*k/E*cf) with cf in double)."""
    g = GOLD["dynamic_capacity_factor_worked"]
    assert abs(o.dynamic_capacity_factor(g["T"]) - g["cf"]) < 1e-15
    for e in range(0, 21):
        assert o.dynamic_capacity_factor(2 ** e) == 1.0 + 0.01 * e
    assert o.dynamic_capacity_factor(0) == 1.0
    assert 1.0 + 0.01 * math.log2(1000) - 1e-15 < o.dynamic_capacity_factor(1000) < 1.0 + 0.01 * math.log2(1000) + 1e-15
    # T 4096, top-2, 8 experts: cf 1.12 -> ceil(1024 * 1.12) = 1147
    assert o.capacity_dynamic(4096, 2, 8) == math.ceil(4096 * 2 / 8 * (1.0 + 0.01 * 12))
    assert o.capacity_dynamic(4096, 2, 8) == 1147
    # 32 tokens, top-2, 64 experts: ceil(1 * 1.05) = 2
    assert o.capacity_dynamic(32, 2, 64) == 2
    assert o.capacity_dynamic(1, 1, 1) == 1


def test_dynamic_capacity(oracle_mod):
    check_dynamic_capacity(oracle_mod)


# ----------------------------------------------------------- router logits --

def check_router_logits(o):
    r = rng(1)
    T, d, E = 5, 12, 7
    x = r.standard_normal((T, d)).astype(np.float32)
    # one-hot gate vectors pick input features: raw[t, e] = x[t, perm[e]]
    perm = r.permutation(d)[:E]
    wr = np.zeros((E, d), np.float32)
    wr[np.arange(E), perm] = 1.0
    raw = o.router_logits(x, wr)
    assert np.array_equal(raw, x[:, perm])
    # bias is added per expert
    b = r.standard_normal(E).astype(np.float32)
    raw_b = o.router_logits(x, wr, b)
    assert np.array_equal(raw_b, (x[:, perm] + b[None, :]).astype(np.float32))
    # linearity in the weights (exact for small integers)
    xi = r.integers(-3, 4, (T, d)).astype(np.float32)
    w1 = r.integers(-3, 4, (E, d)).astype(np.float32)
    w2 = r.integers(-3, 4, (E, d)).astype(np.float32)
    assert np.array_equal(o.router_logits(xi, w1 + w2), o.router_logits(xi, w1) + o.router_logits(xi, w2))
    # bf16 bit patterns widen exactly: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E00 = 0.125
    xb = np.array([[0x3F80, 0xC000, 0x3E00]], np.uint16)
    wb = np.array([[0x3F80, 0x3F80, 0x3F80], [0x3F80, 0x0000, 0x0000]], np.uint16)
    assert np.array_equal(o.router_logits(xb, wb), np.array([[1.0 - 2.0 + 0.125, 1.0]], np.float32))


def test_router_logits_pins(oracle_mod):
    check_router_logits(oracle_mod)


# ------------------------------------------------------------- penalty fma --

def _round_f32_exact(v: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 of an exact rational."""
    a = np.float32(float(v))
    cands = {a, np.nextafter(a, np.float32(np.inf)), np.nextafter(a, np.float32(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        err = abs(Fraction(float(c)) - v)
        key = (err, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def check_scores(o):
    r = rng(2)
    T, E = 40, 9
    raw = r.standard_normal((T, E)).astype(np.float32)
    load = r.random(E).astype(np.float32)
    # lambda 0 and no load are the identity
    assert np.array_equal(o.scores(raw, load, 0.0), raw)
    assert np.array_equal(o.scores(raw, None, 0.7), raw)
    lam = np.float32(0.3)
    s = o.scores(raw, load, lam)
    for t in range(T):
        for e in range(E):
            exact = Fraction(float(raw[t, e])) - Fraction(float(lam)) * Fraction(float(load[e]))
            assert s[t, e] == _round_f32_exact(exact), (t, e)
    # a case where rounding the product first changes the result:
    # raw = 1 + 2^-11 + 2^-22, lam = load = 1 + 2^-12, so lam*load = 1 + 2^-11 + 2^-24
    # (not an fp32); one rounding gives 3*2^-24, two roundings give 2^-22.
    raw1 = np.array([[1.0 + 2.0 ** -11 + 2.0 ** -22]], np.float32)
    load1 = np.array([1.0 + 2.0 ** -12], np.float32)
    lam1 = np.float32(1.0 + 2.0 ** -12)
    got = o.scores(raw1, load1, lam1)[0, 0]
    exact = Fraction(float(raw1[0, 0])) - Fraction(float(lam1)) * Fraction(float(load1[0]))
    assert got == _round_f32_exact(exact) == np.float32(3.0 * 2.0 ** -24)
    two_step = np.float32(raw1[0, 0] - np.float32(lam1 * load1[0]))
    assert got != two_step  # the separate-rounding reading differs here


def test_scores_fma_exact(oracle_mod):
    check_scores(oracle_mod)


# ------------------------------------------------------------------- top-k --

def check_topk(o):
    r = rng(3)
    for E in (1, 2, 3, 5, 8):
        for K in range(1, E + 2):
            s = r.integers(0, 3, (60, E)).astype(np.float32)  # many ties
            cand, cs = o.topk(s, K)
            for t in range(s.shape[0]):
                order = sorted(range(E), key=lambda e: (-s[t, e], e))
                want = order[:K] + [-1] * max(0, K - E)
                assert list(cand[t]) == want, (E, K, t)
                for j, e in enumerate(want):
                    if e >= 0:
                        assert cs[t, j] == s[t, e]
                    else:
                        assert cs[t, j] == -np.inf
    # numpy's stable lexsort agrees on continuous scores
    s = r.standard_normal((200, 16)).astype(np.float32)
    cand, _ = o.topk(s, 3)
    ref = np.lexsort((np.tile(np.arange(16), (200, 1)), -s), axis=1)[:, :3]
    assert np.array_equal(cand, ref)
    # signed zeros are equal scores: the lower index wins
    s = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert list(o.topk(s, 2)[0][0]) == [0, 1]
    s = np.array([[0.0, -0.0, -1.0]], np.float32)
    assert list(o.topk(s, 2)[0][0]) == [0, 1]
    # NaN scores come after every number (-inf included), NaNs by index; a row
    # of NaNs still names E experts
    s = r.integers(0, 3, (60, 6)).astype(np.float32)
    s[r.random(s.shape) < 0.3] = np.nan
    s[::7, 5] = -np.inf
    s[5] = np.nan
    cand, cs = o.topk(s, 7)
    for t in range(s.shape[0]):
        order = sorted(range(6), key=lambda e: (bool(np.isnan(s[t, e])),
                                                0.0 if np.isnan(s[t, e]) else -float(s[t, e]), e))
        assert list(cand[t]) == order + [-1], t
        assert np.array_equal(cs[t, :6], s[t, order], equal_nan=True)


def test_topk_pins(oracle_mod):
    check_topk(oracle_mod)


# ---------------------------------------------------------------- dispatch --

def declarative_dispatch(cand, E, k, C, reroute):
    """The queue written as counting statements, one element at a time.

    A primary request (t, r) to expert e is kept iff fewer than C primary
    requests to e come before it in the arrival order (rank-major, then token).
    Token t asks for a fallback iff one of its primary slots was refused; the
    request goes to cand[t][k] and is kept iff the primaries kept there plus
    the fallback requests to it from earlier tokens number fewer than C.
    """
    T = cand.shape[0]
    K = k + 1
    prim = {}
    for t in range(T):
        for r in range(k):
            e = cand[t, r]
            before = sum(1 for (t2, r2) in itertools.product(range(T), range(k))
                         if cand[t2, r2] == e and (r2, t2) < (r, t))
            prim[(t, r)] = before
    eid = np.full((T, k), -1, np.int64)
    pos = np.full((T, k), -1, np.int64)
    flag = np.full((T, k), 2, np.int64)
    for (t, r), before in prim.items():
        if before < C:
            eid[t, r], pos[t, r], flag[t, r] = cand[t, r], before, 0
    kept_prim = np.zeros(E, np.int64)
    for (t, r), before in prim.items():
        if before < C:
            kept_prim[cand[t, r]] += 1
    if reroute and k < E:
        asks = [t for t in range(T) if any(prim[(t, r)] >= C for r in range(k))]
        for t in asks:
            f = cand[t, k]
            earlier = sum(1 for t2 in asks if t2 < t and cand[t2, k] == f)
            p = kept_prim[f] + earlier
            if p < C:
                r0 = min(r for r in range(k) if prim[(t, r)] >= C)
                eid[t, r0], pos[t, r0], flag[t, r0] = f, p, 1
    return eid, pos, flag


def fifo_simulation(cand, E, k, C, reroute):
    """Literal event-by-event queue simulation with per-expert lists."""
    T = cand.shape[0]
    queues = [[] for _ in range(E)]
    where = {}
    events = [(r, t) for r in range(k) for t in range(T)]
    refused = {t: [] for t in range(T)}
    for (r, t) in events:
        e = cand[t, r]
        if len(queues[e]) < C:
            queues[e].append((t, r))
            where[(t, r)] = (e, len(queues[e]) - 1, 0)
        else:
            refused[t].append(r)
    if reroute and k < E:
        for t in range(T):
            if refused[t]:
                r0 = min(refused[t])
                f = cand[t, k]
                if len(queues[f]) < C:
                    queues[f].append((t, r0))
                    where[(t, r0)] = (f, len(queues[f]) - 1, 1)
    return queues, where


def check_dispatch_exhaustive(o):
    # every ordered candidate list for T=4 tokens, E=3 experts, k=2 (+fallback)
    perms = list(itertools.permutations(range(3)))
    E, k = 3, 2
    n = 0
    for combo in itertools.product(perms, repeat=4):
        cand = np.array(combo, np.int32)
        cs = np.tile(np.array([3.0, 2.0, 1.0], np.float32), (4, 1))
        for C in (1, 2, 3, 4):
            for reroute in (0, 1):
                got = o.dispatch(cand, cs, E, k, C, reroute)
                eid, pos, flag = declarative_dispatch(cand, E, k, C, reroute)
                assert np.array_equal(got["eid"], eid), (combo, C)
                assert np.array_equal(got["pos"], pos), (combo, C)
                assert np.array_equal(got["flag"], flag), (combo, C)
                queues, where = fifo_simulation(cand, E, k, C, reroute)
                assert list(got["kept"]) == [len(q) for q in queues]
                for e in range(E):
                    for p, (t, r) in enumerate(queues[e]):
                        row = got["offsets"][e] + p
                        assert got["token_of_row"][row] == t
                        assert got["row"][t, r] == row
                n += 1
    assert n == 1296 * 8


def test_dispatch_exhaustive_tiny(oracle_mod):
    check_dispatch_exhaustive(oracle_mod)


def check_dispatch_invariants(o, T=300, E=6, k=2, C=90, reroute=1, seed=4):
    r = rng(seed)
    s = (r.standard_normal((T, E)) + np.array([1.5] + [0.0] * (E - 1))).astype(np.float32)
    cand, cs = o.topk(s, k + 1)
    d = o.dispatch(cand, cs, E, k, C, reroute, 0.01)
    rows, dropped, rer = d["totals"]
    assert d["demand"].sum() == T * k
    assert np.array_equal(d["demand"], np.bincount(cand[:, :k].ravel(), minlength=E))
    assert (d["kept"] <= C).all()
    assert rows == d["kept"].sum() == T * k - dropped
    assert rer == (d["flag"] == 1).sum() and dropped == (d["flag"] == 2).sum()
    assert d["offsets"][0] == 0 and np.array_equal(np.diff(d["offsets"]), d["kept"])
    # bijection between kept slots and rows
    kept_mask = d["flag"] != 2
    rws = d["row"][kept_mask]
    assert sorted(rws.tolist()) == list(range(rows))
    ts = np.nonzero(kept_mask)[0]
    assert np.array_equal(d["token_of_row"][rws], ts)
    assert (d["token_of_row"][rows:] == -1).all()
    # a token never holds one expert twice
    for t in range(T):
        es = [e for e in d["eid"][t] if e >= 0]
        assert len(es) == len(set(es))
    # gates: renormalised softmax over kept slots
    for t in range(T):
        m = kept_mask[t]
        if m.any():
            assert abs(d["gate64"][t][m].sum() - 1.0) < 1e-12
            assert abs(float(d["gate"][t][m].astype(np.float64).sum()) - 1.0) < 1e-6
            src = [r_ if d["flag"][t, r_] == 0 else k for r_ in range(k)]
            sc = np.array([cs[t, src[r_]] for r_ in range(k)], np.float64)
            idx = np.nonzero(m)[0]
            for a in idx:
                for b in idx:
                    assert math.isclose(d["gate64"][t, a] / d["gate64"][t, b],
                                        math.exp(sc[a] - sc[b]), rel_tol=1e-12)
        assert (d["gate"][t][~m] == 0).all()
    return d


def check_gate_temperature(o):
    """Gates at temperature tau are the softmax of score / tau over the kept
    slots ("MoE稀疏激活原理与工程实践" §3.1, third step): the routing does not
    change with tau, two kept slots have the gate ratio exp((s_a - s_b) / tau),
    a tiny tau puts the whole gate on the best kept slot and a huge one
    spreads it evenly."""
    T, E, k, C = 300, 6, 2, 90
    r = rng(4)
    s = (r.standard_normal((T, E)) + np.array([1.5] + [0.0] * (E - 1))).astype(np.float32)
    cand, cs = o.topk(s, k + 1)
    base = o.dispatch(cand, cs, E, k, C, 1, 0.01)
    for tau in (0.5, 4.0, 1e-3, 1e3):
        d = o.dispatch(cand, cs, E, k, C, 1, 0.01, tau)
        for n in ("eid", "pos", "flag", "row", "offsets", "token_of_row", "kept", "totals"):
            assert np.array_equal(d[n], base[n]), (tau, n)
        for t in range(T):
            m = d["flag"][t] != 2
            idx = np.nonzero(m)[0]
            src = [r_ if d["flag"][t, r_] == 0 else k for r_ in range(k)]
            sc = np.array([cs[t, src[r_]] for r_ in range(k)], np.float64)
            if len(idx) == 2:
                a, b = idx
                x = (sc[a] - sc[b]) / tau
                if abs(x) < 500:
                    assert math.isclose(d["gate64"][t, a] / d["gate64"][t, b], math.exp(x), rel_tol=1e-12)
            if len(idx):
                assert abs(d["gate64"][t][m].sum() - 1.0) < 1e-12
                if tau == 1e3:
                    assert np.allclose(d["gate64"][t][m], 1.0 / len(idx), atol=2e-3)
                if tau == 1e-3 and len(idx) == 2 and abs(sc[idx[0]] - sc[idx[1]]) > 0.05:
                    best = idx[np.argmax(sc[idx])]
                    assert d["gate64"][t, best] > 1.0 - 1e-12
    return base


def check_router_glu(o):
    """Two-layer router ("MoE稀疏激活原理与工程实践" §3.1, second step), pinned
    through the linear router (itself pinned above): with W2 = I (H = E) the
    logits are silu of the linear router's; far in silu's linear regime they
    are the linear router of the product W2 W1; relabelling the hidden units
    (rows of W1 with the columns of W2) changes nothing; W2 = 0 leaves the
    bias."""
    r = rng(11)
    T, d, E = 40, 24, 6
    H = 2 * E
    x = r.standard_normal((T, d)).astype(np.float32)
    w1 = (r.standard_normal((H, d)) / np.sqrt(d)).astype(np.float32)
    w2 = (r.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32)
    b = r.standard_normal(E).astype(np.float32)
    # W2 = I: silu of the linear logits (no bias, H = E)
    w1e = w1[:E].copy()
    lin = o.router_logits(x, w1e).astype(np.float64)
    glu_i = o.router_logits_glu(x, w1e, np.eye(E, dtype=np.float32))
    assert np.allclose(glu_i, lin / (1.0 + np.exp(-lin)), rtol=1e-6, atol=1e-6)
    # silu's linear regime: pre-activations near 40 (silu(v) = v to 1e-17)
    w1p = np.abs(w1) + 0.05
    xp = (np.abs(x) * 40.0 / (np.abs(x) @ w1p.T).mean()).astype(np.float32)
    glu_l = o.router_logits_glu(xp, w1p, w2).astype(np.float64)
    lin2 = o.router_logits(xp, (w2.astype(np.float64) @ w1p.astype(np.float64)).astype(np.float32))
    assert (xp.astype(np.float64) @ w1p.T.astype(np.float64)).min() > 20.0
    assert np.allclose(glu_l, lin2, rtol=1e-5, atol=1e-4)
    # hidden relabelling
    perm = r.permutation(H)
    g0 = o.router_logits_glu(x, w1, w2, b)
    gp = o.router_logits_glu(x, np.ascontiguousarray(w1[perm]), np.ascontiguousarray(w2[:, perm]), b)
    assert np.allclose(g0, gp, rtol=1e-6, atol=1e-6)
    # W2 = 0: the bias
    assert np.array_equal(o.router_logits_glu(x, w1, np.zeros((E, H), np.float32), b), np.tile(b, (T, 1)))
    # bf16 operands are read exactly (the same values in fp32 give the same logits)
    xb, w1b, w2b = (torch.from_numpy(a).to(torch.bfloat16) for a in (x, w1, w2))
    gb = o.router_logits_glu(xb, w1b, w2b, b)
    gf = o.router_logits_glu(xb.float().numpy(), w1b.float().numpy(), w2b.float().numpy(), b)
    assert np.array_equal(gb, gf)
    # the first layer's bias is one more input feature: a constant-1 column of
    # x whose W1 column is the bias (added before the silu, in the same sum)
    b1 = r.standard_normal(H).astype(np.float32)
    xa = np.ascontiguousarray(np.concatenate([x, np.ones((T, 1), np.float32)], axis=1))
    w1a = np.ascontiguousarray(np.concatenate([w1, b1[:, None]], axis=1))
    assert np.array_equal(o.router_logits_glu(x, w1, w2, b, bias1=b1), o.router_logits_glu(xa, w1a, w2, b))
    # the page's router code form, Linear(d, 2E) -> SiLU -> Linear(2E, E), by torch in float64
    lin1, lin2 = torch.nn.Linear(d, H).double(), torch.nn.Linear(H, E).double()
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1.astype(np.float64)))
        lin1.bias.copy_(torch.from_numpy(b1.astype(np.float64)))
        lin2.weight.copy_(torch.from_numpy(w2.astype(np.float64)))
        lin2.bias.zero_()
        ref = torch.nn.Sequential(lin1, torch.nn.SiLU(), lin2)(torch.from_numpy(x.astype(np.float64))).numpy()
    got = o.router_logits_glu(x, w1, w2, None, bias1=b1).astype(np.float64)
    assert np.allclose(got, ref.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_router_glu(oracle_mod):
    check_router_glu(oracle_mod)


def check_gap_swap(o):
    """Top-2 gap threshold (the adg.csdn.net page, §3.1): where the best two
    scores differ by less than delta, ranks 1 and 2 trade places (the second
    choice becomes the third-ranked expert); elsewhere the list is the plain
    ranking.  A printed-style example, then random rows checked one by one
    against the definition written out in fp32."""
    # best two within the threshold: 0.49 vs 0.48 (gap 0.01 < 0.05)
    s = np.array([[0.48, 0.10, 0.49, 0.30], [0.90, 0.48, 0.20, 0.10]], np.float32)
    cand, cs = o.topk(s, 3)
    c2, cs2 = o.gap_swap(cand, cs, 0.05)
    assert c2[0].tolist() == [2, 3, 0] and np.array_equal(cs2[0], np.float32([0.49, 0.30, 0.48]))
    assert c2[1].tolist() == cand[1].tolist()  # gap 0.42: unchanged
    assert np.array_equal(o.gap_swap(cand, cs, 0.0)[0], cand)  # off
    r = rng(9)
    T, E, K = 2000, 6, 3
    s = (r.standard_normal((T, E)) * 0.1).astype(np.float32)
    cand, cs = o.topk(s, K)
    delta = np.float32(0.05)
    c2, cs2 = o.gap_swap(cand, cs, delta)
    n_swapped = 0
    for t in range(T):
        if np.float32(cs[t, 0] - cs[t, 1]) < delta:
            n_swapped += 1
            assert c2[t].tolist() == [cand[t, 0], cand[t, 2], cand[t, 1]]
            assert np.array_equal(cs2[t], cs[t][[0, 2, 1]])
        else:
            assert np.array_equal(c2[t], cand[t]) and np.array_equal(cs2[t], cs[t])
    assert 0 < n_swapped < T
    # k = 1 (two columns) and a missing third candidate (E = 2): never swapped
    c1, s1 = o.topk(s[:, :2], 2)
    assert np.array_equal(o.gap_swap(c1, s1, 10.0)[0], c1)
    c3, s3 = o.topk(s[:, :2], 3)
    assert np.array_equal(o.gap_swap(c3, s3, 10.0)[0], c3)


def test_gap_swap(oracle_mod):
    check_gap_swap(oracle_mod)


def test_gate_temperature(oracle_mod):
    check_gate_temperature(oracle_mod)


def test_dispatch_invariants(oracle_mod):
    d = check_dispatch_invariants(oracle_mod)
    assert d["totals"][2] > 0 and d["totals"][1] > 0  # both re-routes and drops exercised


def test_dispatch_special_cases(oracle_mod):
    o = oracle_mod
    r = rng(5)
    T, E, k = 50, 5, 2
    s = r.standard_normal((T, E)).astype(np.float32)
    cand, cs = o.topk(s, k + 1)
    # uncapped: nothing dropped or re-routed, experts are the top-k
    d = o.dispatch(cand, cs, E, k, o.capacity(T, k, E, 0.0), 1)
    assert d["totals"][1] == 0 and d["totals"][2] == 0
    assert np.array_equal(d["eid"], cand[:, :k])
    # active fraction k/E with no cap (page figure for 64 experts)
    g = GOLD["active_fraction"]
    for kk_s, pct in g["k_to_percent"].items():
        kk = int(kk_s)
        s64 = r.standard_normal((128, g["E"])).astype(np.float32)
        c64, cs64 = o.topk(s64, kk + 1)
        d64 = o.dispatch(c64, cs64, g["E"], kk, 128, 1)
        frac = 100.0 * d64["totals"][0] / (128 * g["E"])
        assert abs(frac - pct) <= g["printed_half_ulp_percent"] + 1e-9
    # k = E: there is no fallback candidate; overflow is dropped
    cand3, cs3 = o.topk(s[:, :3], 4)
    d = o.dispatch(cand3, cs3, 3, 3, 10, 1)
    assert (d["flag"] != 1).all() and d["totals"][1] == 3 * T - 30
    # capacity 1: each expert keeps exactly its first rank-0 request
    d = o.dispatch(cand, cs, E, k, 1, 0)
    for e in range(E):
        first = [t for t in range(T) if cand[t, 0] == e]
        if first:
            assert d["eid"][first[0], 0] == e and d["pos"][first[0], 0] == 0


def check_aux_loss(o):
    g = GOLD["balance_loss_floor"]
    E, k, coef = g["E"], g["k"], g["coef"]
    T = 1024
    # perfectly balanced selections: token t picks experts t%E and (t+1)%E
    cand = np.stack([np.arange(T) % E, (np.arange(T) + 1) % E, (np.arange(T) + 2) % E], 1).astype(np.int32)
    cs = np.tile(np.array([2.0, 1.0, 0.0], np.float32), (T, 1))
    d = o.dispatch(cand, cs, E, k, o.capacity(T, k, E, 1.0), 1, coef)
    loss = float(d["aux_loss"][0])
    assert math.isclose(loss, coef * k * k / E, rel_tol=1e-6)
    assert abs(loss - g["printed"]) <= g["printed_half_ulp"]
    # the /(T*k) normalisation would miss the printed value
    assert abs(coef * (1.0 / E) - g["printed"]) > g["printed_half_ulp"]
    # all tokens on one expert: coef * k-ish closed form (expert 0 and 1 each get T)
    cand1 = np.tile(np.array([0, 1, 2], np.int32), (T, 1))
    d1 = o.dispatch(cand1, cs, E, k, T, 1, coef)
    assert math.isclose(float(d1["aux_loss"][0]), coef * 2.0, rel_tol=1e-6)


def test_aux_loss_pins(oracle_mod):
    check_aux_loss(oracle_mod)


# ----------------------------------------------------------- expert FFN --

def textbook_swiglu(x, w1, w3, w2):
    """Dense SwiGLU FFN with numpy float64 matmuls."""
    x = x.astype(np.float64)
    a = x @ w1.astype(np.float64).T
    b = x @ w3.astype(np.float64).T
    h = a / (1.0 + np.exp(-a)) * b
    return h @ w2.astype(np.float64).T, h


def check_dense_equivalence(o, dtype="f32"):
    r = rng(6)
    T, d, d_ff = 9, 24, 40
    x = r.standard_normal((T, d)).astype(np.float32)
    wr = r.standard_normal((1, d)).astype(np.float32)
    w1 = (r.standard_normal((1, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    w3 = (r.standard_normal((1, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (r.standard_normal((1, d, d_ff)) / math.sqrt(d_ff)).astype(np.float32)
    if dtype == "bf16":
        x, wr, w1, w3, w2 = (bf16_bits(a) for a in (x, wr, w1, w3, w2))
        xf, w1f, w3f, w2f = (bits_to_f32(a) for a in (x, w1, w3, w2))
    else:
        xf, w1f, w3f, w2f = x, w1, w3, w2
    out = o.forward(x, wr, None, w1, w3, w2, E=1, k=1, cf=0.0)
    ref, href = textbook_swiglu(xf, w1f[0], w3f[0], w2f[0])
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    assert (out["gate64"] == 1.0).all() and (out["eid"] == 0).all()
    y, h = o.ffn_rows(np.zeros(T, np.int32), np.arange(T, dtype=np.int32), x, w1, w3, w2, want_h=True)
    assert np.allclose(h, href, rtol=1e-12, atol=1e-12)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------- one-byte expert weights --

# Values fixed by the OCP 8-bit floating point specification for E4M3 (code:
# value); the largest finite value, the smallest normal and subnormal, one,
# a fraction step and the signed zero.
E4M3_SPEC = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}


def check_fp8_decode(o):
    """E4M3 decode against the specification's values, torch's float8_e4m3fn
    on all 256 codes (an independent implementation), the NaN codes and the
    strict order of the positive codes."""
    for code, v in E4M3_SPEC.items():
        assert o.fp8_e4m3_value(code) == v, hex(code)
    assert math.copysign(1.0, o.fp8_e4m3_value(0x80)) == -1.0 and o.fp8_e4m3_value(0x80) == 0.0
    codes = np.arange(256, dtype=np.uint8)
    got = o.fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert (np.diff(got[:0x7F]) > 0).all()
    assert np.array_equal(got[0x80:0xFF], -got[:0x7F])


def e4m3_bytes(r, shape):
    """Random E4M3 codes without the two NaN codes."""
    q = r.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((q & 0x7F) == 0x7F, q ^ 1, q).astype(np.uint8)


def check_dequant_rows(o):
    """w[r][c] = scale[r] * value(q[r][c]): against torch's float8 widening
    times the scale in float64 (exact), with rows != columns and distinct
    scales so that a transposed scale or operand fails."""
    r = rng(21)
    q = e4m3_bytes(r, (3, 5, 7))
    s = (r.random((3, 5)) * 4 + 0.01).astype(np.float32)
    w = o.dequant_rows(q, s)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(s).double()[..., None]
    assert np.array_equal(w, ref.numpy())


def check_ffn_double_elements(o):
    """The expert FFN over double elements (dequantised weights, bf16 inputs
    widened) equals the dense textbook SwiGLU in float64."""
    r = rng(22)
    T, d, d_ff = 7, 24, 40
    x = bits_to_f32(bf16_bits(r.standard_normal((T, d)).astype(np.float32))).astype(np.float64)
    w1 = o.dequant_rows(e4m3_bytes(r, (1, d_ff, d)), np.full((1, d_ff), 1 / 64, np.float32))
    w3 = o.dequant_rows(e4m3_bytes(r, (1, d_ff, d)), np.full((1, d_ff), 1 / 32, np.float32))
    w2 = o.dequant_rows(e4m3_bytes(r, (1, d, d_ff)), (r.random((1, d)) / 50).astype(np.float32))
    y, h = o.ffn_rows(np.zeros(T, np.int32), np.arange(T, dtype=np.int32), x, w1, w3, w2, want_h=True)
    ref, href = textbook_swiglu(x, w1[0], w3[0], w2[0])
    assert np.allclose(h, href, rtol=1e-12, atol=1e-12)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_fp8_decode(oracle_mod):
    check_fp8_decode(oracle_mod)


def test_dequant_rows(oracle_mod):
    check_dequant_rows(oracle_mod)


def test_ffn_double_elements(oracle_mod):
    check_ffn_double_elements(oracle_mod)


def test_dense_equivalence_f32(oracle_mod):
    check_dense_equivalence(oracle_mod, "f32")


def test_dense_equivalence_bf16(oracle_mod):
    check_dense_equivalence(oracle_mod, "bf16")


def check_identical_experts(o):
    r = rng(7)
    T, d, d_ff, E, k = 40, 16, 32, 4, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    wr = r.standard_normal((E, d)).astype(np.float32)
    one1 = r.standard_normal((d_ff, d)).astype(np.float32) / 4
    one3 = r.standard_normal((d_ff, d)).astype(np.float32) / 4
    one2 = r.standard_normal((d, d_ff)).astype(np.float32) / 6
    w1, w3, w2 = (np.ascontiguousarray(np.broadcast_to(a, (E,) + a.shape)) for a in (one1, one3, one2))
    out = o.forward(x, wr, None, w1, w3, w2, E=E, k=k, cf=0.5)  # heavy capping
    assert out["totals"][1] > 0  # some slots dropped
    ref, _ = textbook_swiglu(x, one1, one3, one2)
    has = (out["flag"] != 2).any(axis=1)
    assert has.any() and (~has).any()
    assert np.allclose(out["y"][has], ref[has], rtol=1e-10, atol=1e-12)
    assert (out["y"][~has] == 0).all()
    # the same through the per-row path and the combine step
    kept = out["flag"] != 2
    rows = out["row"][kept]
    order = np.argsort(rows)
    src = np.nonzero(kept)[0][order].astype(np.int32)
    experts = out["eid"][kept][order].astype(np.int32)
    y_rows = o.ffn_rows(experts, src, x, w1, w3, w2).astype(np.float32)
    yc = o.combine(out["row"], out["gate"], y_rows)
    assert np.allclose(yc[has], ref[has], rtol=1e-5, atol=1e-5)


def test_identical_experts(oracle_mod):
    check_identical_experts(oracle_mod)


def check_expert_relabel(o):
    """Renaming experts renames the routing and leaves the output unchanged."""
    r = rng(8)
    T, d, d_ff, E, k = 48, 16, 24, 5, 2
    x = r.standard_normal((T, d)).astype(np.float32)
    wr = r.standard_normal((E, d)).astype(np.float32)
    w1 = r.standard_normal((E, d_ff, d)).astype(np.float32) / 4
    w3 = r.standard_normal((E, d_ff, d)).astype(np.float32) / 4
    w2 = r.standard_normal((E, d, d_ff)).astype(np.float32) / 5
    base = o.forward(x, wr, None, w1, w3, w2, E=E, k=k, cf=1.0)
    perm = np.array([3, 0, 4, 1, 2])
    inv = np.argsort(perm)
    moved = o.forward(x, wr[perm], None, w1[perm], w3[perm], w2[perm], E=E, k=k, cf=1.0)
    assert base["totals"][1] + base["totals"][2] > 0  # capping is active
    assert np.array_equal(np.where(moved["eid"] >= 0, perm[np.maximum(moved["eid"], 0)], -1), base["eid"])
    assert np.array_equal(moved["kept"], base["kept"][perm])
    assert np.array_equal(inv[inv], inv[inv])  # (perm is a permutation)
    assert np.allclose(moved["y"], base["y"], rtol=1e-12, atol=1e-12)
    # and each routed expert really is applied: one token against the dense form
    t = int(np.nonzero((base["flag"] == 0).all(axis=1))[0][0])
    y = np.zeros(d)
    for j in range(k):
        e = base["eid"][t, j]
        ye, _ = textbook_swiglu(x[t:t + 1], w1[e], w3[e], w2[e])
        y += base["gate64"][t, j] * ye[0]
    assert np.allclose(base["y"][t], y, rtol=1e-12, atol=1e-12)


def test_expert_relabel(oracle_mod):
    check_expert_relabel(oracle_mod)


def test_combine_closed_form(oracle_mod):
    o = oracle_mod
    y_rows = np.arange(12, dtype=np.float32).reshape(4, 3)
    row = np.array([[2, -1], [0, 3]], np.int32)
    gate = np.array([[1.0, 0.0], [0.25, 0.75]], np.float32)
    y = o.combine(row, gate, y_rows)
    assert np.array_equal(y, np.array([[6, 7, 8], [0.25 * 0 + 0.75 * 9, 0.25 * 1 + 0.75 * 10, 0.25 * 2 + 0.75 * 11]]))


def test_example_shape(oracle_mod):
    g = GOLD["example_output_shape"]
    o = oracle_mod
    T, d = g["B"] * g["S"], 32  # hidden shrunk; the token count is the page's B*S
    r = rng(9)
    x = r.standard_normal((T, d)).astype(np.float32)
    wr = r.standard_normal((8, d)).astype(np.float32)
    w1 = r.standard_normal((8, 16, d)).astype(np.float32) / 6
    w2 = r.standard_normal((8, d, 16)).astype(np.float32) / 4
    out = o.forward(x, wr, None, w1, w1, w2, E=8, k=2, cf=1.25)
    assert out["y"].reshape(g["B"], g["S"], d).shape == (g["B"], g["S"], d)


def check_load_window(o):
    """Windowed load statistic ("企业官网建设流程全解析" page §2: selection
    frequency over a sliding window of recent tokens, 1024 on the page, with
    a decay factor 0.99), pinned by closed forms of the iterated update:
      * n windows that all repeat one selection pattern of frequency f give
        alpha^n load0 + (1 - alpha^n) f (geometric series);
      * decay 1 leaves the statistic as it was; decay 0 gives the last
        window's frequency, its selections over k x its own token count
        (a last window shorter than the others included);
      * a statistic that sums to 1 still sums to 1 (each window's
        frequencies do);
      * the page's parameters: 100 windows of 1024 tokens that all pick
        expert 0 (top-1) take a zero statistic to 1 - 0.99^100."""
    r = rng(21)
    E, k, W = 6, 2, 16
    pat = np.stack([r.permutation(E)[:k + 1] for _ in range(W)]).astype(np.int32)
    f = np.bincount(pat[:, :k].ravel(), minlength=E) / (k * W)
    load0 = (r.random(E) / E).astype(np.float32)
    for n, alpha in ((1, 0.99), (7, 0.9), (50, 0.5)):
        cand = np.tile(pat, (n, 1))
        got = o.load_window(cand, E, k, load0, W, alpha).astype(np.float64)
        want = alpha ** n * load0.astype(np.float64) + (1 - alpha ** n) * f
        assert np.allclose(got, want, rtol=1e-6, atol=1e-7), (n, alpha, got, want)
    cand = np.concatenate([np.tile(pat, (3, 1)), pat[:5]])  # three full windows and one of 5 tokens
    assert np.array_equal(o.load_window(cand, E, k, load0, W, 1.0), load0)
    last = np.bincount(pat[:5, :k].ravel(), minlength=E) / (k * 5)
    assert np.allclose(o.load_window(cand, E, k, load0, W, 0.0), last, rtol=1e-7, atol=0)
    u = np.full(E, 1.0 / E, np.float32)
    cand = np.stack([r.permutation(E)[:k + 1] for _ in range(203)]).astype(np.int32)
    assert abs(float(o.load_window(cand, E, k, u, 17, 0.8).astype(np.float64).sum()) - 1.0) < 1e-6
    # the page's window and decay: top-1, every token picks expert 0
    cand = np.zeros((100 * 1024, 2), np.int32)
    cand[:, 1] = 1
    got = o.load_window(cand, 4, 1, np.zeros(4, np.float32), 1024, 0.99)
    assert abs(float(got[0]) - (1.0 - 0.99 ** 100)) < 1e-6 and np.all(got[1:] == 0)
    # candidates that name no expert select nothing; the fallback rank is not a selection
    cand = np.array([[-1, 2, 0], [1, 7, 0]], np.int32)
    got = o.load_window(cand, 3, 2, np.zeros(3, np.float32), 8, 0.0)
    assert np.allclose(got, [0.0, 0.25, 0.25])


def test_load_window(oracle_mod):
    check_load_window(oracle_mod)


def check_dequant_rows_i8(o):
    """INT8 codes (two's complement) with fp32 row scales: every code at
    scale 1 is its integer value (numpy's own int8 conversion), and a scaled
    row is the exact product scale * code (exact in double)."""
    codes = np.arange(-128, 128, dtype=np.int8).reshape(2, 128)
    w = o.dequant_rows_i8(codes, np.ones(2, np.float32))
    assert np.array_equal(w, codes.astype(np.float64))
    s = np.array([0.0123, -3.5], np.float32)
    w = o.dequant_rows_i8(codes, s)
    assert np.array_equal(w, codes.astype(np.float64) * s.astype(np.float64)[:, None])
    assert w[0, 0] == -128 * float(s[0]) and w[1, -1] == 127 * float(s[1])


def test_dequant_rows_i8(oracle_mod):
    check_dequant_rows_i8(oracle_mod)


def check_dequant_rows_i4(o):
    """INT4 codes, two per byte: every nibble value at scale 1 is the two's
    complement integer it spells (0x0..0x7 -> 0..7, 0x8..0xF -> -8..-1,
    written out), in either half of a byte; the low nibble is the earlier
    element (a byte 0x21 holds 1 then 2); a scaled row is the exact product
    scale * code."""
    spelled = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
    # row 0: byte j = (j, 0): the low nibbles run through 0..15 (high 0);
    # row 1: byte j = (0, j): the high nibbles do
    q = np.array([[j for j in range(16)], [j << 4 for j in range(16)]], np.uint8)
    w = o.dequant_rows_i4(q, np.ones(2, np.float32))
    assert w.shape == (2, 32)
    assert w[0, 0::2].tolist() == spelled and w[0, 1::2].tolist() == [0.0] * 16
    assert w[1, 1::2].tolist() == spelled and w[1, 0::2].tolist() == [0.0] * 16
    w = o.dequant_rows_i4(np.array([[0x21, 0x8F]], np.uint8), np.ones(1, np.float32))
    assert w.tolist() == [[1.0, 2.0, -1.0, -8.0]]
    s = np.array([0.0123, -3.5], np.float32)
    w = o.dequant_rows_i4(q, s)
    assert w[0, 16] == -8 * float(s[0]) and w[1, 15] == 7 * float(s[1])
    assert np.array_equal(w[:, 0::2][0], np.array(spelled, np.float64) * float(s[0]))


def test_dequant_rows_i4(oracle_mod):
    check_dequant_rows_i4(oracle_mod)
