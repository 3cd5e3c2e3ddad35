"""Pins of the CPU oracle against things other than itself.

Each pin is a plain function so the planted-mistake test at the bottom can
run the whole set against mutated copies of the oracle: every mutant must
fail at least one pin. The pins use brute force on tiny inputs (pure-Python
loops with math.fsum), closed forms, invariants of the layer, and the
constants the page prints (tests/golden/step35_layer_constants.json).
"""
import json
import math
import os
import struct
from unittest import mock

import numpy as np
import pytest

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(v: float) -> float:
    return struct.unpack("f", struct.pack("f", v))[0]


def rand_layer(rng, T, D, E, K, F, Fs, scale_r=1.0):
    return dict(
        x=rng.standard_normal((T, D)),
        w_router=rng.standard_normal((E, D)) * scale_r,
        w_gate=rng.standard_normal((E, F, D)) / math.sqrt(D),
        w_up=rng.standard_normal((E, F, D)) / math.sqrt(D),
        w_down=rng.standard_normal((E, D, F)) / math.sqrt(F),
        s_gate=rng.standard_normal((Fs, D)) / math.sqrt(D) if Fs else None,
        s_up=rng.standard_normal((Fs, D)) / math.sqrt(D) if Fs else None,
        s_down=rng.standard_normal((D, Fs)) / math.sqrt(Fs) if Fs else None,
        bias=None,
    )


# ------------------------------------------------------------ brute force ---

def brute_route(x, wr, K, bias=None):
    """Pure-Python router: fsum logits, exp/fsum softmax, K linear max scans."""
    T, D = len(x), len(x[0])
    E = len(wr)
    idx, prob = [], []
    for t in range(T):
        l = [math.fsum(x[t][d] * wr[e][d] for d in range(D)) + (0.0 if bias is None else bias[e])
             for e in range(E)]
        m = max(l)
        w = [math.exp(v - m) for v in l]
        s = math.fsum(w)
        p = [f32(v / s) for v in w]
        taken, row_i, row_p = set(), [], []
        for _ in range(K):
            best = None
            for e in range(E):           # first maximum wins: lower index on ties
                if e not in taken and (best is None or p[e] > p[best]):
                    best = e
            taken.add(best)
            row_i.append(best)
            row_p.append(p[best])
        idx.append(row_i)
        prob.append(row_p)
    return np.array(idx), np.array(prob, dtype=np.float32)


def brute_ffn_row(xr, wg, wu, wd):
    F, D = len(wg), len(xr)
    h = []
    for f in range(F):
        g = math.fsum(wg[f][d] * xr[d] for d in range(D))
        u = math.fsum(wu[f][d] * xr[d] for d in range(D))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [math.fsum(wd[d][f] * h[f] for f in range(F)) for d in range(D)]


def brute_permute(idx, E):
    """Per expert, walk the pairs in token-major order."""
    T, K = idx.shape
    sorted_token, dest = [], [None] * (T * K)
    offsets = [0]
    for e in range(E):
        for t in range(T):
            for j in range(K):
                if idx[t, j] == e:
                    dest[t * K + j] = len(sorted_token)
                    sorted_token.append(t)
        offsets.append(len(sorted_token))
    return np.array(offsets), np.array(sorted_token), np.array(dest)


# ------------------------------------------------------------------- pins ---

def pin_route_bruteforce():
    for seed, (T, D, E, K) in enumerate([(5, 4, 7, 3), (4, 6, 9, 9), (6, 3, 5, 1), (3, 8, 16, 8)]):
        rng = np.random.default_rng(100 + seed)
        x, wr = rng.standard_normal((T, D)), rng.standard_normal((E, D))
        bias = rng.standard_normal(E) if seed % 2 else None
        r = O.route(x, wr, K, bias)
        bi, bp = brute_route(x.tolist(), wr.tolist(), K, None if bias is None else bias.tolist())
        assert np.array_equal(r["idx"], bi), (seed, r["idx"], bi)
        assert np.array_equal(r["prob"], bp), seed


def pin_route_ties():
    # experts 1 and 4 have identical router rows: equal probabilities, lower index first
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 5))
    wr = rng.standard_normal((6, 5)) * 0.1
    wr[4] = wr[1]
    wr[1] += 3.0 * np.sign(x.mean(axis=0))  # make the pair likely to be chosen
    wr[4] = wr[1]
    r = O.route(x, wr, 3)
    for t in range(6):
        row = list(r["idx"][t])
        if 1 in row and 4 in row:
            assert row.index(1) < row.index(4)
        if 4 in row:
            assert 1 in row, "index 4 chosen without its lower-index twin 1"
    # all logits equal: the first K experts, each with probability fp32(1/E)
    E, K = 10, 4
    r = O.route(np.ones((2, 3)), np.zeros((E, 3)), K)
    assert np.array_equal(r["idx"], np.tile(np.arange(K), (2, 1)))
    assert np.all(r["prob"] == np.float32(f32(1.0 / E)))
    assert np.all(r["gap"] == 0.0)


def pin_route_properties():
    rng = np.random.default_rng(3)
    x, wr = rng.standard_normal((20, 16)), rng.standard_normal((12, 16))
    r = O.route(x, wr, 5)
    assert np.allclose(r["p64"].sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(r["prob"].astype(np.float64), axis=1) <= 0)
    assert np.array_equal(r["prob"], np.take_along_axis(r["p32"], r["idx"], axis=1))
    assert np.all(r["gap"] >= 0)
    # K = E selects every expert once; gap is infinite
    r = O.route(x, wr, 12)
    assert np.array_equal(np.sort(r["idx"], axis=1), np.tile(np.arange(12), (20, 1)))
    assert np.all(np.isinf(r["gap"]))
    # huge logits stay finite (softmax is shift invariant)
    r = O.route(x * 1e3, wr, 5)
    assert np.all(np.isfinite(r["p64"])) and np.allclose(r["p64"].sum(axis=1), 1.0)


def pin_route_bias():
    rng = np.random.default_rng(5)
    x, wr = rng.standard_normal((30, 8)), rng.standard_normal((10, 8)) * 0.3
    b = rng.standard_normal(10)
    r0, r1 = O.route(x, wr, 4, b), O.route(x, wr, 4, b + 2.5)   # shift: same routing
    assert np.array_equal(r0["idx"], r1["idx"])
    big = np.zeros(10)
    big[6] = 60.0                                               # expert 6 always first
    r = O.route(x, wr, 4, big)
    assert np.all(r["idx"][:, 0] == 6) and np.all(r["prob"][:, 0] > 0.999)


def pin_permute():
    rng = np.random.default_rng(11)
    for T, E, K in [(9, 5, 2), (13, 7, 3), (4, 6, 6), (1, 3, 1), (17, 12, 4)]:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        p = O.permute(idx, E)
        off, st, de = brute_permute(idx, E)
        assert np.array_equal(p["offsets"], off)
        assert np.array_equal(p["sorted_token"], st)
        assert np.array_equal(p["dest"], de)
        assert p["counts"].sum() == T * K and p["offsets"][-1] == T * K
        assert np.array_equal(np.sort(p["dest"]), np.arange(T * K))      # bijection
        for e in range(E):
            seg = p["sorted_token"][p["offsets"][e]:p["offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)                               # token order
        # unpermute(permute(rows)) is the identity
        rows = rng.standard_normal((T, 3))
        perm = rows[p["sorted_token"]]
        back = perm[p["dest"]].reshape(T, K, 3)
        assert np.array_equal(back, np.repeat(rows[:, None], K, axis=1))


def pin_ffn_closed_form():
    # one input, one hidden unit: y = w_d * silu(w_g x) * (w_u x)
    y = O.swiglu_ffn(np.array([[2.0]]), np.array([[0.5]]), np.array([[3.0]]), np.array([[-1.0]]))
    silu1 = 1.0 / (1.0 + math.exp(-1.0))
    assert math.isclose(y[0, 0], -6.0 * silu1, rel_tol=1e-15)
    # gate weights zero: silu(0) = 0 -> output zero
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 4))
    z = O.swiglu_ffn(x, np.zeros((5, 4)), rng.standard_normal((5, 4)), rng.standard_normal((4, 5)))
    assert np.all(z == 0)
    # strongly positive gate: silu(g) = g to double precision, the FFN is W_d((W_g x)*(W_u x))
    wg = np.abs(rng.standard_normal((5, 4))) + 50.0
    xp = np.abs(x) + 1.0
    wu, wd = rng.standard_normal((5, 4)), rng.standard_normal((4, 5))
    lin = ((xp @ wg.T) * (xp @ wu.T)) @ wd.T
    assert np.allclose(O.swiglu_ffn(xp, wg, wu, wd), lin, rtol=1e-13, atol=0)


def pin_ffn_bruteforce():
    rng = np.random.default_rng(9)
    D, F = 5, 3
    x = rng.standard_normal((4, D))
    wg, wu, wd = rng.standard_normal((F, D)), rng.standard_normal((F, D)), rng.standard_normal((D, F))
    y = O.swiglu_ffn(x, wg, wu, wd)
    for t in range(4):
        ref = brute_ffn_row(x[t].tolist(), wg.tolist(), wu.tolist(), wd.tolist())
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-14)
    # grouped: segment e uses expert e's weights
    E = 3
    W = [(rng.standard_normal((F, D)), rng.standard_normal((F, D)), rng.standard_normal((D, F)))
         for _ in range(E)]
    offsets = [0, 2, 2, 5]
    xr = rng.standard_normal((5, D))
    y = O.grouped_ffn(xr, offsets, lambda e: W[e])
    for r, e in [(0, 0), (1, 0), (2, 2), (3, 2), (4, 2)]:
        ref = brute_ffn_row(xr[r].tolist(), *(w.tolist() for w in W[e]))
        assert np.allclose(y[r], ref, rtol=1e-12, atol=1e-14)


def pin_layer_worked_example():
    """D=2, E=3, K=2, F=Fs=1, one token x=(1,0); every number by hand.

    logits (0, ln 2, ln 3) -> p = (1/6, 1/3, 1/2) -> top-2 = (2, 1).
    expert 1: g=1, u=2 -> h = 2 silu(1); y1 = (h, -h)
    expert 2: g=-1, u=1 -> h = silu(-1); y2 = (2h, h/2)
    shared: g=2, u=1 -> h = silu(2); ys = (h, h)
    out = ys + f32(1/2) y2 + f32(1/3) y1
    """
    x = np.array([[1.0, 0.0]])
    wr = np.array([[0.0, 0.0], [math.log(2.0), 0.0], [math.log(3.0), 0.0]])
    wg = np.array([[[0.0, 0.0]], [[1.0, 0.0]], [[-1.0, 0.0]]])
    wu = np.array([[[0.0, 0.0]], [[2.0, 0.0]], [[1.0, 0.0]]])
    wd = np.array([[[0.0], [0.0]], [[1.0], [-1.0]], [[2.0], [0.5]]])
    L = dict(x=x, w_router=wr, w_gate=wg, w_up=wu, w_down=wd,
             s_gate=np.array([[2.0, 0.0]]), s_up=np.array([[1.0, 0.0]]),
             s_down=np.array([[1.0], [1.0]]), bias=None)
    r = O.layer_forward(x, O.LayerWeights.from_dict(L), 2)
    assert list(r["idx"][0]) == [2, 1]
    assert r["prob"][0, 0] == np.float32(0.5) and r["prob"][0, 1] == np.float32(f32(1 / 3))
    s = lambda g: g / (1.0 + math.exp(-g))
    p1, p2 = f32(1 / 3), 0.5
    want = [s(2.0) + p2 * 2 * s(-1.0) + p1 * 2 * s(1.0),
            s(2.0) + p2 * 0.5 * s(-1.0) - p1 * 2 * s(1.0)]
    assert np.allclose(r["out"][0], want, rtol=1e-12, atol=1e-15)


def pin_layer_special_cases():
    rng = np.random.default_rng(21)
    T, D, E, K, F = 12, 6, 5, 2, 4
    L = rand_layer(rng, T, D, E, K, F, F)
    W = O.LayerWeights.from_dict(L)
    base = O.layer_forward(L["x"], W, K)
    ys = O.swiglu_ffn(L["x"], L["s_gate"], L["s_up"], L["s_down"])
    # routed experts silenced: output is the shared expert alone
    Lz = dict(L, w_down=np.zeros_like(L["w_down"]))
    assert np.array_equal(O.layer_forward(L["x"], O.LayerWeights.from_dict(Lz), K)["out"], ys)
    # all experts identical: out = ys + (sum_k prob) FFN(x)
    Li = dict(L, w_gate=np.repeat(L["w_gate"][:1], E, 0), w_up=np.repeat(L["w_up"][:1], E, 0),
              w_down=np.repeat(L["w_down"][:1], E, 0))
    ri = O.layer_forward(L["x"], O.LayerWeights.from_dict(Li), K)
    f0 = O.swiglu_ffn(L["x"], L["w_gate"][0], L["w_up"][0], L["w_down"][0])
    want = ys + ri["prob"].astype(np.float64).sum(axis=1, keepdims=True) * f0
    assert np.allclose(ri["out"], want, rtol=1e-12, atol=1e-13)
    # K = E: the dense mixture sum_e p32_e FFN_e(x) + ys, no permutation involved
    rd = O.layer_forward(L["x"], W, E)
    dense = ys.copy()
    for e in range(E):
        dense += rd["p32"][:, e:e + 1].astype(np.float64) * O.swiglu_ffn(
            L["x"], L["w_gate"][e], L["w_up"][e], L["w_down"][e])
    assert np.allclose(rd["out"], dense, rtol=1e-12, atol=1e-13)
    # permuting tokens permutes output rows
    perm = rng.permutation(T)
    rp = O.layer_forward(L["x"][perm], W, K)
    assert np.allclose(rp["out"], base["out"][perm], rtol=1e-12, atol=1e-13)
    # relabelling experts (router rows move with their weights) leaves the output unchanged
    q = rng.permutation(E)
    Lq = dict(L, w_router=L["w_router"][q], w_gate=L["w_gate"][q], w_up=L["w_up"][q],
              w_down=L["w_down"][q])
    rq = O.layer_forward(L["x"], O.LayerWeights.from_dict(Lq), K)
    assert np.allclose(rq["out"], base["out"], rtol=1e-12, atol=1e-13)
    # sampled rows agree with the full layer
    rr = O.layer_rows(L["x"], W, K, [0, 5, 11])
    assert np.allclose(rr["out_rows"], base["out"][[0, 5, 11]], rtol=1e-12, atol=1e-13)


def pin_dynamic_topk_route():
    """R12 by brute force: token t's first k_t choices are the brute-force top-k_t, then -1 / 0."""
    for seed, (T, D, E, K) in enumerate([(7, 4, 9, 4), (5, 6, 6, 6), (6, 3, 12, 8)]):
        rng = np.random.default_rng(300 + seed)
        x, wr = rng.standard_normal((T, D)), rng.standard_normal((E, D))
        kt = rng.integers(-1, K + 2, size=T)           # out-of-range values are clamped
        kt[0], kt[-1] = 0, K
        r = O.route(x, wr, K, None, kt)
        for t in range(T):
            n = min(max(int(kt[t]), 0), K)
            bi, bp = brute_route([x[t].tolist()], wr.tolist(), n) if n else (np.zeros((1, 0)), np.zeros((1, 0)))
            assert np.array_equal(r["idx"][t, :n], bi[0]), (seed, t)
            assert np.array_equal(r["prob"][t, :n], bp[0].astype(np.float32)), (seed, t)
            assert np.all(r["idx"][t, n:] == -1) and np.all(r["prob"][t, n:] == 0), (seed, t)
            if n == 0 or n == E:
                assert np.isinf(r["gap"][t])
            else:
                _, b_next = brute_route([x[t].tolist()], wr.tolist(), n + 1)
                assert r["gap"][t] == float(bp[0][-1]) - float(b_next[0][-1])


def pin_dynamic_topk_permute():
    """Pairs without an expert get no row: brute-force per-expert walk, dest -1."""
    rng = np.random.default_rng(41)
    for T, E, K in [(9, 5, 3), (13, 7, 4), (6, 4, 4)]:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        kt = rng.integers(0, K + 1, size=T)
        for t in range(T):
            idx[t, kt[t]:] = -1
        p = O.permute(idx, E)
        off, st, de = brute_permute(idx, E)
        valid = idx.reshape(-1) >= 0
        assert np.array_equal(p["offsets"], off) and np.array_equal(p["sorted_token"], st)
        assert np.all(p["dest"][~valid] == -1)
        assert np.array_equal(p["dest"][valid], np.array([d for d in de if d is not None]))
        assert p["offsets"][-1] == kt.sum() == valid.sum()
        assert np.array_equal(np.sort(p["dest"][valid]), np.arange(valid.sum()))


def pin_dynamic_topk_layer():
    rng = np.random.default_rng(23)
    T, D, E, K, F = 14, 6, 7, 4, 3
    L = rand_layer(rng, T, D, E, K, F, F)
    W = O.LayerWeights.from_dict(L)
    ys = O.swiglu_ffn(L["x"], L["s_gate"], L["s_up"], L["s_down"])
    # no routed experts at all: the shared expert alone, exactly
    r0 = O.layer_forward(L["x"], W, K, np.zeros(T, dtype=np.int64))
    assert np.array_equal(r0["out"], ys)
    # a token with k_t experts gets the same output as the fixed top-k_t layer
    kt = np.array([2, K] * (T // 2))
    rd = O.layer_forward(L["x"], W, K, kt)
    r2, rk = O.layer_forward(L["x"], W, 2), O.layer_forward(L["x"], W, K)
    assert np.allclose(rd["out"][kt == 2], r2["out"][kt == 2], rtol=1e-12, atol=1e-13)
    assert np.allclose(rd["out"][kt == K], rk["out"][kt == K], rtol=1e-12, atol=1e-13)
    # all experts identical: out = ys + (sum of the token's k_t probabilities) FFN(x)
    Li = dict(L, w_gate=np.repeat(L["w_gate"][:1], E, 0), w_up=np.repeat(L["w_up"][:1], E, 0),
              w_down=np.repeat(L["w_down"][:1], E, 0))
    kt = rng.integers(0, K + 1, size=T)
    ri = O.layer_forward(L["x"], O.LayerWeights.from_dict(Li), K, kt)
    f0 = O.swiglu_ffn(L["x"], L["w_gate"][0], L["w_up"][0], L["w_down"][0])
    psum = np.array([math.fsum(float(v) for v in ri["p32"][t][np.argsort(-ri["p32"][t], kind="stable")[:kt[t]]])
                     for t in range(T)])
    assert np.allclose(ri["out"], ys + psum[:, None] * f0, rtol=1e-12, atol=1e-13)
    # sampled rows agree with the full layer
    rr = O.layer_rows(L["x"], W, K, [1, 6, 13], kt)
    rf = O.layer_forward(L["x"], W, K, kt)
    assert np.allclose(rr["out_rows"], rf["out"][[1, 6, 13]], rtol=1e-12, atol=1e-13)


def pin_ep_receive_plan():
    """Hand-worked receive plan, then invariants on random counts."""
    # chunks r-major: (0,0) rows 0,1; (0,1) none; (0,2) row 2; (1,0) row 3; (1,1) rows 4,5,6; (1,2) none
    p = O.ep_receive_plan([[2, 0, 1], [1, 3, 0]])
    assert p["gather"].tolist() == [0, 1, 3, 4, 5, 6, 2]
    assert p["offsets"].tolist() == [0, 3, 6, 7]
    assert p["scatter"].tolist() == [0, 1, 6, 2, 3, 4, 5]
    rng = np.random.default_rng(8)
    for R, El in [(8, 36), (3, 5), (1, 4), (6, 1)]:
        c = rng.integers(0, 7, size=(R, El)) * (rng.random((R, El)) > 0.2)
        p = O.ep_receive_plan(c)
        n = int(c.sum())
        assert np.array_equal(np.sort(p["gather"]), np.arange(n))             # a permutation of the rows
        assert np.array_equal(p["scatter"][p["gather"]], np.arange(n))
        assert np.array_equal(np.diff(p["offsets"]), c.sum(axis=0))           # segment = the expert's rows
        # inside an expert, sources in turn: receive rows increase
        for e in range(El):
            seg = p["gather"][p["offsets"][e]:p["offsets"][e + 1]]
            assert np.all(np.diff(seg) > 0)


def pin_group_stats():
    """Balance statistics: closed forms (uniform router, balanced routing) and brute force."""
    G, E, T = 4, 12, 6
    # all logits equal: every group holds mass 1/G; top-2 takes experts 0 and 1 (group 0)
    r = O.route(np.ones((T, 3)), np.zeros((E, 3)), 2)
    st = O.group_stats(r["p64"], r["idx"], G)
    assert np.allclose(st["p"], 1.0 / G, rtol=0, atol=1e-15)
    assert st["pairs"].tolist() == [2 * T, 0, 0, 0] and st["f"].tolist() == [1.0, 0, 0, 0]
    assert math.isclose(st["l_ep"], G * 1.0 * (1.0 / G), rel_tol=1e-14)
    # perfectly balanced: uniform p and one pair per group per token -> L_EP = 1
    idx = np.array([[g * (E // G) for g in range(G)]] * T)
    st = O.group_stats(np.full((T, E), 1.0 / E), idx, G)
    assert math.isclose(st["l_ep"], 1.0, rel_tol=1e-14)
    # brute force on random probabilities and choices (with empty slots)
    rng = np.random.default_rng(12)
    p = rng.random((T, E))
    p /= p.sum(axis=1, keepdims=True)
    idx = np.stack([rng.permutation(E)[:3] for _ in range(T)])
    idx[1, 2] = -1
    st = O.group_stats(p, idx, G)
    for g in range(G):
        m = math.fsum(p[t][e] for t in range(T) for e in range(E) if e // (E // G) == g)
        n = sum(1 for t in range(T) for j in range(3) if idx[t][j] >= 0 and idx[t][j] // (E // G) == g)
        assert math.isclose(st["mass"][g], m, rel_tol=1e-14) and st["pairs"][g] == n
    assert math.isclose(st["f"].sum(), 1.0, rel_tol=1e-14) and math.isclose(st["p"].sum(), 1.0, rel_tol=1e-14)


def pin_ep_share_composition():
    """Per-source permutes, the receive plan and a grouped FFN give each received row its expert's FFN."""
    rng = np.random.default_rng(31)
    R, Tl, D, E, K, F, G = 3, 5, 4, 8, 2, 3, 2
    El = E // G
    L = rand_layer(rng, R * Tl, D, E, K, F, 0)
    W = O.LayerWeights.from_dict(L)
    for g in range(G):
        chunks, counts, want = [], np.zeros((R, El), dtype=np.int64), []
        for r in range(R):
            xs = L["x"][r * Tl:(r + 1) * Tl]
            rt = O.route(xs, L["w_router"], K)
            pm = O.permute(rt["idx"], E)
            for e in range(El):
                a, b = pm["offsets"][g * El + e], pm["offsets"][g * El + e + 1]
                counts[r, e] = b - a
                chunks.append(xs[pm["sorted_token"][a:b]])
                want.extend(O.swiglu_ffn(xs[t:t + 1], *W.expert(g * El + e))[0] for t in pm["sorted_token"][a:b])
        recv = np.concatenate(chunks) if chunks else np.zeros((0, D))
        plan = O.ep_receive_plan(counts)
        y_em = O.grouped_ffn(recv[plan["gather"]], plan["offsets"], lambda e: W.expert(g * El + e))
        y_recv = y_em[plan["scatter"]]
        assert np.allclose(y_recv, np.array(want).reshape(-1, D), rtol=1e-12, atol=1e-14)


def pin_fp8_codec():
    """OCP E4M3 values the format fixes, rounding ties to even, saturation, subnormals, round trip."""
    d = O.e4m3_decode
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0xB8) == -1.0 and d(0x40) == 2.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0 and np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x00) == 0.0
    assert d(0x30) == 0.5 and d(0x37) == 0.9375 and d(0x77) == 240.0
    pos = d(np.arange(127))
    assert np.all(np.diff(pos) > 0)                                       # codes 0..126 increase
    enc = lambda *v: O.e4m3_encode(np.float32(v)).tolist()
    assert enc(1.0625, 1.1875, 0.96875) == [0x38, 0x3A, 0x38]             # ties go to the even code
    assert enc(1.06, 1.07) == [0x38, 0x39]                                # otherwise the nearest
    assert enc(449.0, 464.0, 1e30, -3e5) == [0x7E, 0x7E, 0x7E, 0xFE]      # saturation, no NaN
    assert enc(1.5 * 2 ** -9, 2.5 * 2 ** -9, 2 ** -11, 7.5 * 2 ** -9) == [0x02, 0x02, 0x00, 0x08]
    assert enc(0.0, -0.0) == [0x00, 0x80]
    c = np.arange(256)
    fin = ~np.isnan(d(c))
    assert np.array_equal(O.e4m3_encode(d(c)[fin].astype(np.float32)), c[fin].astype(np.uint8))
    # against the decoded set by brute force: the nearest value, ties to the even code
    rng = np.random.default_rng(17)
    v = np.float32(rng.standard_normal(300) * np.exp(rng.uniform(-9, 6, 300)))
    q = O.e4m3_encode(v)
    for x, code in zip(v.tolist(), q.tolist()):
        a = min(abs(x), 448.0)
        best = min(range(127), key=lambda k: (abs(float(pos[k]) - a), k % 2))
        assert code & 0x7F == best and (code >> 7) == (1 if math.copysign(1, x) < 0 else 0)


def pin_fp8_quantisation():
    """Per-row scales: the largest magnitude of each row lands on 448; zero rows keep scale 1."""
    rng = np.random.default_rng(19)
    w = rng.standard_normal((2, 6, 64)).astype(np.float32) * np.float32(rng.uniform(0.01, 3, (2, 6, 1)))
    w[1, 2] = 0.0
    q, s = O.quantize_rows_fp8(w)
    assert q.dtype == np.uint8 and s.dtype == np.float32 and q.shape == w.shape and s.shape == (2, 6)
    amax = np.abs(w).max(axis=-1)
    assert s[1, 2] == 1.0 and np.all(q[1, 2] == 0)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    assert np.all(np.abs(O.e4m3_decode(q)).max(axis=-1)[nz] == 448.0)
    # the dequantised weights stay within half a step of E4M3 (relative 2^-4) plus the subnormal step
    wd = O.dequantize_fp8(q, s)
    step = np.maximum(np.abs(w.astype(np.float64)) * 2.0 ** -4, s[..., None] * 2.0 ** -10)
    assert np.all(np.abs(wd - w) <= step + 1e-30)


def pin_rows_output():
    """Output rows for a given routing (any expert ids, empty slots, repeats): pure-Python brute force."""
    rng = np.random.default_rng(47)
    T, D, E, K, F = 6, 5, 7, 3, 4
    L = rand_layer(rng, T, D, E, K, F, 3)
    W = O.LayerWeights.from_dict(L)
    rows = [4, 1, 5]
    idx = np.array([[2, 6, -1], [6, 6, 0], [-1, -1, -1]])   # not a top-k routing: the oracle takes it as given
    prob = np.array([[0.5, 0.25, 0.9], [0.125, 0.375, 1.0], [0.3, 0.3, 0.3]])
    got = O.rows_output(L["x"], W, rows, idx, prob)
    for i, t in enumerate(rows):
        xr = L["x"][t].tolist()
        want = brute_ffn_row(xr, L["s_gate"].tolist(), L["s_up"].tolist(), L["s_down"].tolist())
        for j in range(K):
            e = int(idx[i, j])
            if e >= 0:
                y = brute_ffn_row(xr, L["w_gate"][e].tolist(), L["w_up"][e].tolist(), L["w_down"][e].tolist())
                want = [a + prob[i, j] * b for a, b in zip(want, y)]
        assert np.allclose(got[i], want, rtol=1e-12, atol=1e-13), (i, got[i], want)
    # with the oracle's own top-k routing it is the full layer's rows
    full = O.layer_forward(L["x"], W, K)
    sel = [0, 3, 5]
    assert np.allclose(O.rows_output(L["x"], W, sel, full["idx"][sel], full["prob"][sel]), full["out"][sel],
                       rtol=1e-12, atol=1e-13)


def pin_expert_load():
    """Expert Activation Skew = max count / mean count over all experts: hand-worked values,
    closed forms, invariances, and the counts of a routing whose choices are forced."""
    r = O.expert_load(np.array([0, 0, 4, 2]))
    # worked by hand: max 4, mean (0+0+4+2)/4 = 1.5, skew 4/1.5 = 8/3, two experts touched
    assert r["max"] == 4.0 and r["mean"] == 1.5 and r["touched"] == 2
    assert math.isclose(r["skew"], 8.0 / 3.0, rel_tol=1e-15)
    # closed forms: uniform counts give 1; every pair on one of E experts gives E
    assert O.expert_load(np.full(288, 57))["skew"] == 1.0
    one = np.zeros(288, dtype=np.int64)
    one[17] = 8192 * 8
    assert math.isclose(O.expert_load(one)["skew"], 288.0, rel_tol=1e-15)
    assert O.expert_load(one)["touched"] == 1
    assert O.expert_load(np.zeros(5, dtype=np.int64))["skew"] == 0.0
    # invariances: relabelling experts and scaling all counts leave the skew unchanged
    rng = np.random.default_rng(41)
    c = rng.integers(0, 50, 36)
    c[3] = 0
    s0 = O.expert_load(c)["skew"]
    assert math.isclose(O.expert_load(rng.permutation(c))["skew"], s0, rel_tol=1e-14)
    assert math.isclose(O.expert_load(7 * c)["skew"], s0, rel_tol=1e-14)
    # brute force: pure-Python max and mean over all experts
    assert math.isclose(s0, max(c.tolist()) / (math.fsum(c.tolist()) / len(c)), rel_tol=1e-14)
    # a routing with forced choices: all logits equal, so every token takes experts 0..K-1
    # (ties to the lower index): K experts hold T pairs each, the other E-K none, skew = E/K
    T, E, K = 10, 12, 3
    rt = O.route(np.ones((T, 2)), np.zeros((E, 2)), K)
    ld = O.expert_load(O.permute(rt["idx"], E)["counts"])
    assert ld["max"] == T and ld["touched"] == K and math.isclose(ld["skew"], E / K, rel_tol=1e-15)


def pin_group_counts():
    """Per-group counts of G contiguous equal expert groups: hand-worked, brute force, the page's 8 x 36."""
    assert O.group_counts(np.arange(12), 3).tolist() == [0 + 1 + 2 + 3, 4 + 5 + 6 + 7, 8 + 9 + 10 + 11]
    assert O.group_counts(np.arange(12), 1).tolist() == [66]
    assert O.group_counts(np.arange(12), 12).tolist() == list(range(12))
    g = json.load(open(os.path.join(GOLDEN, "step35_layer_constants.json")))["values"]
    G, per = g["ep_groups"]["value"], g["experts_per_group"]["value"]
    E = G * per
    rng = np.random.default_rng(43)
    c = rng.integers(0, 400, E)
    got = O.group_counts(c, G)
    want = [0] * G
    for e in range(E):          # brute force: walk the experts, group e // (E / G)
        want[e // per] += int(c[e])
    assert got.tolist() == want and int(got.sum()) == int(c.sum())
    # one hot expert lands in its own group only
    hot = np.zeros(E, dtype=np.int64)
    hot[per + 5] = 9
    assert O.group_counts(hot, G).tolist() == [0, 9] + [0] * (G - 2)
    with pytest.raises(ValueError):
        O.group_counts(np.arange(10), 3)


def pin_page_constants():
    """The page's structural numbers, and the width reading they force."""
    g = json.load(open(os.path.join(GOLDEN, "step35_layer_constants.json")))["values"]
    v = {k: d["value"] for k, d in g.items()}
    import synth
    for name in ("decode", "prefill", "skew", "full"):
        s = synth.spec(name)
        assert (s.E, s.K, s.D) == (v["routed_experts_per_layer"], v["top_k"], v["d_model"])
        assert s.Fs > 0 and v["shared_experts_per_layer"] == 1
    assert v["top_k"] + v["shared_experts_per_layer"] == v["experts_run_per_token"]
    assert round(100 * v["top_k"] / v["routed_experts_per_layer"], 2) == v["routed_fraction_percent"]
    assert v["ep_groups"] * v["experts_per_group"] == v["routed_experts_per_layer"]
    # expert width: 1280 fits the 196.81B / 11B totals; the literal 4096 cannot
    D, E, L = v["d_model"], v["routed_experts_per_layer"], v["moe_layers"]
    moe = lambda F: L * ((E + 1) * 3 * D * F + E * D) / 1e9
    act = lambda F: L * 9 * 3 * D * F / 1e9
    assert moe(1280) < v["total_params_billion"] < moe(1280) + 10
    assert act(1280) < v["active_params_billion"]
    assert moe(4096) > 3 * v["total_params_billion"]
    assert synth.spec("prefill").F == 1280


PINS = [pin_route_bruteforce, pin_route_ties, pin_route_properties, pin_route_bias, pin_permute,
        pin_ffn_closed_form, pin_ffn_bruteforce, pin_layer_worked_example,
        pin_layer_special_cases, pin_dynamic_topk_route, pin_dynamic_topk_permute, pin_dynamic_topk_layer,
        pin_ep_receive_plan, pin_group_stats, pin_ep_share_composition, pin_fp8_codec, pin_fp8_quantisation,
        pin_rows_output, pin_expert_load, pin_group_counts, pin_page_constants]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------- planted mistakes ---

def _renormalised(p32, k, k_per_token=None):
    idx, prob, gap = (_orig["select_topk"](p32, k) if k_per_token is None else
                      _orig["select_topk"](p32, k, k_per_token))
    tot = prob.sum(axis=1, keepdims=True)
    return idx, np.where(tot > 0, prob / np.where(tot > 0, tot, 1), 0).astype(np.float32), gap


def _ties_high(p32, k, k_per_token=None):
    E = p32.shape[1]
    order = E - 1 - np.argsort(-p32[:, ::-1], axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    prob = np.take_along_axis(p32, order[:, :k], axis=1).astype(np.float32)
    return idx, prob, np.zeros(p32.shape[0])


def _softmax_after_topk(x, w_router, k, bias=None, k_per_token=None):
    l = O.router_logits(x, w_router, bias)
    order = np.argsort(-l, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(l, order, axis=1)
    p = O.softmax(top).astype(np.float32)
    p32 = O.softmax(l).astype(np.float32)
    return dict(logits=l, p64=O.softmax(l), p32=p32, idx=order.astype(np.int32), prob=p,
                gap=np.ones(len(l)))


def _no_max_sub(logits):
    w = np.exp(logits)
    return w / w.sum(axis=1, keepdims=True)


def _swapped_gate_up(x_rows, w_gate, w_up, w_down):
    return _orig["swiglu_ffn"](x_rows, w_up, w_gate, w_down)


def _sigmoid_not_silu(g):
    return 1.0 / (1.0 + np.exp(-g))


def _unstable_permute(idx, n_experts):
    p = _orig["permute"](idx, n_experts)
    st, de = p["sorted_token"].copy(), p["dest"].copy()
    off = p["offsets"]
    for e in range(n_experts):                  # reverse token order inside each segment
        a, b = off[e], off[e + 1]
        st[a:b] = st[a:b][::-1]
    inv = np.empty_like(de)
    for r in range(len(de)):
        inv[de[r]] = r
    T, k = idx.shape
    pos = {}
    for r, t in enumerate(st):
        pos.setdefault(int(t), []).append(r)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if e < 0:
                continue
            rows = [r for r in pos[t] if off[e] <= r < off[e + 1]]
            de[t * k + j] = rows[0]
    return dict(p, sorted_token=st, dest=de)


def _inclusive_offsets(idx, n_experts):
    p = _orig["permute"](idx, n_experts)
    return dict(p, offsets=np.concatenate([np.cumsum(p["counts"]), [idx.size]]))


def _kmajor_dest(ys, y_perm, dest, prob):
    T, k = np.asarray(prob).shape
    return _orig["combine"](ys, y_perm, np.asarray(dest).reshape(k, T).T.reshape(-1), prob)


def _drop_shared(ys, y_perm, dest, prob):
    return _orig["combine"](None, y_perm, dest, prob)


def _drop_bias(x, w_router, bias=None):
    return _orig["router_logits"](x, w_router, None)


def _transposed_down(x_rows, w_gate, w_up, w_down):
    g = O.as_f64(x_rows) @ O.as_f64(w_gate).T
    u = O.as_f64(x_rows) @ O.as_f64(w_up).T
    h = O.silu(g) * u
    wd = O.as_f64(w_down)
    if wd.shape[0] == wd.shape[1]:
        return h @ wd
    return h @ wd.reshape(wd.shape[1], wd.shape[0])   # plausible reshape-for-transpose slip


def _dynamic_k_ignored(p32, k, k_per_token=None):
    return _orig["select_topk"](p32, k)


def _dropped_slot_kept(p32, k, k_per_token=None):
    if k_per_token is None:
        return _orig["select_topk"](p32, k)
    idx, prob, gap = _orig["select_topk"](p32, k, k_per_token)
    full, _, _ = _orig["select_topk"](p32, k)
    return np.where(idx < 0, full, idx).astype(np.int32), prob, gap   # expert kept, weight 0


def _no_expert_as_expert0(idx, n_experts):
    return _orig["permute"](np.where(np.asarray(idx) < 0, 0, idx), n_experts)


def _plan_source_major(counts):
    c = np.maximum(np.asarray(counts, dtype=np.int64), 0)
    p = _orig["ep_receive_plan"](c)
    g = np.arange(int(c.sum()))                                  # rows left in receive order
    s = np.empty_like(g)
    s[g] = np.arange(len(g))
    return dict(p, gather=g, scatter=s)


def _stats_from_chosen_only(p64, idx, n_groups):
    p64 = np.asarray(p64, dtype=np.float64)
    kept = np.zeros_like(p64)
    ii = np.asarray(idx)
    for t in range(ii.shape[0]):
        for e in ii[t]:
            if e >= 0:
                kept[t, e] = p64[t, e]
    return _orig["group_stats"](kept, idx, n_groups)


def _encode_truncating(v):
    v = np.asarray(v, dtype=np.float32)
    pos = O.e4m3_decode(np.arange(127))
    a = np.minimum(np.abs(v.astype(np.float64)), 448.0)
    code = np.clip(np.searchsorted(pos, a, side="right") - 1, 0, 126)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _scale_by_max(w):
    q, s = _orig["quantize_rows_fp8"](w)
    w32 = O.as_f64(w).astype(np.float32)
    amax = np.abs(w32).max(axis=-1)
    s2 = np.where(amax > 0, amax, np.float32(1)).astype(np.float32)
    return O.e4m3_encode((w32 / s2[..., None]).astype(np.float32)), s2


def _skew_mean_over_touched(counts):
    c = np.asarray(counts, dtype=np.float64)
    t = c[c > 0]
    mean = t.mean() if t.size else 0.0
    return dict(max=float(c.max()) if c.size else 0.0, mean=float(mean),
                skew=float(c.max() / mean) if mean > 0 else 0.0, touched=int(t.size))


def _rows_output_slots_reversed(x, W, rows, idx_rows, prob_rows):
    return _orig["rows_output"](x, W, rows, idx_rows, np.asarray(prob_rows)[:, ::-1])


def _strided_groups(counts, groups):
    c = np.asarray(counts)
    return np.array([int(c[g::groups].sum()) for g in range(groups)])


_orig = {n: getattr(O, n) for n in ("rows_output", "quantize_rows_fp8", "ep_receive_plan", "group_stats", "select_topk", "swiglu_ffn", "permute", "combine",
                                    "router_logits", "softmax", "silu", "route")}

MUTANTS = {
    "renormalised_topk": ("select_topk", _renormalised),
    "ties_to_higher_index": ("select_topk", _ties_high),
    "softmax_after_selection": ("route", _softmax_after_topk),
    "softmax_without_max_subtraction": ("softmax", _no_max_sub),
    "gate_up_swapped": ("swiglu_ffn", _swapped_gate_up),
    "sigmoid_instead_of_silu": ("silu", _sigmoid_not_silu),
    "unstable_permute": ("permute", _unstable_permute),
    "inclusive_offsets": ("permute", _inclusive_offsets),
    "choice_major_dest": ("combine", _kmajor_dest),
    "shared_expert_dropped": ("combine", _drop_shared),
    "router_bias_dropped": ("router_logits", _drop_bias),
    "down_projection_transposed": ("swiglu_ffn", _transposed_down),
    "dynamic_k_ignored": ("select_topk", _dynamic_k_ignored),
    "dropped_slot_keeps_expert": ("select_topk", _dropped_slot_kept),
    "no_expert_routed_to_expert_0": ("permute", _no_expert_as_expert0),
    "receive_plan_left_source_major": ("ep_receive_plan", _plan_source_major),
    "group_mass_of_chosen_experts_only": ("group_stats", _stats_from_chosen_only),
    "fp8_encode_truncates": ("e4m3_encode", _encode_truncating),
    "fp8_scale_without_448": ("quantize_rows_fp8", _scale_by_max),
    "skew_mean_over_touched_experts": ("expert_load", _skew_mean_over_touched),
    "expert_groups_strided": ("group_counts", _strided_groups),
    "row_weights_in_reversed_slots": ("rows_output", _rows_output_slots_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    attr, fn = MUTANTS[name]
    failed = []
    with mock.patch.object(O, attr, fn), np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except AssertionError:     # a crash does not count: the pin must notice
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
