"""One GPU's expert-parallel share on the GPU against the oracle (reading R13).

A share is built the way the dispatch exchange would deliver it: every source
rank routes and permutes its own tokens (moe_route, moe_permute with the row
gather), and the slice of its permuted rows that belongs to the share's expert
group is its chunk; the receive buffer is the chunks of all sources in rank
order, with the [source][local expert] count matrix beside it. The share then
runs moe_ep_receive_plan, the two expert GEMM halves on the receive buffer in
place (the plan's gather as their row map) and moe_gather_rows with the plan's
scatter, which leaves every received row's expert output in receive order.
Checked: the plan bit for bit, every sampled received row against its
expert's FFN on its token, and the balance statistics of moe_route_group_stats.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from moe_testutil import compare_out, compare_routing, device_layer, oracle_weights, to_host
from oracle import moe_oracle as O
from test_gpu_parity import sample_rows

pytestmark = pytest.mark.gpu


def build_share(spec, L, n_src, group, n_groups, packed):
    """Receive buffer, counts and per-row (token, expert) of group `group`; spec.T tokens in all."""
    cfg = moe.config_for(spec, packed=packed)
    W = moe.pack_layer(L) if packed else L
    Tl, El = spec.T // n_src, spec.E // n_groups
    idx, _ = moe.route(cfg, L["x"], W["w_router"], L["bias"])
    chunks, counts, tokens, experts = [], [], [], []
    for r in range(n_src):
        sl = slice(r * Tl, (r + 1) * Tl)
        offs, st, _, xp = moe.permute(cfg, idx[sl].contiguous(), L["x"][sl].contiguous())
        oh, sth = to_host(offs).astype(np.int64), to_host(st).astype(np.int64)
        a, b = oh[group * El], oh[(group + 1) * El]
        chunks.append(xp[a:b])
        counts.append(np.diff(oh)[group * El:(group + 1) * El])
        tokens.append(sth[a:b] + r * Tl)
        experts.append(np.repeat(np.arange(group * El, (group + 1) * El), np.diff(oh)[group * El:(group + 1) * El]))
    recv = torch.cat(chunks).contiguous()
    counts = np.stack(counts).astype(np.int32)
    return cfg, W, recv, counts, np.concatenate(tokens), np.concatenate(experts)


def run_share(spec, cfg, W, recv, counts, group, n_groups):
    El = spec.E // n_groups
    n = recv.shape[0]
    cnt = torch.from_numpy(counts).cuda()
    offsets, gather, scatter = moe.ep_receive_plan(cnt, n)
    local = moe.Config(spec.D, El, spec.K, spec.F, 0, cfg.dtype, cfg.out_dtype, cfg.packed)
    sl = slice(group * El, (group + 1) * El)
    h = moe.expert_gate_up(local, offsets, recv, W["w_gate"][sl], W["w_up"][sl], gather=gather, n_rows=n)
    y = moe.expert_down(local, offsets, h, W["w_down"][sl])
    y_recv = moe.gather_rows(y, scatter)
    torch.cuda.synchronize()
    return offsets, gather, scatter, y_recv


def check_share(spec, L, n_src, group, n_groups, packed, rows=None):
    cfg, W, recv, counts, tokens, experts = build_share(spec, L, n_src, group, n_groups, packed)
    offsets, gather, scatter, y_recv = run_share(spec, cfg, W, recv, counts, group, n_groups)
    ref = O.ep_receive_plan(counts)
    assert np.array_equal(to_host(offsets).astype(np.int64), ref["offsets"])
    assert np.array_equal(to_host(gather).astype(np.int64), ref["gather"])
    assert np.array_equal(to_host(scatter).astype(np.int64), ref["scatter"])
    # the receive buffer is each source's permuted rows: row i is token tokens[i]
    n = recv.shape[0]
    rows = np.arange(n) if rows is None else rows[rows < n]
    x_host = L["x"].cpu()
    assert torch.equal(recv.cpu()[torch.from_numpy(rows)], x_host[torch.from_numpy(tokens[rows])])
    Wo = oracle_weights(L)
    want = np.zeros((len(rows), spec.D))
    for e in np.unique(experts[rows]):
        sel = np.nonzero(experts[rows] == e)[0]
        want[sel] = O.swiglu_ffn(x_host[torch.from_numpy(tokens[rows][sel])], *Wo.expert(int(e)))
    return compare_out(to_host(y_recv[torch.from_numpy(rows).cuda()]), want, 2e-2, "received rows' expert outputs")


@pytest.mark.parametrize("group", [0, 3])
def test_ep_share_small(group):
    """4 source ranks x 64 tokens, 16 experts in 4 groups; every received row checked."""
    spec = synth.spec("tiny", T=256, D=256, E=16, K=4, F=128, Fs=0, dtype="bf16", seed=41)
    L = device_layer(spec)
    c = check_share(spec, L, 4, group, 4, packed=False)
    print(f"group {group}: out_rel={c['rel']:.3e}")


def test_ep_receive_plan_edges():
    """Empty chunks, a source with nothing for the share, and a row capacity below the total."""
    counts = np.array([[0, 5, 0], [0, 0, 0], [3, 1, 2]], dtype=np.int32)
    cnt = torch.from_numpy(counts).cuda()
    offsets, gather, scatter = moe.ep_receive_plan(cnt, 11)
    torch.cuda.synchronize()
    ref = O.ep_receive_plan(counts)
    assert np.array_equal(to_host(offsets), ref["offsets"])
    assert np.array_equal(to_host(gather), ref["gather"]) and np.array_equal(to_host(scatter), ref["scatter"])
    # capacity 6 of 11 rows: receive rows i < 6 get scatter[i]; gather[q] is written where q < 6
    offsets, gather, scatter = moe.ep_receive_plan(cnt, 6)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(offsets), ref["offsets"])
    assert np.array_equal(to_host(scatter), ref["scatter"][:6])
    g = to_host(gather)
    for i in range(6):
        q = ref["scatter"][i]
        if q < 6:
            assert g[q] == i
    # 8 x 36 random counts, as the decode/prefill share has
    rng = np.random.default_rng(4)
    counts = (rng.integers(0, 300, size=(8, 36)) * (rng.random((8, 36)) > 0.1)).astype(np.int32)
    n = int(counts.sum())
    offsets, gather, scatter = moe.ep_receive_plan(torch.from_numpy(counts).cuda(), n)
    torch.cuda.synchronize()
    ref = O.ep_receive_plan(counts)
    for a, b in ((offsets, ref["offsets"]), (gather, ref["gather"]), (scatter, ref["scatter"])):
        assert np.array_equal(to_host(a).astype(np.int64), b)


def test_gather_rows():
    """Rows of any width, index clamped to the source rows."""
    src = torch.arange(7 * 12, dtype=torch.float32, device="cuda").reshape(7, 12)
    idx = torch.tensor([6, 0, 3, 3, -2, 9], dtype=torch.int32, device="cuda")
    out = moe.gather_rows(src, idx)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), src.cpu()[torch.tensor([6, 0, 3, 3, 0, 6])])
    odd = torch.arange(5 * 3, dtype=torch.uint8, device="cuda").reshape(5, 3)  # 3-byte rows
    out = moe.gather_rows(odd, torch.tensor([4, 1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), odd.cpu()[torch.tensor([4, 1])])


@pytest.mark.parametrize("name,G", [("bf16_tiles128", 4), ("tiny", 8)])
def test_route_group_stats_small(name, G):
    from test_gpu_parity import SMALL
    spec = SMALL[name]
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    idx, prob, stats = moe.route_group_stats(cfg, L["x"], L["w_router"], G, L["bias"])
    idx2, prob2 = moe.route(cfg, L["x"], L["w_router"], L["bias"])
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(prob, prob2)
    check_stats(spec, L, idx, stats, G)


def check_stats(spec, L, idx, stats, G, k=None):
    W = oracle_weights(L)
    ref = O.route(L["x"].cpu(), W.router, spec.K, W.bias)
    st = O.group_stats(ref["p64"], to_host(idx), G)
    s = to_host(stats)
    assert np.array_equal(s[G:], st["pairs"].astype(np.float64)), "pair counts per group"
    assert np.allclose(s[:G], st["mass"], rtol=1e-5, atol=1e-6 * spec.T), (s[:G], st["mass"])
    f = s[G:] / s[G:].sum()
    l_ep = G * float(np.sum(f * s[:G] / spec.T))
    assert abs(l_ep - st["l_ep"]) <= 1e-5 * st["l_ep"]
    return l_ep


@pytest.mark.parametrize("name", ["prefill", "skew"])
def test_route_group_stats_full_size(name):
    """G = 8 groups of 36 experts: the page's split (section 3.2.3); skew is far from balanced."""
    spec = synth.spec(name)
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    idx, prob, stats = moe.route_group_stats(cfg, L["x"], L["w_router"], 8, L["bias"])
    torch.cuda.synchronize()
    W = oracle_weights(L)
    ref = O.route(L["x"].cpu(), W.router, spec.K, W.bias)
    compare_routing(to_host(idx), to_host(prob), ref, L["x"].cpu(), W.router)
    l_ep = check_stats(spec, L, idx, stats, 8)
    print(f"{name}: L_EP = {l_ep:.4f}")
    if name == "skew":
        assert l_ep > 1.5


def test_ep_share_full_size():
    """Group 0 of 8 (36 experts) under 8 source ranks x 8192 tokens of the prefill shape: the share
    the page's EP=8 deployment gives one GPU (about 65536 received rows). Sampled rows."""
    spec = synth.spec("prefill", T=8 * 8192)
    print("EP share: 8 ranks x 8192 tokens, group 0 of 8", flush=True)
    L = device_layer(spec)
    rows = sample_rows(8 * 8192, 24, 9)
    c = check_share(spec, L, 8, 0, 8, packed=True, rows=rows)
    print(f"EP share: out_rel={c['rel']:.3e}")
