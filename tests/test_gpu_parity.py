"""GPU parity of the HIP library (through its C ABI) against the CPU oracle.

Small layers are compared in full; the five named workloads at their full
sizes are compared on all routing and permutation results and on sampled
output rows. Comparison rules are in moe_testutil.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from moe_testutil import (check_near_ties, compare_bf16_out, compare_out, compare_permutation, compare_routing,
                          compare_rows, device_layer, near_tie_reference, oracle_weights, out_tol, to_host)
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

# Small layers that the oracle finishes in seconds; they span several row and
# column tiles with ragged tails and exercise every kernel variant:
#   bf16 fast path with 256-row tiles (many rows per expert, or from 48 mean rows
#   per expert with the form that skips empty half items), 128-, 64- and
#   32-row tiles (few rows per expert; also with the shared expert fused as
#   one more group spanning two tiles), the generic path (fp32, or widths not multiple of
#   64), a shared expert of another width (not fused), no shared expert,
#   fp32 output, K = E, a single expert.
SMALL = {
    "tiny": synth.spec("tiny"),
    # 88 mean rows per group: 128-row tiles when the expert width is below 128 (the 256x256
    # kernel needs contractions of at least 128), else the 256x256 kernel's skipping form
    "bf16_tiles128": synth.spec("tiny", T=300, D=512, E=16, K=4, F=64, Fs=64, dtype="bf16", seed=1),
    "bf16_tiles256_mid": synth.spec("tiny", T=300, D=512, E=16, K=4, F=256, Fs=256, dtype="bf16", seed=1),
    "bf16_tiles32": synth.spec("tiny", T=37, D=256, E=16, K=6, F=192, Fs=128, dtype="bf16", seed=2),
    "bf16_tiles32_fused": synth.spec("tiny", T=37, D=256, E=64, K=6, F=192, Fs=192, dtype="bf16", seed=9),
    "bf16_tiles64": synth.spec("tiny", T=150, D=256, E=16, K=4, F=192, Fs=192, dtype="bf16", seed=10),
    "bf16_tiles256": synth.spec("tiny", T=600, D=512, E=8, K=2, F=320, Fs=320, dtype="bf16", seed=8),
    # 256-row tiles at 141 mean rows per group: most experts fill at most half a tile, so the
    # 256x256 kernel takes its form that skips the empty half of an item
    "bf16_tiles256_sparse": synth.spec("tiny", T=800, D=256, E=16, K=2, F=256, Fs=256, dtype="bf16", seed=9),
    "bf16_generic_widths": synth.spec("tiny", T=50, D=200, E=12, K=3, F=72, Fs=72, dtype="bf16", seed=3),
    "bf16_no_shared": synth.spec("tiny", T=129, D=384, E=24, K=8, F=128, Fs=0, dtype="bf16", seed=4),
    "bf16_k_equals_e": synth.spec("tiny", T=33, D=256, E=8, K=8, F=64, Fs=64, dtype="bf16", seed=5),
    "bf16_one_expert": synth.spec("tiny", T=70, D=128, E=1, K=1, F=128, Fs=64, dtype="bf16", seed=6),
    "f32_skew": synth.spec("tiny", T=200, D=192, E=40, K=5, F=96, Fs=96, skew=True, seed=7),
}


def with_out(cfg, out_dtype):
    return moe.Config(cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_expert, cfg.d_shared, cfg.dtype, out_dtype)


def check_outputs(spec, cfg, L, out, ref_out, rows=None, tie=None, tie_ref=None):
    """bf16 layers: strict bound on the fp32-output run, bf16 output within bound + half ulp.
    tie / tie_ref: near-tie tokens and their oracle rows under the GPU's routing, held to the same
    rule against the RMS of the compared rows."""
    sel = (lambda a: a) if rows is None else (lambda a: a[torch.from_numpy(rows).to(a.device)])
    at = lambda a, r: a[torch.from_numpy(np.asarray(r)).to(a.device)]
    if spec.dtype == "bf16":
        out32 = moe.layer_forward(with_out(cfg, torch.float32), L["x"], L)
        c32 = compare_out(to_host(sel(out32)), ref_out, 2e-2, "out (fp32 before the final cast)")
        assert torch.equal(out, out32.to(torch.bfloat16)), "bf16 output is not the rounding of the fp32 output"
        c16 = compare_bf16_out(to_host(sel(out)), ref_out)
        if tie is not None and len(tie):
            rms = rms_of(ref_out, tie_ref)
            compare_rows(to_host(at(out32, tie)), tie_ref, rms, 2e-2, False, "near-tie rows (fp32)")
            compare_rows(to_host(at(out, tie)), tie_ref, rms, 2e-2, True, "near-tie rows (bf16)")
        return c32, c16
    c = compare_out(to_host(sel(out)), ref_out, out_tol(spec))
    if tie is not None and len(tie):
        compare_rows(to_host(at(out, tie)), tie_ref, rms_of(ref_out, tie_ref), out_tol(spec), False, "near-tie rows")
    return c, c


def rms_of(*parts) -> float:
    """RMS over all compared rows (the near-tie rows included: a layer may have nothing else)."""
    a = np.concatenate([np.asarray(p, dtype=np.float64).reshape(-1) for p in parts])
    return math.sqrt(float(np.mean(a ** 2))) if a.size else 0.0


def run_full_compare(spec, L=None):
    L = L if L is not None else device_layer(spec)
    cfg = moe.config_for(spec)
    out, idx, prob, offs = moe.layer_forward(cfg, L["x"], L, routing=True)
    torch.cuda.synchronize()
    W = oracle_weights(L)
    ref = O.layer_forward(L["x"].cpu(), W, spec.K)
    r = compare_routing(to_host(idx), to_host(prob), ref, L["x"].cpu(), W.router)
    keep = ref["gap"] >= 1e-6
    tie = check_near_ties(to_host(idx), to_host(prob), ref, L["x"].cpu(), W.router, spec.K)
    tie_ref = near_tie_reference(L["x"].cpu(), W, tie, to_host(idx), ref) if tie.size else None
    # permutation of the GPU's own ids must equal the oracle's permutation of them
    p_ref = O.permute(to_host(idx), spec.E)
    assert np.array_equal(to_host(offs).astype(np.int64), p_ref["offsets"])
    rows = np.nonzero(keep)[0]
    c32, c16 = check_outputs(spec, cfg, L, out, ref["out"][rows], rows, tie, tie_ref)
    return r, c32, c16


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    r, c32, c16 = run_full_compare(SMALL[name])
    print(f"{name}: near_ties={r['near_ties']} prob_err={r['prob_err']:.2e} "
          f"out_rel(before cast)={c32['rel']:.3e} out_rel(output)={c16['rel']:.3e}")


def test_stages_small():
    """Each stage on identical inputs: route, permute (+gather), grouped FFN, combine.

    At expert width 64 (the 128-row tile layer) the one bf16 rounding of h alone moves
    the grouped-FFN output by 2.03% of its RMS, so the stage check runs at width 256."""
    spec = SMALL["bf16_tiles256_mid"]
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    W = oracle_weights(L)
    idx, prob, gap = moe.route(cfg, L["x"], L["w_router"], L["bias"], want_gap=True)
    ref = O.route(L["x"].cpu(), W.router, spec.K, W.bias)
    compare_routing(to_host(idx), to_host(prob), ref, L["x"].cpu(), W.router)
    keep = ref["gap"] >= 1e-6
    assert np.allclose(to_host(gap)[keep], ref["gap"][keep], atol=2e-7)

    offs, st, dest, x_perm = moe.permute(cfg, idx, L["x"])
    p_ref = O.permute(to_host(idx), spec.E)
    compare_permutation(to_host(offs), to_host(st), to_host(dest), p_ref)
    assert torch.equal(x_perm.cpu(), L["x"].cpu()[torch.from_numpy(p_ref["sorted_token"])])

    # grouped FFN over the permuted rows, both with the fused gather and on x_perm
    y = moe.grouped_ffn(cfg, offs, L["x"], L["w_gate"], L["w_up"], L["w_down"], gather=st)
    y2 = moe.grouped_ffn(cfg, offs, x_perm, L["w_gate"], L["w_up"], L["w_down"])
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    y_ref = O.grouped_ffn(x_perm.cpu(), p_ref["offsets"], W.expert)
    compare_out(to_host(y), y_ref, 2e-2, "grouped ffn")

    # shared expert as a single group over x
    ys = moe.grouped_ffn(cfg, torch.tensor([0, spec.T], dtype=torch.int32, device="cuda"), L["x"],
                         L["s_gate"][None], L["s_up"][None], L["s_down"][None])
    ys_ref = O.swiglu_ffn(L["x"].cpu(), *W.shared())
    compare_out(to_host(ys), ys_ref, 2e-2, "shared ffn")

    # combine on the GPU's own expert outputs: only fp32 summation order and the output rounding differ
    out = moe.combine(cfg, y, dest, prob, ys)
    out_ref = O.combine(to_host(ys), to_host(y), to_host(dest), to_host(prob))
    compare_bf16_out(to_host(out), out_ref, 1e-6, "combine")
    cfg32 = moe.Config(cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_expert, cfg.d_shared, cfg.dtype, torch.float32)
    out32 = moe.combine(cfg32, y, dest, prob, ys)
    compare_out(to_host(out32), out_ref, 1e-6, "combine fp32")


def test_expert_outputs_beyond_fp16_range():
    """Down projections scaled by 2^17 (exact in bf16): expert outputs reach ~5e5, far beyond the
    fp16 range (65504). On the 256-row-tile path the routed outputs are staged as fp16 with one
    power-of-two scale per 64-column row chunk, so they must come through as at unit scale."""
    spec = SMALL["bf16_tiles256"]
    L = dict(device_layer(spec))
    scale = 2.0 ** 17
    L["w_down"] = (L["w_down"].float() * scale).to(torch.bfloat16)
    L["s_down"] = (L["s_down"].float() * scale).to(torch.bfloat16)
    r, c32, c16 = run_full_compare(spec, L=L)
    print(f"scaled down projections: RMS {c32['rms']:.3e} out_rel(before cast)={c32['rel']:.3e}")
    assert c32["rms"] > 65504.0  # the outputs really are beyond the fp16 range


def test_routed_only():
    """Shared expert removed: the routed experts alone set the output RMS."""
    spec = synth.spec("tiny", T=256, D=512, E=32, K=8, F=256, Fs=0, dtype="bf16", seed=11)
    run_full_compare(spec)


def test_degenerate_routing():
    """All tokens on one expert (huge bias), zero-token experts, a single token, T = 0."""
    spec = synth.spec("tiny", T=64, D=256, E=16, K=2, F=128, Fs=128, dtype="bf16", seed=12)
    L = device_layer(spec)
    bias = torch.zeros(spec.E, dtype=torch.float32)
    bias[5] = 50.0
    L = dict(L, bias=bias.cuda())
    run_full_compare(spec, L=L)
    cfg = moe.config_for(spec)
    _, idx, _, offs = moe.layer_forward(cfg, L["x"], L, routing=True)
    counts = np.diff(to_host(offs))
    assert counts[5] == spec.T and counts.sum() == spec.T * spec.K
    one = dict(L, x=L["x"][:1].contiguous())
    s1 = synth.spec("tiny", T=1, D=256, E=16, K=2, F=128, Fs=128, dtype="bf16", seed=12)
    run_full_compare(s1, L=one)
    empty = moe.layer_forward(cfg, L["x"][:0], L)
    assert empty.shape == (0, spec.D)


def test_deterministic():
    spec = SMALL["bf16_tiles128"]
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    a = moe.layer_forward(cfg, L["x"], L, routing=True)
    b = moe.layer_forward(cfg, L["x"], L, routing=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_generator_cpu_gpu_identical():
    """The device inputs are the generator's: bit-identical to the same streams drawn on the CPU."""
    spec = synth.spec("decode")
    L = device_layer(spec)
    for e in (0, 137, spec.E - 1):
        g, u, d = synth.make_expert(spec, e, "cpu")
        assert torch.equal(L["w_gate"][e].cpu(), g)
        assert torch.equal(L["w_up"][e].cpu(), u)
        assert torch.equal(L["w_down"][e].cpu(), d)
    assert torch.equal(L["x"].cpu(), synth.make_x(spec, "cpu"))
    assert torch.equal(L["w_router"].cpu(), synth.make_router(spec, "cpu"))
    sg, su, sd = synth.make_expert(spec, spec.E, "cpu")
    assert torch.equal(L["s_down"].cpu(), sd)


# --------------------------------------------------------- full-size workloads ---

def sample_rows(T: int, n: int, seed: int, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must)
    rows.update(int(r) for r in rng.choice(T, size=min(n, T), replace=False))
    rows.update({0, T - 1})
    return np.array(sorted(rows))


# the four workloads, and the prefill shape at 512 tokens (32-row tiles with about 14 rows per
# expert, router over 16 contraction slices) and 1024 tokens (64-row tiles, 8 slices)
@pytest.mark.parametrize("name,n_rows,T", [("decode", 32, None), ("prefill", 12, None), ("skew", 12, None),
                                           ("full", 6, None), ("prefill", 12, 512), ("prefill", 12, 1024)])
def test_layer_full_size(name, n_rows, T):
    spec = synth.spec(name) if T is None else synth.spec(name, T=T)
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    out, idx, prob, offs = moe.layer_forward(cfg, L["x"], L, routing=True)
    torch.cuda.synchronize()
    W = oracle_weights(L)
    x_host = L["x"].cpu()
    ref = O.route(x_host, W.router, spec.K, W.bias)
    r = compare_routing(to_host(idx), to_host(prob), ref, x_host, W.router)
    # permutation: exact against the oracle's permutation of the GPU's ids, plus invariants
    gidx = to_host(idx)
    p_ref = O.permute(gidx, spec.E)
    offs_h = to_host(offs).astype(np.int64)
    assert np.array_equal(offs_h, p_ref["offsets"])
    counts = np.diff(offs_h)
    assert counts.sum() == spec.T * spec.K
    load = O.expert_load(counts)
    # sampled output rows (the hottest expert's first token included)
    hot = int(np.argmax(counts))
    first_hot = int(np.nonzero(np.any(gidx == hot, axis=1))[0][0])
    rows = sample_rows(spec.T, n_rows, 1234, must=[first_hot])
    rows = rows[ref["gap"][rows] >= 1e-6]
    rr = O.layer_rows(x_host, W, spec.K, rows)
    # near ties: a valid top-K set, and the output of the experts the GPU chose
    tie = check_near_ties(gidx, to_host(prob), ref, x_host, W.router, spec.K)
    tie_ref = near_tie_reference(x_host, W, tie, gidx, ref) if tie.size else None
    c32, c16 = check_outputs(spec, cfg, L, out, rr["out_rows"], rows, tie, tie_ref)
    msg = (f"{name} T={spec.T}: near_ties={r['near_ties']} prob_err={r['prob_err']:.2e} prob_rel={r['prob_rel']:.2e} "
           f"bound_use={r['bound_use']:.3f} touched={load['touched']} "
           f"skew={load['skew']:.2f} out_rel(before cast)={c32['rel']:.3e} out_rel(output)={c16['rel']:.3e} "
           f"rows={len(rows)} near_tie_rows_checked={len(tie)}")
    if spec.groups:
        msg += f" group_counts={O.group_counts(counts, spec.groups).tolist()}"
    print(msg)
    if name == "skew":
        assert load["skew"] > 10.0  # the Zipf-like bias makes the hottest expert >10x the mean load


MANY_ITEMS = {
    "d256_f512": synth.spec("tiny", T=16384, D=256, E=16, K=2, F=512, Fs=512, dtype="bf16", seed=21),
    # the shortest contractions the 256x256 kernel takes (128: two A stages per item) and an odd
    # number of A stages per item (192: three), so the two A slots alternate across items
    "d128_f192": synth.spec("tiny", T=32768, D=128, E=8, K=2, F=192, Fs=192, dtype="bf16", seed=22),
}


@pytest.mark.parametrize("name", list(MANY_ITEMS))
def test_layer_many_items_per_block(name):
    """Many rows per expert with narrow layers: the 256x256 GEMM's blocks (one per CU) each take
    several (row tile, column block) items in turn (the load stream continues from one item into
    the next), and the shared expert's row tiles run in several chunks of row tiles. Routing
    and permutation in full, output rows sampled."""
    spec = MANY_ITEMS[name]
    L = device_layer(spec)
    cfg = moe.config_for(spec, packed=True)
    P = moe.pack_layer(L)
    out, idx, prob, offs = moe.layer_forward(cfg, L["x"], P, routing=True)
    torch.cuda.synchronize()
    W = oracle_weights(L)
    x_host = L["x"].cpu()
    ref = O.route(x_host, W.router, spec.K, W.bias)
    compare_routing(to_host(idx), to_host(prob), ref, x_host, W.router)
    p_ref = O.permute(to_host(idx), spec.E)
    assert np.array_equal(to_host(offs).astype(np.int64), p_ref["offsets"])
    counts = np.diff(p_ref["offsets"])
    rows_per_group = (spec.T * spec.K + spec.T) / (spec.E + 1)
    assert rows_per_group >= 96 and counts.max() > 256  # 256-row tiles, groups of several tiles
    rows = sample_rows(spec.T, 24, 77)
    rows = rows[ref["gap"][rows] >= 1e-6]
    rr = O.layer_rows(x_host, W, spec.K, rows)
    cfg_rows = moe.config_for(spec)  # the fp32-output rerun inside check_outputs uses row-major weights
    c32, c16 = check_outputs(spec, cfg_rows, L, out, rr["out_rows"], rows)
    print(f"many items: rows={len(rows)} out_rel(before cast)={c32['rel']:.3e} out_rel(output)={c16['rel']:.3e}")


def test_stage_permutation_full_prefill():
    """Standalone moe_permute at the prefill size equals the oracle's permutation exactly."""
    spec = synth.spec("prefill")
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    idx, prob = moe.route(cfg, L["x"], L["w_router"], L["bias"])
    offs, st, dest = moe.permute(cfg, idx)
    torch.cuda.synchronize()
    p_ref = O.permute(to_host(idx), spec.E)
    compare_permutation(to_host(offs), to_host(st), to_host(dest), p_ref)


def whole_segments(spec, L, W_dev, cfg):
    """Every row of whole expert segments through the layer's own expert launch (the E routed
    groups plus the shared expert as one more group, rows gathered through the permutation:
    the arguments moe_layer_forward passes to its expert GEMMs), against the oracle's FFN.
    Segments: the hottest expert (several 256-row tiles), the smallest expert above 256 rows
    (two tiles), the smallest above 512 rows if any, and the shared expert's first and last
    row tiles."""
    T, K, E, F = spec.T, spec.K, spec.E, spec.F
    P = T * K
    idx, _ = moe.route(cfg, L["x"], W_dev["w_router"], L["bias"])
    offs, st, _ = moe.permute(cfg, idx)
    offs_ext = torch.cat([offs, torch.tensor([P + T], dtype=torch.int32, device=offs.device)])
    h = moe.expert_gate_up(cfg, offs_ext, L["x"], W_dev["w_gate"], W_dev["w_up"], gather=st, n_rows=P + T,
                           s_gate=W_dev["s_gate"], s_up=W_dev["s_up"])
    y = moe.expert_down(cfg, offs_ext, h, W_dev["w_down"], s_down=W_dev["s_down"])
    torch.cuda.synchronize()
    del h
    oh = to_host(offs_ext).astype(np.int64)
    sth = to_host(st).astype(np.int64)
    counts = np.diff(oh[:E + 1])
    W = oracle_weights(L)
    x_host = L["x"].cpu()
    segs = [("hottest expert", int(np.argmax(counts)))]
    for lim in (256, 512):
        over = np.nonzero(counts > lim)[0]
        if over.size:
            segs.append((f"smallest expert above {lim} rows", int(over[np.argmin(counts[over])])))
    done = []
    for label, e in segs:
        a, b = int(oh[e]), int(oh[e + 1])
        ref = O.swiglu_ffn(x_host[torch.from_numpy(sth[a:b])], *W.expert(e))
        c = compare_out(to_host(y[a:b]), ref, 2e-2, f"{label} {e} ({b - a} rows)")
        done.append(f"{label} {e}: {b - a} rows, rel {c['rel']:.2e}")
    sg = W.shared()
    for label, t0 in (("shared expert, first tile", 0), ("shared expert, last tile", max(0, T - 256))):
        t1 = min(T, t0 + 256)
        ref = O.swiglu_ffn(x_host[t0:t1], *sg)
        c = compare_out(to_host(y[P + t0:P + t1]), ref, 2e-2, label)
        done.append(f"{label}: {t1 - t0} rows, rel {c['rel']:.2e}")
    assert counts.max() > 256, "the hottest expert should span several row tiles"
    return done


@pytest.mark.parametrize("name", ["prefill", "skew", "full"])
def test_whole_segments_full_size(name):
    """Whole expert segments at the full workload sizes, every row compared (packed weights, the
    layout the benchmark times)."""
    spec = synth.spec(name)
    L = device_layer(spec)
    cfg = moe.config_for(spec, packed=True)
    Wp = moe.pack_layer(L)
    done = whole_segments(spec, L, Wp, cfg)
    del Wp
    torch.cuda.empty_cache()
    print(f"{name}: " + "; ".join(done))


@pytest.mark.parametrize("name", list(MANY_ITEMS))
def test_whole_segments_many_items(name):
    """Whole segments of the narrow many-items layers (several items per 256x256 block)."""
    spec = MANY_ITEMS[name]
    L = device_layer(spec)
    cfg = moe.config_for(spec, packed=True)
    done = whole_segments(spec, L, moe.pack_layer(L), cfg)
    print(f"{name}: " + "; ".join(done))
