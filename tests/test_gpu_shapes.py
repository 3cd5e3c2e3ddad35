"""Seeded sweep of layer shapes on the GPU against the oracle.

The parity cases elsewhere pick one shape per kernel path. This sweep draws
24 more from a fixed generator: token counts on both sides of every switch the
library makes (1 token; 32/33 and 64/65 around the router's split form and the
single-block permutation at T*K = 1024; 6144/6145 and 12288/12289 around
the fused router),
widths that do and do not fit the MFMA tiles (expert widths of at least 96
with more than 3000 tokens, see _shapes), 1 to 48 experts, K from 1 to 8,
no shared expert or one of another width, fp32 and bf16 layers, skewed
routing. Each layer is compared in full with the comparison rules of the
parity tests (near-tie tokens held to the validity rule), and bf16 layers
whose widths allow the packed layout must give bit-identical results with
packed weights. The layers of up to 3000 tokens also run with per-token
expert counts drawn from {0, K/2, K}, and those whose widths allow it with
fp8 expert weights (against the oracle on the dequantised weights).

test_large_token_count runs 262144 tokens (2M routed pairs, 32-bit row
offsets far from their limit) with routing and the permutation checked in
full and the output on sampled rows.

LIMITS adds layers at the edges of the configuration the library accepts:
1024 routed experts and K = 64 (the largest it takes) on the decode-size,
32-row and 256-row tile paths; 1022 and 1023 experts at T*K = 1024 (the
single-block permutation takes at most 1022); 320 and 321 experts at 6200
tokens (the fused router takes at most 320).
"""
from __future__ import annotations

import random

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from oracle import moe_oracle as O
from moe_testutil import check_near_ties, compare_routing, device_layer, near_tie_reference, oracle_weights, to_host
from test_gpu_dynamic_topk import k_draw, run_dynamic
from test_gpu_fp8 import run_fp8
from test_gpu_parity import check_outputs, run_full_compare, sample_rows

pytestmark = pytest.mark.gpu


def _shapes(n: int = 24, seed: int = 2026) -> dict:
    rng = random.Random(seed)
    tokens = [1, 2, 5, 31, 32, 33, 63, 64, 65, 97, 128, 129, 257, 511, 1025, 2049, 3000, 12288, 12289, 6144, 6145]
    widths = [64, 128, 192, 256, 320, 384, 512, 72, 200]
    ffn = [32, 64, 96, 128, 160, 192, 256, 320]
    out = {}
    for i in range(n):
        T = tokens[i % len(tokens)] if i < len(tokens) else rng.choice(tokens)
        big = T > 3000
        D = rng.choice(widths[1:4] if big else widths)   # the fused router takes d_model >= 128
        E = rng.randint(1, 48)
        K = rng.randint(1, min(E, 8))
        # with many tokens, widths of at least 96: at width 64 and below the one bf16 rounding of
        # h alone moves single outputs by about 2e-2 of the RMS (test_error_budget.py), so the
        # largest of millions of compared values can pass the bound without any fault
        F = rng.choice(ffn[2:6] if big else ffn)
        Fs = rng.choice([0, F, 64, 128])
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        skew = rng.random() < 0.25
        out[f"s{i:02d}_T{T}_D{D}_E{E}_K{K}_F{F}_Fs{Fs}_{dtype}{'_skew' if skew else ''}"] = synth.spec(
            "tiny", T=T, D=D, E=E, K=K, F=F, Fs=Fs, dtype=dtype, skew=skew, seed=100 + i)
    return out


SHAPES = _shapes()


def test_sweep_spans_the_switches():
    ts = {s.T for s in SHAPES.values()}
    assert {1, 32, 33, 64, 65, 6144, 6145, 12288, 12289} <= ts
    assert any(s.dtype == "f32" for s in SHAPES.values()) and any(s.Fs == 0 for s in SHAPES.values())


@pytest.mark.parametrize("name", list(SHAPES))
def test_shape(name):
    spec = SHAPES[name]
    print(f"shape {name}", flush=True)
    r, c32, c16 = run_full_compare(spec)
    print(f"{name}: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")
    if spec.dtype == "bf16" and spec.D % 64 == 0 and spec.F % 64 == 0 and spec.Fs % 64 == 0:
        L = device_layer(spec)
        rows = moe.layer_forward(moe.config_for(spec), L["x"], L, routing=True)
        packed = moe.layer_forward(moe.config_for(spec, packed=True), L["x"], moe.pack_layer(L), routing=True)
        torch.cuda.synchronize()
        for what, a, b in zip(("out", "topk_idx", "topk_prob", "offsets"), rows, packed):
            assert torch.equal(a, b), f"{name}: {what} differs between packed and row-major weights"


DYN = [n for n, s in SHAPES.items() if s.T <= 3000]
FP8 = [n for n, s in SHAPES.items()
       if s.T <= 3000 and s.dtype == "bf16" and s.D % 64 == 0 and s.F % 64 == 0 and s.Fs % 64 == 0]


@pytest.mark.parametrize("name", DYN)
def test_shape_dynamic_topk(name):
    spec = SHAPES[name]
    print(f"shape {name}, dynamic top-k", flush=True)
    r, c32, c16 = run_dynamic(spec, device_layer(spec), k_draw(spec))
    print(f"{name}: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


@pytest.mark.parametrize("name", FP8)
def test_shape_fp8(name):
    spec = SHAPES[name]
    print(f"shape {name}, fp8 expert weights", flush=True)
    r, c32, c16 = run_fp8(spec, device_layer(spec))
    print(f"{name}: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


LIMITS = {
    # bf16 expert widths of at least 128: at width 64 the one bf16 rounding of h alone moves the
    # largest output by about 2.2e-2 of the RMS (float64, 1023 experts, K = 64, 16 tokens), past
    # the 2e-2 bound without any fault
    # the largest expert count and K: 16 tokens (split router, T*K = 1024 with E > 1022: the
    # general permutation), 40 tokens (32-row tiles), 1024 tokens (256-row tiles: 64 rows per expert)
    "E1024_K64_T16": synth.spec("tiny", T=16, D=256, E=1024, K=64, F=128, Fs=128, dtype="bf16", seed=301),
    "E1024_K64_T40": synth.spec("tiny", T=40, D=256, E=1024, K=64, F=128, Fs=256, dtype="bf16", seed=302),
    "E1024_K64_T1024": synth.spec("tiny", T=1024, D=256, E=1024, K=64, F=128, Fs=128, dtype="bf16", seed=303),
    "E1024_K64_T40_f32": synth.spec("tiny", T=40, D=128, E=1024, K=64, F=32, Fs=0, dtype="f32", seed=304),
    # the single-block permutation at its expert limit and one past it (T*K = 1024)
    "E1022_K64_T16": synth.spec("tiny", T=16, D=256, E=1022, K=64, F=128, Fs=128, dtype="bf16", seed=305),
    "E1023_K64_T16": synth.spec("tiny", T=16, D=256, E=1023, K=64, F=128, Fs=128, dtype="bf16", seed=306),
    # the fused router at its expert limit and one past it (6145 to 12288 tokens)
    "E320_K8_T6200": synth.spec("tiny", T=6200, D=256, E=320, K=8, F=128, Fs=128, dtype="bf16", seed=307),
    "E321_K8_T6200": synth.spec("tiny", T=6200, D=256, E=321, K=8, F=128, Fs=128, dtype="bf16", seed=308),
    # K = 1 over 1024 experts with many tokens (two-kernel router, one row per pair)
    "E1024_K1_T3000": synth.spec("tiny", T=3000, D=256, E=1024, K=1, F=128, Fs=0, dtype="bf16", seed=309),
}


@pytest.mark.parametrize("name", list(LIMITS))
def test_limits(name):
    spec = LIMITS[name]
    print(f"limit {name}", flush=True)
    r, c32, c16 = run_full_compare(spec)
    print(f"{name}: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


@pytest.mark.parametrize("name", ["E1024_K64_T40", "E1024_K64_T1024"])
def test_limits_dynamic_topk(name):
    spec = LIMITS[name]
    print(f"limit {name}, dynamic top-k", flush=True)
    r, c32, c16 = run_dynamic(spec, device_layer(spec), k_draw(spec))
    print(f"{name}: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


def test_limits_fp8():
    spec = LIMITS["E1024_K64_T1024"]
    print("limit E1024_K64_T1024, fp8 expert weights", flush=True)
    r, c32, c16 = run_fp8(spec, device_layer(spec))
    print(f"fp8: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


def test_large_token_count():
    """262144 tokens over 64 experts (K = 8: 2M routed pairs, 32768 rows per expert, 256-row tiles,
    the two-kernel router and the rank/place permutation): routing and permutation in full, the
    output on sampled rows and on the near-tie tokens."""
    spec = synth.spec("tiny", T=262144, D=128, E=64, K=8, F=128, Fs=128, dtype="bf16", seed=311)
    print("large token count", flush=True)
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    out, idx, prob, offs = moe.layer_forward(cfg, L["x"], L, routing=True)
    torch.cuda.synchronize()
    W = oracle_weights(L)
    x_host = L["x"].cpu()
    ref = O.route(x_host, W.router, spec.K, W.bias)
    r = compare_routing(to_host(idx), to_host(prob), ref, x_host, W.router)
    gidx = to_host(idx)
    assert np.array_equal(to_host(offs).astype(np.int64), O.permute(gidx, spec.E)["offsets"])
    rows = sample_rows(spec.T, 24, 4321)
    rows = rows[ref["gap"][rows] >= 1e-6]
    rr = O.layer_rows(x_host, W, spec.K, rows)
    tie = check_near_ties(gidx, to_host(prob), ref, x_host, W.router, spec.K)
    tie = tie[:64]  # the validity rule holds for all of them; outputs for the first 64
    tie_ref = near_tie_reference(x_host, W, tie, gidx, ref) if tie.size else None
    c32, c16 = check_outputs(spec, cfg, L, out, rr["out_rows"], rows, tie, tie_ref)
    print(f"T={spec.T}: near_ties={r['near_ties']} out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")
