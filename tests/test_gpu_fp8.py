"""FP8 (OCP E4M3) expert weights on the GPU against the oracle (reading R14).

moe_quantize_fp8 must give the oracle's codes and scales bit for bit (the
codes in the packed fp8 layout, unpacked here by its documented formula). The
layer with fp8 weights (moe_layer_forward, MOE_LAYOUT_FP8) is compared with
the oracle's layer on the dequantised weights decode(q) * s, under the same
tolerance rules as the bf16 layer: the fp32-output run within 2e-2 of RMS,
the bf16 output the rounding of that run; near-tie tokens held to the
validity rule of the bf16 tests. Small layers in full over the 32-, 64- and
128-row tiles, the decode and prefill workloads on sampled rows.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from moe_testutil import check_near_ties, compare_bf16_out, compare_out, compare_routing, compare_rows, device_layer, \
    oracle_weights, to_host
from oracle import moe_oracle as O
from test_gpu_parity import SMALL, rms_of, sample_rows

pytestmark = pytest.mark.gpu


def unpack_fp8(codes: np.ndarray, rows: int) -> np.ndarray:
    """Packed fp8 layout -> row-major codes [..., rows, cols] (the layout of include/moe.h)."""
    lead, R16, cols = codes.shape[:-2], codes.shape[-2], codes.shape[-1]
    flat = codes.reshape(*lead, R16 * cols)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    off = ((r // 16) * (cols // 64) + c // 64) * 1024 + ((r % 16) + 16 * ((c % 32) // 8)) * 16 + \
          ((c % 64) // 32) * 8 + c % 8
    return flat[..., off]


@pytest.mark.parametrize("shape", [(3, 20, 64), (1, 288, 128), (2, 16, 192), (1, 1, 64)])
def test_quantize_fp8_matches_oracle(shape):
    g = torch.Generator().manual_seed(sum(shape))
    w = torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[:-1] + (1,), generator=g) * 3)
    w[0, 0] = 0.0                                 # an all-zero row: scale 1, codes 0
    if shape[1] > 3:
        w[0, 2, :5] = torch.tensor([1e30, -1e30, 3e-38, -0.0, 1.0])   # extremes, subnormal, signed zero
    w = w.to(torch.bfloat16)
    codes, scales = moe.quantize_fp8(w.cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = O.quantize_rows_fp8(w.float().numpy())
    assert np.array_equal(to_host(scales), s_ref), "scales differ"
    got = unpack_fp8(to_host(codes), shape[1])
    assert np.array_equal(got, q_ref), f"{int((got != q_ref).sum())} codes differ"
    R16 = (shape[1] + 15) // 16 * 16
    if R16 > shape[1]:   # padding rows hold zero codes
        full = unpack_fp8(to_host(codes), R16)
        assert np.all(full[..., shape[1]:, :] == 0)


def fp8_oracle_weights(L) -> O.LayerWeights:
    """The layer the fp8 path computes: router unchanged, experts decode(q) * s (oracle quantisation)."""
    W = oracle_weights(L)
    deq = lambda w: O.dequantize_fp8(*O.quantize_rows_fp8(w))
    expert = lambda e: tuple(deq(m) for m in W.expert(e))
    sh = W.shared()
    shared = (lambda: tuple(deq(m) for m in sh)) if sh is not None else None
    return O.LayerWeights(W.router, expert, shared, W.bias)


def run_fp8(spec, L, rows=None, k=None):
    cfg = moe.config_for(spec, fp8=True)
    Q = moe.quantize_layer(L)
    out, idx, prob, offs = moe.layer_forward(cfg, L["x"], Q, routing=True, k_per_token=k)
    out32 = moe.layer_forward(dataclasses.replace(cfg, out_dtype=torch.float32), L["x"], Q, k_per_token=k)
    torch.cuda.synchronize()
    del Q
    Wq = fp8_oracle_weights(L)
    x_host = L["x"].cpu()
    kh = None if k is None else to_host(k)
    ref = O.route(x_host, Wq.router, spec.K, Wq.bias) if kh is None else O.route(x_host, Wq.router, spec.K, Wq.bias, kh)
    r = compare_routing(to_host(idx), to_host(prob), ref, x_host, Wq.router)
    # near ties: a valid top-k set, and the output of the experts the GPU chose
    gi = to_host(idx)
    tie = check_near_ties(gi, to_host(prob), ref, x_host, Wq.router, spec.K, kh)
    keep = np.nonzero(ref["gap"] >= 1e-6)[0]
    rows = keep if rows is None else np.intersect1d(rows, keep)
    # one oracle pass over the experts for the compared rows (the oracle's routing) and the
    # near-tie rows (the GPU's ids, the oracle's p of them): each expert dequantised once
    ig = gi[tie].astype(np.int64)
    p_tie = np.where(ig >= 0, np.take_along_axis(ref["p32"][tie].astype(np.float64), np.maximum(ig, 0), axis=1), 0.0)
    all_out = O.rows_output(x_host, Wq, np.concatenate([rows, tie]), np.concatenate([ref["idx"][rows], ig]),
                            np.concatenate([ref["prob"][rows].astype(np.float64), p_tie]))
    rr = {"out_rows": all_out[:len(rows)]}
    tie_ref = all_out[len(rows):]
    sel = lambda a, r=rows: to_host(a[torch.from_numpy(np.asarray(r)).to(a.device)])
    c32 = compare_out(sel(out32), rr["out_rows"], 2e-2, "fp8 layer, fp32 output")
    assert torch.equal(out, out32.to(torch.bfloat16)), "bf16 output is not the rounding of the fp32 output"
    c16 = compare_bf16_out(sel(out), rr["out_rows"])
    if tie.size:
        rms = rms_of(rr["out_rows"], tie_ref)
        compare_rows(sel(out32, tie), tie_ref, rms, 2e-2, False, "near-tie rows (fp8, fp32 output)")
        compare_rows(sel(out, tie), tie_ref, rms, 2e-2, True, "near-tie rows (fp8, bf16 output)")
    return r, c32, c16


FP8_SMALL = ["bf16_tiles32", "bf16_tiles32_fused", "bf16_tiles64", "bf16_tiles128", "bf16_tiles256",
             "bf16_tiles256_sparse", "bf16_k_equals_e", "bf16_router_rows_padded"]


@pytest.mark.parametrize("name", FP8_SMALL)
def test_fp8_layer_small(name):
    spec = SMALL[name] if name in SMALL else synth.spec("tiny", T=50, D=256, E=12, K=3, F=128, Fs=128,
                                                         dtype="bf16", seed=13)
    L = device_layer(spec)
    r, c32, c16 = run_fp8(spec, L)
    print(f"{name}: out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


def test_fp8_layer_dynamic_topk():
    spec = SMALL["bf16_tiles128"]
    L = device_layer(spec)
    k = synth.dynamic_k(spec, (0, 2, spec.K), "cuda")
    run_fp8(spec, L, k=k)


def test_fp8_shared_expert_of_another_width():
    """The shared expert in its own launch (width differs): its scales come through the same path."""
    spec = synth.spec("tiny", T=96, D=256, E=8, K=2, F=128, Fs=192, dtype="bf16", seed=15)
    L = device_layer(spec)
    run_fp8(spec, L)


@pytest.mark.parametrize("name", ["decode", "prefill", "skew", "full"])
def test_fp8_full_size(name):
    spec = synth.spec(name)
    print(f"fp8 weights, full size: {name}", flush=True)
    L = device_layer(spec)
    r, c32, c16 = run_fp8(spec, L, rows=sample_rows(spec.T, 6, 3))  # the oracle quantises each expert it uses
    print(f"{name}: out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")


@pytest.mark.parametrize("name", ["d256_f512", "d128_f192"])
def test_fp8_many_items_per_block(name):
    """fp8 weights through the 256x256 kernel with several items per block (the stream of 64-element
    stages runs on across items), the shortest and an odd number of stages per item; sampled rows."""
    from test_gpu_parity import MANY_ITEMS
    spec = MANY_ITEMS[name]
    L = device_layer(spec)
    r, c32, c16 = run_fp8(spec, L, rows=sample_rows(spec.T, 24, 11))
    print(f"{name}: out_rel(before cast)={c32['rel']:.3e} out_rel={c16['rel']:.3e}")
