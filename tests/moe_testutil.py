"""Shared helpers of the parity tests: workloads on the device, the oracle's
view of the same weights, and the comparison rules.

Comparison rules (the layer's tolerances):
  - routing: expert ids equal as ordered lists, except tokens whose oracle
    gap between the K-th and (K+1)-th float32 probability is below 1e-6
    (near-ties, counted and reported); selected probabilities within 1e-6;
  - permutation (offsets, sorted_token, dest): bit-exact given the same ids;
  - output: max |gpu - oracle| <= 2e-2 * RMS(oracle) over compared rows
    (bf16 inputs and output, fp32 accumulation); fp32 layers 1e-4 * RMS.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from oracle import moe_oracle as O

NEAR_TIE = 1e-6
PROB_TOL = 1e-6


def out_tol(spec) -> float:
    return 2e-2 if spec.dtype == "bf16" else 1e-4


_LAYERS: dict = {}


def device_layer(spec, device="cuda") -> dict:
    """Inputs of `spec` generated on the device (weights cached across workloads of equal shape)."""
    key = (spec.D, spec.E, spec.F, spec.Fs, spec.dtype, spec.seed, str(device))
    if key not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        w = synth.make_layer(synth.spec("tiny", T=1, D=spec.D, E=spec.E, K=1, F=spec.F, Fs=spec.Fs,
                                        dtype=spec.dtype, seed=spec.seed), device)
        _LAYERS[key] = w
    base = _LAYERS[key]
    L = dict(base)
    L["x"] = synth.make_x(spec, device)
    b = synth.router_bias(spec)
    L["bias"] = None if b is None else b.to(device)
    return L


def oracle_weights(L: dict) -> O.LayerWeights:
    """The oracle's view of the layer: every tensor copied to host memory when first used."""
    cache = {}

    def host(t):
        return None if t is None else t.detach().cpu()

    def expert(e):
        if e not in cache:
            if len(cache) > 48:
                cache.clear()
            cache[e] = (host(L["w_gate"][e]), host(L["w_up"][e]), host(L["w_down"][e]))
        return cache[e]

    def shared():
        if L.get("s_gate") is None:
            return None
        return host(L["s_gate"]), host(L["s_up"]), host(L["s_down"])

    return O.LayerWeights(host(L["w_router"]), expert, shared, host(L.get("bias")))


def compare_routing(idx_gpu, prob_gpu, ref) -> dict:
    """Ordered-id equality and probability closeness outside near-ties."""
    idx_gpu = np.asarray(idx_gpu)
    prob_gpu = np.asarray(prob_gpu, dtype=np.float64)
    keep = ref["gap"] >= NEAR_TIE
    bad = np.nonzero(keep & np.any(idx_gpu != ref["idx"], axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens routed differently, first {bad[:5]}: " \
                          f"gpu {idx_gpu[bad[0]]} oracle {ref['idx'][bad[0]]}"
    dp = np.abs(prob_gpu - ref["prob"].astype(np.float64))[keep]
    assert dp.size == 0 or dp.max() <= PROB_TOL, f"probability error {dp.max():.3e}"
    return dict(near_ties=int((~keep).sum()), prob_err=float(dp.max()) if dp.size else 0.0)


def compare_permutation(offs, st, dest, ref) -> None:
    assert np.array_equal(np.asarray(offs, np.int64), ref["offsets"]), "offsets differ"
    assert np.array_equal(np.asarray(st, np.int64), ref["sorted_token"]), "sorted_token differs"
    assert np.array_equal(np.asarray(dest, np.int64), ref["dest"]), "dest differs"


def compare_out(out_gpu, out_ref, tol_rel: float, what="out") -> dict:
    g = np.asarray(out_gpu, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    rms = math.sqrt(float(np.mean(out_ref ** 2))) if out_ref.size else 0.0
    err = float(np.max(np.abs(g - out_ref))) if out_ref.size else 0.0
    assert err <= tol_rel * rms + 1e-30, f"{what}: max abs error {err:.4e} > {tol_rel} * RMS {rms:.4e}"
    return dict(max_abs=err, rms=rms, rel=err / rms if rms else 0.0)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()
