"""Shared helpers of the parity tests: workloads on the device, the oracle's
view of the same weights, and the comparison rules.

Comparison rules (the layer's tolerances):
  - routing: expert ids equal as ordered lists, except tokens whose oracle
    gap between the K-th and (K+1)-th float32 probability is below 1e-6
    (near-ties, counted and reported). Selected probabilities: a logit error
    d shifts p by at most a factor exp(+-2d); the logits are length-D dot
    products of exact bf16 products summed in fp32, whose error is bounded
    (probabilistically, Higham and Mary 2019) by sqrt(D) * u * sum_d |x_d w_d|
    with u = 2^-24. So |p_gpu - p| <= 2 p sqrt(D) u S_te + 8 u p, with S_te
    the sum of absolute products of token t and expert e;
  - permutation (offsets, sorted_token, dest): bit-exact given the same ids;
  - output of a bf16 layer (bf16 inputs, fp32 accumulation): the layer run
    with an fp32 output, i.e. the arithmetic before the final cast, satisfies
    max |gpu - oracle| <= 2e-2 * RMS(oracle); the bf16 output is within
    2e-2 * RMS + half a bf16 ulp of the oracle value, element by element.
    The half ulp is the final cast's own error: rounding the exact result to
    bf16 can by itself exceed 2e-2 * RMS once |out| >= 4 with RMS < 0.78;
  - output of an fp32 layer: max |gpu - oracle| <= 1e-4 * RMS(oracle);
  - near-tie tokens (several top-K sets are right): the GPU's ids must be K
    distinct experts whose oracle probabilities, widened by the same bound,
    reach every unchosen expert's (min over chosen of p + b >= max over
    unchosen of p - b), its probabilities within the bound of the oracle's at
    those ids and non-increasing; and the token's output must match the
    oracle's output recomputed with the GPU's ids (and the oracle's
    probabilities of them), to the output rule above.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from oracle import moe_oracle as O

NEAR_TIE = 1e-6


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


U32 = 2.0 ** -24


def prob_bound(x, w_router, idx, prob) -> np.ndarray:
    """Per selected (t, k): 2 p sqrt(D) u S + 8 u p, S = sum_d |x_td W_r[e,d]| (see the module notes)."""
    xa = np.abs(O.as_f64(x))
    wa = np.abs(O.as_f64(w_router))
    S = np.take_along_axis(xa @ wa.T, np.asarray(idx, dtype=np.int64), axis=1)
    p = np.asarray(prob, dtype=np.float64)
    return 2.0 * p * math.sqrt(xa.shape[1]) * U32 * S + 8.0 * U32 * p


def compare_routing(idx_gpu, prob_gpu, ref, x, w_router) -> dict:
    """Ordered-id equality outside near-ties; probabilities within the fp32 accumulation bound."""
    idx_gpu = np.asarray(idx_gpu)
    prob_gpu = np.asarray(prob_gpu, dtype=np.float64)
    keep = ref["gap"] >= NEAR_TIE
    bad = np.nonzero(keep & np.any(idx_gpu != ref["idx"], axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens routed differently, first {bad[:5]}: " \
                          f"gpu {idx_gpu[bad[0]]} oracle {ref['idx'][bad[0]]}"
    pref = ref["prob"].astype(np.float64)
    dp = np.abs(prob_gpu - pref)[keep]
    bound = prob_bound(x, w_router, ref["idx"], pref)[keep]
    worst = int(np.argmax(dp - bound)) if dp.size else 0
    assert dp.size == 0 or np.all(dp <= bound), \
        f"probability error {dp.flat[worst]:.3e} > bound {bound.flat[worst]:.3e}"
    rel = dp / np.maximum(pref[keep], 1e-30)
    return dict(near_ties=int((~keep).sum()), prob_err=float(dp.max()) if dp.size else 0.0,
                prob_rel=float(rel.max()) if rel.size else 0.0,
                bound_use=float(np.max(dp / np.where(bound > 0, bound, 1.0))) if dp.size else 0.0)


def check_near_ties(idx_gpu, prob_gpu, ref, x, w_router, K: int, k_per_token=None) -> np.ndarray:
    """Validity of the GPU's routing of the near-tie tokens (see the module notes); returns those tokens.
    With k_per_token, token t's set is its first k_t = clip(k_t, 0, K) slots, the rest holding -1."""
    tie = np.nonzero(ref["gap"] < NEAR_TIE)[0]
    if tie.size == 0:
        return tie
    p = ref["p32"][tie].astype(np.float64)                      # [n, E]
    xa = np.abs(O.as_f64(x)[tie])
    wa = np.abs(O.as_f64(w_router))
    b = 2.0 * p * math.sqrt(xa.shape[1]) * U32 * (xa @ wa.T) + 8.0 * U32 * p
    ig = np.asarray(idx_gpu)[tie].astype(np.int64)
    pg = np.asarray(prob_gpu, dtype=np.float64)[tie]
    E = p.shape[1]
    kt = np.full(len(tie), K) if k_per_token is None else np.clip(np.asarray(k_per_token)[tie], 0, K)
    for i, t in enumerate(tie):
        n = int(kt[i])
        chosen = ig[i][:n]
        assert np.all(ig[i][n:] == -1), f"near-tie token {t}: slots past its {n} experts hold ids"
        assert np.all((chosen >= 0) & (chosen < E)) and len(set(chosen.tolist())) == n, \
            f"near-tie token {t}: ids {chosen} are not {n} distinct experts"
        mask = np.zeros(E, dtype=bool)
        mask[chosen] = True
        low = float(np.min((p[i] + b[i])[mask])) if n else np.inf
        high = float(np.max((p[i] - b[i])[~mask])) if (~mask).any() else -np.inf
        assert low >= high, f"near-tie token {t}: chosen {chosen} is not a top-{n} set within the bound " \
                            f"({low:.9g} < {high:.9g})"
        assert np.all(np.abs(pg[i][:n] - p[i][chosen]) <= b[i][chosen]), f"near-tie token {t}: probabilities off"
        assert np.all(np.diff(pg[i][:n]) <= 0), f"near-tie token {t}: probabilities not in descending order"
    return tie


def near_tie_reference(x, W, tie, idx_gpu, ref) -> np.ndarray:
    """The oracle's output rows of the near-tie tokens, recomputed with the GPU's ids and the oracle's p of them."""
    ig = np.asarray(idx_gpu)[tie].astype(np.int64)
    pr = np.take_along_axis(ref["p32"][tie].astype(np.float64), np.maximum(ig, 0), axis=1)
    return O.rows_output(x, W, tie, ig, np.where(ig >= 0, pr, 0.0))


def compare_rows(out_gpu_rows, out_ref_rows, rms: float, tol_rel: float, bf16: bool, what: str) -> float:
    """Rows compared against a reference RMS taken elsewhere (the whole compared output)."""
    g = np.asarray(out_gpu_rows, dtype=np.float64)
    r = np.asarray(out_ref_rows, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - r)
    bound = tol_rel * rms + (bf16_half_ulp(r) if bf16 else 0.0)
    assert np.all(err <= bound), f"{what}: error {float(np.max(err - bound)):.3e} over the bound"
    return float(err.max()) / rms if rms else 0.0


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


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |v| (8 significant bits): 2**(floor(log2|v|) - 8)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 8)


def compare_bf16_out(out16, out_ref, tol_rel: float = 2e-2, what="out bf16") -> dict:
    """bf16 output: |gpu - oracle| <= tol_rel * RMS + half ulp(oracle), element by element."""
    g = np.asarray(out16, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    rms = math.sqrt(float(np.mean(out_ref ** 2))) if out_ref.size else 0.0
    err = np.abs(g - out_ref)
    bound = tol_rel * rms + bf16_half_ulp(out_ref)
    worst = int(np.argmax(err - bound)) if err.size else 0
    assert err.size == 0 or np.all(err <= bound), \
        f"{what}: error {err.flat[worst]:.4e} > bound {bound.flat[worst]:.4e} at |ref| {abs(out_ref.flat[worst]):.3f}"
    return dict(max_abs=float(err.max()) if err.size else 0.0, rms=rms,
                rel=float(err.max()) / rms if rms else 0.0)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()
