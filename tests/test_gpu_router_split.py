"""The router at the model's width (d_model 4096, 288 experts, top-8) at every
token count where its form changes, through moe_route, against the oracle.

Up to 6144 tokens the library runs the router GEMM with its contraction cut
into 16, 8, 4, 2 or 1 slices (more slices the fewer row tiles there are) and
a top-k kernel that adds the slices' partial logits in order; from 6145 to
12288 tokens the fused router kernel; above that the unsplit GEMM and the
one-wave-per-token top-k. The token counts below take each slice count and
both sides of the switches. Routing is compared in full (ordered ids outside
near-ties, probabilities within the fp32 accumulation bound, near-tie tokens
held to the validity rule), with row-major and packed router weights, whose
results must be identical. The oracle routes the 12289 tokens once; a prefix
of x is the same tokens, so each count compares against the oracle's prefix.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from oracle import moe_oracle as O
from moe_testutil import check_near_ties, compare_routing, to_host

pytestmark = pytest.mark.gpu

# 16 slices (65 .. 512 tokens: 1 .. 4 row tiles of 128 x 5 column blocks), 8 (1024), 4 (2048),
# 2 (4096), 1 (6144), fused (6145, 12288), unsplit two-kernel (12289)
TOKENS = [65, 128, 512, 513, 1024, 2048, 4096, 6144, 6145, 12288, 12289]
SPEC = synth.spec("prefill", T=max(TOKENS))


@pytest.fixture(scope="module")
def router_case():
    x = synth.make_x(SPEC, "cuda")
    w = synth.make_router(SPEC, "cuda")
    b = synth.router_bias(SPEC)
    bias = None if b is None else b.to("cuda")
    x_host, w_host = x.cpu(), w.cpu()
    ref = O.route(x_host, w_host, SPEC.K, None if b is None else b.cpu())
    return x, w, bias, x_host, w_host, ref


@pytest.mark.parametrize("T", TOKENS)
def test_router_at_model_width(router_case, T):
    x, w, bias, x_host, w_host, ref = router_case
    print(f"router d_model={SPEC.D} E={SPEC.E} K={SPEC.K} T={T}", flush=True)
    spec = synth.spec("prefill", T=T)
    xs = x[:T]
    idx, prob = moe.route(moe.config_for(spec), xs, w, bias)
    idx_p, prob_p = moe.route(moe.config_for(spec, packed=True), xs, moe.pack_weights(w), bias)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_p) and torch.equal(prob, prob_p), "packed and row-major router weights differ"
    r_t = {k: v[:T] for k, v in ref.items()}
    gi, gp = to_host(idx), to_host(prob)
    r = compare_routing(gi, gp, r_t, x_host[:T], w_host)
    check_near_ties(gi, gp, r_t, x_host[:T], w_host, SPEC.K)
    print(f"T={T}: near_ties={r['near_ties']} prob_rel={r['prob_rel']:.3e} bound_use={r['bound_use']:.3f}")
    assert np.all(gi >= 0) and np.all(gi < SPEC.E)
