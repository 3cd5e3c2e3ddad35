"""The layer entry point that allocates nothing (moe_layer_forward_noalloc), through the C ABI.

Its workspace is the library's static device scratch. Two calls in a row, the
second with fewer tokens, must give exactly what moe_layer_forward gives with a
caller workspace (the kernels are deterministic and the same); a layer whose
workspace would exceed the scratch is rejected before anything runs.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from moe_testutil import compare_routing, device_layer, oracle_weights, to_host
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


def _outputs(cfg, T, dev):
    return (torch.empty((T, cfg.d_model), dtype=cfg.odtype, device=dev),
            torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev),
            torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev),
            torch.empty((cfg.n_experts + 1,), dtype=torch.int32, device=dev))


@pytest.mark.parametrize("name,packed", [("decode", True), ("small", False)])
def test_noalloc_equals_layer_forward(name, packed):
    if name == "decode":
        spec = synth.spec("decode")
        sizes = (spec.T, 19)
    else:
        spec = synth.spec("tiny", T=300, D=512, E=16, K=4, F=256, Fs=256, dtype="bf16", seed=1)
        sizes = (300, 123)
    L = device_layer(spec)
    cfg = moe.config_for(spec, packed=packed)
    W = moe.pack_layer(L) if packed else L
    wt = moe.weights_struct(cfg, W)
    dev = L["x"].device
    scratch = moe.noalloc_scratch_bytes()
    assert scratch == 64 << 20
    for T in sizes:  # two calls in a row on the shared scratch, the second smaller
        assert moe.lib().moe_layer_workspace_bytes(ctypes.byref(cfg.c()), T) <= scratch
        x = L["x"][:T].contiguous()
        out, idx, prob, offs = _outputs(cfg, T, dev)
        moe.layer_forward_noalloc(cfg, x, out, wt, idx, prob, offs)
        ref_out, ref_idx, ref_prob, ref_offs = moe.layer_forward(cfg, x, W, routing=True, weights=wt)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx) and torch.equal(prob, ref_prob) and torch.equal(offs, ref_offs)
        assert torch.equal(out, ref_out), f"T={T}: output differs from moe_layer_forward"
        # and the routing against the oracle (the output equals moe_layer_forward's, whose parity is tested)
        Wo = oracle_weights(L)
        ref = O.route(x.cpu(), Wo.router, spec.K, Wo.bias)
        compare_routing(to_host(idx), to_host(prob), ref, x.cpu(), Wo.router)
        assert np.array_equal(np.diff(to_host(offs).astype(np.int64)), O.permute(to_host(idx), spec.E)["counts"])


def test_noalloc_rejects_layers_beyond_the_scratch():
    spec = synth.spec("decode")
    L = device_layer(spec)
    cfg = moe.config_for(spec)
    wt = moe.weights_struct(cfg, L)
    T = 1024
    assert moe.lib().moe_layer_workspace_bytes(ctypes.byref(cfg.c()), T) > moe.noalloc_scratch_bytes()
    x = torch.zeros((T, spec.D), dtype=cfg.dtype, device=L["x"].device)
    out = torch.full((T, spec.D), 7.0, dtype=cfg.odtype, device=x.device)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_forward_noalloc(cfg, x, out, wt)
    assert e.value.status == 4 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing ran
