"""The layer captured in a HIP graph and replayed, through the C ABI.

Every step of the layer is a kernel launch on the caller's stream; the library
records no memset or copy and allocates nothing during a call, so a caller can
capture the layer once (static input, output and workspace buffers) and replay
it. Each replay here runs on new input values copied into the static input,
with eager work and a synchronisation between replays, and must give exactly
what the eager call gives for the same input (the kernels are deterministic).
Both the entry point with a caller workspace (moe_layer_forward) and the one
without (moe_layer_forward_noalloc, the form meant for callers that cannot
allocate) are captured.
"""
from __future__ import annotations

import pytest
import torch

import synth
import top_routed_expert_amd as moe
from moe_testutil import device_layer

pytestmark = pytest.mark.gpu

GRAPH_LAYERS = {
    # 32-row tiles, split router, single-block permutation (decode-like)
    "small_batch": synth.spec("tiny", T=32, D=512, E=32, K=8, F=256, Fs=256, dtype="bf16", seed=41),
    # router over four contraction slices with the wave top-k, rank/place permutation, 256x256
    # expert GEMMs, 16-bit expert outputs
    "large_batch": synth.spec("tiny", T=2048, D=256, E=8, K=2, F=256, Fs=256, dtype="bf16", seed=42),
    # the fused router kernel (6145 to 12288 tokens)
    "fused_router": synth.spec("tiny", T=6200, D=256, E=8, K=2, F=256, Fs=256, dtype="bf16", seed=43),
}


def _inputs(spec, n, dev):
    g = torch.Generator(device="cpu").manual_seed(spec.seed)
    return [torch.randn((spec.T, spec.D), generator=g).to(torch.bfloat16).to(dev) for _ in range(n)]


@pytest.mark.parametrize("name", list(GRAPH_LAYERS))
@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_equal_eager(name, noalloc):
    spec = GRAPH_LAYERS[name]
    L = device_layer(spec)
    cfg = moe.config_for(spec, packed=True)
    W = moe.pack_layer(L)
    wt = moe.weights_struct(cfg, W)
    dev = L["x"].device
    xs = _inputs(spec, 4, dev)
    x_static = xs[0].clone()
    out = torch.empty((spec.T, spec.D), dtype=cfg.odtype, device=dev)

    def step():
        if noalloc:
            moe.layer_forward_noalloc(cfg, x_static, out, wt)
        else:
            moe.layer_forward(cfg, x_static, W, out=out, weights=wt)

    # warm up eagerly on a side stream (the usual order before a capture), then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for i, x in enumerate(xs):
        ref = moe.layer_forward(cfg, x, W, weights=wt)   # eager work between the replays
        torch.cuda.synchronize()
        x_static.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}: replay {i} differs from the eager call"
