"""Packed weight layout on the GPU: moe_pack_weights writes the layout that
include/moe.h documents, and every entry point gives bit-identical results
with packed and with row-major weights (the kernels load the same values
into the same operand registers, so nothing but the addressing changes)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
import top_routed_expert_amd as moe
from moe_testutil import device_layer
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def pack_reference(w: np.ndarray) -> np.ndarray:
    """The documented layout, on the host: 16 x 32 fragments, ct-major then kb;
    lane l = c + 16q of fragment (ct, kb) holds W[16ct + c][32kb + 8q .. +8]."""
    n, rows, cols = w.shape
    R = (rows + 15) // 16 * 16
    wp = np.zeros((n, R, cols), dtype=w.dtype)
    wp[:, :rows] = w
    v = wp.reshape(n, R // 16, 16, cols // 32, 4, 8)  # n, ct, c, kb, q, e
    return v.transpose(0, 1, 3, 4, 2, 5).reshape(n, R, cols)  # n, ct, kb, (q, c) = lane, e


@pytest.mark.parametrize("shape", [(3, 20, 64), (1, 288, 128), (2, 16, 32), (1, 1, 96)])
def test_pack_layout(shape):
    g = torch.Generator().manual_seed(sum(shape))
    w = torch.randn(shape, generator=g).to(torch.bfloat16)
    p = moe.pack_weights(w.cuda())
    torch.cuda.synchronize()
    got = p.cpu().view(torch.int16).numpy()
    want = pack_reference(w.view(torch.int16).numpy())
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    # a 2-D matrix packs like a stack of one
    p2 = moe.pack_weights(w[0].cuda())
    assert torch.equal(p2.cpu(), p[0].cpu())


PACKABLE = {k: v for k, v in SMALL.items()
            if v.dtype == "bf16" and v.D % 64 == 0 and v.F % 64 == 0 and v.Fs % 64 == 0}
PACKABLE["bf16_router_rows_padded"] = synth.spec("tiny", T=50, D=256, E=12, K=3, F=128, Fs=128, dtype="bf16",
                                                 seed=13)


def _layer_both(spec, L):
    rows = moe.layer_forward(moe.config_for(spec), L["x"], L, routing=True)
    packed = moe.layer_forward(moe.config_for(spec, packed=True), L["x"], moe.pack_layer(L), routing=True)
    torch.cuda.synchronize()
    return rows, packed


@pytest.mark.parametrize("name", list(PACKABLE))
def test_packed_layer_equals_rows(name):
    spec = PACKABLE[name]
    rows, packed = _layer_both(spec, device_layer(spec))
    for what, a, b in zip(("out", "topk_idx", "topk_prob", "offsets"), rows, packed):
        assert torch.equal(a, b), f"{name}: {what} differs between packed and row-major weights"


def test_packed_entry_points_equal_rows():
    spec = PACKABLE["bf16_tiles128"]
    L = device_layer(spec)
    P = moe.pack_layer(L)
    cr, cp = moe.config_for(spec), moe.config_for(spec, packed=True)
    ir, pr = moe.route(cr, L["x"], L["w_router"], L["bias"])
    ip, pp = moe.route(cp, L["x"], P["w_router"], P["bias"])
    assert torch.equal(ir, ip) and torch.equal(pr, pp)
    offs, st, dest = moe.permute(cr, ir)
    yr = moe.grouped_ffn(cr, offs, L["x"], L["w_gate"], L["w_up"], L["w_down"], gather=st)
    yp = moe.grouped_ffn(cp, offs, L["x"], P["w_gate"], P["w_up"], P["w_down"], gather=st)
    assert torch.equal(yr, yp)
    # the two halves with the shared expert as the extra group
    T, E = spec.T, spec.E
    offs_ext = torch.cat([offs, offs[-1:] + T])
    n_rows = T * spec.K + T
    hr = moe.expert_gate_up(cr, offs_ext, L["x"], L["w_gate"], L["w_up"], gather=st, n_rows=n_rows,
                            s_gate=L["s_gate"], s_up=L["s_up"])
    hp = moe.expert_gate_up(cp, offs_ext, L["x"], P["w_gate"], P["w_up"], gather=st, n_rows=n_rows,
                            s_gate=P["s_gate"], s_up=P["s_up"])
    assert torch.equal(hr, hp)
    dr = moe.expert_down(cr, offs_ext, hr, L["w_down"], s_down=L["s_down"])
    dp = moe.expert_down(cp, offs_ext, hp, P["w_down"], s_down=P["s_down"])
    torch.cuda.synchronize()
    assert torch.equal(dr, dp)
    assert E == offs.shape[0] - 1


@pytest.mark.parametrize("name", ["decode", "prefill", "skew"])
def test_packed_full_size_equals_rows(name):
    spec = synth.spec(name)
    print(f"packed vs row-major, full size: {name}", flush=True)
    rows, packed = _layer_both(spec, device_layer(spec))
    for what, a, b in zip(("out", "topk_idx", "topk_prob", "offsets"), rows, packed):
        assert torch.equal(a, b), f"{name}: {what} differs between packed and row-major weights"
