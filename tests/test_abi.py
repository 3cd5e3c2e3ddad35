"""Host-side tests of the C ABI (no GPU): the library loads and exports every
function include/moe.h declares, status strings, workspace queries, and every
argument check that must fail before anything is enqueued."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import top_routed_expert_amd as moe
from top_routed_expert_amd import moe as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, UNSUP, WS, MISALIGNED, HIP = range(7)


def header_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def cfg(**kw) -> M.MoeConfig:
    c = dict(d_model=256, n_experts=16, top_k=4, d_expert=128, d_shared=128, dtype=moe.BF16, out_dtype=moe.BF16,
             weight_layout=moe.LAYOUT_ROWS)
    c.update(kw)
    return M.MoeConfig(**c)


FAKE = 0x10000  # aligned, never dereferenced: every call below fails its checks first


def test_exports_every_declared_function():
    L = moe.lib()
    names = header_functions()
    assert len(names) == 26, names
    for n in names:
        assert hasattr(L, n), f"libmoe.so does not export {n}"
    assert set(names) == set(M._SIGS), "binding signatures out of sync with the header"


def test_status_strings():
    L = moe.lib()
    seen = set()
    for s in range(7):
        txt = L.moe_status_string(s).decode()
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 7
    assert L.moe_status_string(99).decode() == "unknown status"


def test_workspace_queries():
    L = moe.lib()
    c = cfg()
    r = L.moe_route_workspace_bytes(ctypes.byref(c), 100)
    assert r >= 100 * 16 * 4
    p = L.moe_permute_workspace_bytes(ctypes.byref(c), 100)
    assert p >= 100 * 4 * 4 + 16 * 4
    f = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 16, 400, 128)
    assert f >= 400 * 128 * 2
    lay = L.moe_layer_workspace_bytes(ctypes.byref(c), 100)
    assert lay >= (100 * 4 + 100) * 256 * 4  # fp32 expert outputs of routed + shared rows
    assert L.moe_layer_workspace_bytes(ctypes.byref(c), 0) >= 0
    # monotone in T
    assert L.moe_layer_workspace_bytes(ctypes.byref(c), 1000) > lay
    bad = [cfg(top_k=17), cfg(n_experts=0), cfg(n_experts=2000), cfg(dtype=7), cfg(d_model=-1), cfg(top_k=65, n_experts=100)]
    for b in bad:
        assert L.moe_layer_workspace_bytes(ctypes.byref(b), 10) == M.SIZE_MAX
        assert L.moe_route_workspace_bytes(ctypes.byref(b), 10) == M.SIZE_MAX
    assert L.moe_layer_workspace_bytes(None, 10) == M.SIZE_MAX
    assert L.moe_layer_workspace_bytes(ctypes.byref(c), -1) == M.SIZE_MAX
    assert L.moe_layer_workspace_bytes(ctypes.byref(c), 1 << 30) == M.SIZE_MAX
    assert L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 0, 10, 128) == M.SIZE_MAX
    assert L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 4, 10, 0) == M.SIZE_MAX


def test_packed_weights_queries_and_checks():
    L = moe.lib()
    # n_mats * ceil(rows/16)*16 * cols * 2 bytes
    assert L.moe_packed_weights_bytes(1, 288, 4096) == 288 * 4096 * 2
    assert L.moe_packed_weights_bytes(3, 12, 64) == 3 * 16 * 64 * 2
    assert L.moe_packed_weights_bytes(0, 12, 64) == 0
    assert L.moe_packed_weights_bytes(1, 16, 48) == M.SIZE_MAX      # cols % 32 != 0
    assert L.moe_packed_weights_bytes(-1, 16, 64) == M.SIZE_MAX
    need = L.moe_packed_weights_bytes(2, 20, 64)
    call = lambda n=2, r=20, c=64, src=FAKE, dst=FAKE, nb=need: L.moe_pack_weights(n, r, c, src, dst, nb, None)
    assert call(c=40) == SHAPE
    assert call(n=0) == OK                      # nothing to pack
    assert call(src=None) == NULL
    assert call(dst=FAKE + 8) == MISALIGNED
    assert call(nb=need - 1) == WS and str(need) in _last()
    # packed layout needs bf16 and widths multiple of 64
    for bad in (cfg(weight_layout=3), cfg(weight_layout=moe.LAYOUT_PACKED, dtype=moe.F32),
                cfg(weight_layout=moe.LAYOUT_FP8, dtype=moe.F32), cfg(weight_layout=moe.LAYOUT_FP8, d_expert=96),
                cfg(weight_layout=moe.LAYOUT_PACKED, d_model=320 - 32), cfg(weight_layout=moe.LAYOUT_PACKED, d_expert=96)):
        assert L.moe_layer_workspace_bytes(ctypes.byref(bad), 10) == M.SIZE_MAX
    good = cfg(weight_layout=moe.LAYOUT_PACKED)
    assert L.moe_layer_workspace_bytes(ctypes.byref(good), 10) != M.SIZE_MAX
    ws = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(good), 4, 64, 96)
    assert L.moe_grouped_ffn(ctypes.byref(good), 4, 64, FAKE, FAKE, 64, None, FAKE, FAKE, FAKE, 96, FAKE, FAKE, ws,
                             None) == UNSUP and "64" in _last()
    assert moe.Config(256, 16, 4, 128, 128, packed=True).wshape(16, 256) == (16, 256)
    assert moe.Config(256, 12, 4, 128, 128, packed=True).wshape(12, 256) == (16, 256)
    assert moe.Config(256, 12, 4, 128, 128).wshape(12, 256) == (12, 256)


def _last():
    return moe.lib().moe_last_error().decode()


def test_route_checks():
    L = moe.lib()
    c = cfg()
    ws = L.moe_route_workspace_bytes(ctypes.byref(c), 8)
    call = lambda c_, T, x=FAKE, w=FAKE, b=None, i=FAKE, p=FAKE, g=None, wsp=FAKE, wsb=ws: \
        L.moe_route(c_, T, x, w, b, i, p, g, wsp, wsb, None)
    assert call(None, 8) == NULL and "cfg" in _last()
    assert call(ctypes.byref(cfg(top_k=20)), 8) == SHAPE
    assert call(ctypes.byref(cfg(dtype=3)), 8) == UNSUP
    assert call(ctypes.byref(cfg(n_experts=1025)), 8) == UNSUP
    assert call(ctypes.byref(c), -1) == SHAPE
    assert call(ctypes.byref(c), 0) == OK          # nothing to do, nothing enqueued
    assert call(ctypes.byref(c), 8, x=None) == NULL
    assert call(ctypes.byref(c), 8, i=None) == NULL
    assert call(ctypes.byref(c), 8, wsp=None) == NULL
    assert call(ctypes.byref(c), 8, x=FAKE + 8) == MISALIGNED
    assert call(ctypes.byref(c), 8, g=FAKE + 4) == MISALIGNED
    assert call(ctypes.byref(c), 8, wsb=ws - 1) == WS and str(ws) in _last()
    assert call(ctypes.byref(cfg(d_model=252)), 8) == UNSUP   # bf16 rows of 504 bytes


def test_permute_checks():
    L = moe.lib()
    c = cfg()
    ws = L.moe_permute_workspace_bytes(ctypes.byref(c), 8)
    call = lambda T, idx=FAKE, off=FAKE, st=FAKE, de=FAKE, x=None, xp=None, wsp=FAKE, wsb=ws: \
        L.moe_permute(ctypes.byref(c), T, idx, off, st, de, x, xp, wsp, wsb, None)
    assert call(0) == OK
    assert call(8, idx=None) == NULL
    assert call(8, x=FAKE) == NULL               # x without x_perm
    assert call(8, de=FAKE + 2) == MISALIGNED
    assert call(8, wsb=0) == WS
    assert call(-3) == SHAPE


def test_grouped_ffn_checks():
    L = moe.lib()
    c = cfg()
    ws = L.moe_grouped_ffn_workspace_bytes(ctypes.byref(c), 4, 64, 128)
    call = lambda G=4, rows=64, off=FAKE, x=FAKE, gat=None, d_ff=128, y=FAKE, wsb=ws: \
        L.moe_grouped_ffn(ctypes.byref(c), G, rows, off, x, 64, gat, FAKE, FAKE, FAKE, d_ff, y, FAKE, wsb, None)
    assert call(rows=0) == OK
    assert call(G=0) == SHAPE
    assert call(G=2000) == SHAPE
    assert call(d_ff=0) == SHAPE
    assert call(off=None) == NULL
    assert call(y=None) == NULL
    assert call(gat=FAKE + 4) == MISALIGNED
    assert call(d_ff=100) == UNSUP or call(d_ff=100) == WS   # bf16 rows need d_ff % 8 == 0
    assert call(d_ff=132) == UNSUP
    assert call(wsb=ws - 16) == WS


def test_expert_half_checks():
    L = moe.lib()
    c = cfg()
    ws = L.moe_expert_workspace_bytes(ctypes.byref(c), 5, 64, 128)
    assert ws != M.SIZE_MAX and L.moe_expert_workspace_bytes(ctypes.byref(c), 0, 64, 128) == M.SIZE_MAX
    gu = lambda n_gather=0, gat=None, sg=None, su=None, wsb=ws, rows=64: L.moe_expert_gate_up(
        ctypes.byref(c), 4, rows, FAKE, FAKE, 64, gat, n_gather, FAKE, FAKE, sg, su, 128, FAKE, FAKE, wsb, None)
    assert gu(rows=0) == OK
    assert gu(n_gather=8) == NULL                 # gather required when n_gather > 0
    assert gu(n_gather=65, gat=FAKE) == SHAPE     # n_gather > n_rows
    assert gu(sg=FAKE) == NULL                    # s_gate without s_up
    assert gu(sg=FAKE, su=FAKE + 4) == MISALIGNED
    assert gu(sg=FAKE, su=FAKE, wsb=L.moe_expert_workspace_bytes(ctypes.byref(c), 5, 64, 128) - 1) == WS
    dn = lambda sd=None, y=FAKE, wsb=ws: L.moe_expert_down(ctypes.byref(c), 4, 64, FAKE, FAKE, FAKE, sd, 128, y,
                                                           FAKE, wsb, None)
    assert dn(y=None) == NULL
    assert dn(sd=FAKE + 2) == MISALIGNED
    assert dn(wsb=16) == WS


def test_combine_and_layer_checks():
    L = moe.lib()
    c = cfg()
    assert L.moe_combine(ctypes.byref(c), 0, FAKE, FAKE, FAKE, None, FAKE, None) == OK
    assert L.moe_combine(ctypes.byref(c), 4, None, FAKE, FAKE, None, FAKE, None) == NULL
    assert L.moe_combine(ctypes.byref(c), 4, FAKE, FAKE, FAKE, FAKE + 12, FAKE, None) == MISALIGNED
    ws = L.moe_layer_workspace_bytes(ctypes.byref(c), 8)
    w = M.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    call = lambda T=8, cc=c, ww=w, wsb=ws: L.moe_layer_forward(ctypes.byref(cc), T, FAKE, ctypes.byref(ww), FAKE,
                                                               None, None, None, FAKE, wsb, None)
    assert call(T=0) == OK
    assert call(wsb=ws - 1) == WS
    assert L.moe_layer_forward(ctypes.byref(c), 8, FAKE, None, FAKE, None, None, None, FAKE, ws, None) == NULL
    no_shared = M.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    assert call(ww=no_shared) == NULL and "d_shared" in _last()
    no_router = M.MoeWeights(None, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(ww=no_router) == NULL
    bad_bias = M.MoeWeights(FAKE, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert call(ww=bad_bias) == MISALIGNED
    c0 = cfg(d_shared=0)
    ws0 = L.moe_layer_workspace_bytes(ctypes.byref(c0), 8)
    assert call(cc=c0, ww=no_shared, wsb=ws0 - 1) == WS   # no shared expert: its weights may be NULL


def test_noalloc_layer_checks():
    """moe_layer_forward_noalloc: every check fails before the device is touched; a layer whose
    workspace exceeds the static scratch is refused."""
    L = moe.lib()
    c = cfg()
    assert L.moe_noalloc_scratch_bytes() == 64 << 20
    w = M.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    call = lambda T=8, cc=c, ww=w, x=FAKE, out=FAKE: L.moe_layer_forward_noalloc(
        ctypes.byref(cc), T, x, ctypes.byref(ww), out, None, None, None, None)
    assert call(T=0) == OK
    assert L.moe_layer_forward_noalloc(None, 8, FAKE, ctypes.byref(w), FAKE, None, None, None, None) == NULL
    assert call(T=-1) == SHAPE
    assert call(x=None) == NULL and call(out=None) == NULL
    assert call(ww=M.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)) == NULL
    assert call(x=FAKE + 8) == MISALIGNED
    big = cfg(d_model=4096, n_experts=288, top_k=8, d_expert=1280, d_shared=1280)
    T = 1024
    assert L.moe_layer_workspace_bytes(ctypes.byref(big), T) > L.moe_noalloc_scratch_bytes()
    assert call(T=T, cc=big) == WS and "static scratch" in _last()
    if not torch.cuda.is_available():   # valid arguments: the device query is the first HIP call
        assert call() == HIP and "static scratch" in _last()


def test_binding_rejects_host_tensors():
    c = moe.Config(256, 16, 4, 128, 128, torch.bfloat16)
    x = torch.zeros(8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        moe.route(c, x, torch.zeros(16, 256, dtype=torch.bfloat16))


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB_PATH", os.path.join(ROOT, "does_not_exist", "libmoe.so"))
    with pytest.raises(RuntimeError, match="missing"):
        M.lib()


def test_dynamic_and_expert_parallel_entry_checks():
    """Argument checks of the dynamic-top-k, group-statistics, receive-plan and row-gather entry points."""
    L = moe.lib()
    c = cfg()
    ws = L.moe_route_workspace_bytes(ctypes.byref(c), 8)
    # dynamic router: a misaligned per-token count array is refused, T = 0 is a no-op
    assert L.moe_route_dynamic(ctypes.byref(c), 8, FAKE, FAKE, None, FAKE + 4, FAKE, FAKE, None, FAKE, ws,
                               None) == MISALIGNED
    assert L.moe_route_dynamic(ctypes.byref(c), 0, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, ws, None) == OK
    lw = L.moe_layer_workspace_bytes(ctypes.byref(c), 8)
    wts = M.MoeWeights()
    assert L.moe_layer_forward_dynamic(ctypes.byref(c), 8, FAKE, ctypes.byref(wts), None, FAKE, None, None, None,
                                       FAKE, lw, None) == NULL
    # group statistics: G must divide E and lie in [1, 16]
    assert L.moe_route_group_stats_workspace_bytes(ctypes.byref(c), 8, 3) == M.SIZE_MAX   # 16 % 3
    assert L.moe_route_group_stats_workspace_bytes(ctypes.byref(c), 8, 0) == M.SIZE_MAX
    gw = L.moe_route_group_stats_workspace_bytes(ctypes.byref(c), 8, 4)
    assert gw >= ws + 8 * 4 * 4
    gcall = lambda G=4, st=FAKE, wsb=gw: L.moe_route_group_stats(ctypes.byref(c), 8, FAKE, FAKE, None, None, G, FAKE,
                                                                   FAKE, st, FAKE, wsb, None)
    assert gcall(G=32) == SHAPE
    assert gcall(st=None) == NULL
    assert gcall(wsb=gw - 1) == WS
    # receive plan: at most 1024 chunks, a bounded row capacity, every output present
    plan = lambda ns=8, nl=36, cnt=FAKE, mx=100, off=FAKE, ga=FAKE, sc=FAKE: \
        L.moe_ep_receive_plan(ns, nl, cnt, mx, off, ga, sc, None)
    assert plan(ns=32, nl=33) == SHAPE
    assert plan(ns=0) == SHAPE
    assert plan(mx=-1) == SHAPE and plan(mx=1 << 31) == SHAPE
    assert plan(ga=None) == NULL and plan(cnt=None) == NULL
    assert plan(sc=FAKE + 4) == MISALIGNED
    # row gather
    gat = lambda src=FAKE, ns=10, rb=64, idx=FAKE, n=5, dst=FAKE: L.moe_gather_rows(src, ns, rb, idx, n, dst, None)
    assert gat(rb=0) == SHAPE and gat(n=-1) == SHAPE and gat(ns=0) == SHAPE
    assert gat(n=0, src=None) == OK
    assert gat(idx=None) == NULL and gat(dst=FAKE + 2) == MISALIGNED


def test_fp8_queries_and_checks():
    L = moe.lib()
    # n_mats * ceil(rows/16)*16 * cols bytes, cols a multiple of 64
    assert L.moe_fp8_weights_bytes(288, 1280, 4096) == 288 * 1280 * 4096
    assert L.moe_fp8_weights_bytes(2, 20, 64) == 2 * 32 * 64
    assert L.moe_fp8_weights_bytes(1, 16, 96) == M.SIZE_MAX and L.moe_fp8_weights_bytes(-1, 16, 64) == M.SIZE_MAX
    need = L.moe_fp8_weights_bytes(2, 20, 64)
    call = lambda n=2, r=20, c=64, src=FAKE, dst=FAKE, nb=need, sc=FAKE: \
        L.moe_quantize_fp8(n, r, c, src, dst, nb, sc, None)
    assert call(c=96) == SHAPE and call(r=-1) == SHAPE
    assert call(n=0) == OK
    assert call(sc=None) == NULL and call(src=None) == NULL
    assert call(dst=FAKE + 8) == MISALIGNED
    assert call(nb=need - 1) == WS and str(need) in _last()
    # fp8 weights reach the kernels only through the layer (which takes their scales)
    f8 = cfg(weight_layout=moe.LAYOUT_FP8)
    assert L.moe_layer_workspace_bytes(ctypes.byref(f8), 10) != M.SIZE_MAX
    ws = L.moe_expert_workspace_bytes(ctypes.byref(f8), 4, 64, 128)
    assert L.moe_expert_gate_up(ctypes.byref(f8), 4, 64, FAKE, FAKE, 64, None, 0, FAKE, FAKE, None, None, 128, FAKE,
                                FAKE, ws, None) == UNSUP and "fp8" in _last()
    lw = L.moe_layer_workspace_bytes(ctypes.byref(f8), 8)
    w = M.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)   # scales missing
    assert L.moe_layer_forward(ctypes.byref(f8), 8, FAKE, ctypes.byref(w), FAKE, None, None, None, FAKE, lw,
                               None) == NULL and "scale" in _last()
    w = M.MoeWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4)
    assert L.moe_layer_forward(ctypes.byref(f8), 8, FAKE, ctypes.byref(w), FAKE, None, None, None, FAKE, lw,
                               None) == MISALIGNED
