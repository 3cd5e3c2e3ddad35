"""Benchmark of one sparse-MoE FFN layer (Step 3.5 Flash shape) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skew|full|tiny]

A step is one moe_layer_forward over one batch of synthetic tokens already
resident in HBM: router linear + softmax + top-8, permutation, routed and
shared expert SwiGLU FFNs, weighted combine. The timed region holds exactly
K steps; each step is bracketed by HIP events on the stream the library
launches on, with a 512 MiB write between steps (outside the events) so the
256 MiB Infinity Cache does not keep the previous step's experts.

One JSON line is printed. The headline (value, ms_per_step, config) is the
--workload (default: decode, T=32). Besides it the line carries:
  roofline      the dominant kernel (expert gate/up projection with the
                SwiGLU epilogue, timed alone through moe_expert_gate_up with
                the layer's exact arguments): algorithmic bytes or flops per
                launch / average launch time, against the MI355X peak;
  cpu_baseline  the CPU oracle timed on bounded samples of the decode and
                prefill batches (expert weights copied to host before timing);
  workloads     the other four named workloads (tiny, prefill, skew, full
                width) measured the same way, each with its own roofline; the
                full-width entry carries the per-group activation counts of
                the 8 x 36 expert groups and the Expert Activation Skew;
  measured_peaks what plain library work reaches on this GPU (a 2 GiB
                device copy, an 8192^3 bf16 torch.matmul); MFMA-bound
                rooflines also give frac_of_vendor_gemm, their rate over
                that matmul's.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 MI355X; % bf16 MFMA peak (prefill) / % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X fp32 vector, TFLOP/s
FLUSH_BYTES = 512 << 20


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "top_routed_expert_amd", "csrc", f)
                  for f in ("grouped_gemm.hip", "grouped_gemm_big8.hip", "moe_internal.h")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the gate/up kernel from the committed PMC summary.

    The summary holds lines `source_sha256: <hash>` and
    `traffic_bytes[<workload>]: <bytes>`; the figure is used only while the
    kernel sources still hash the same (else null: the kernel changed since
    the counters were taken).
    """
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    import re
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes\[%s\]:\s*([0-9.eE+]+)" % re.escape(workload), text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return int(float(t.group(1)))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "prefill", "skew", "full"])
    ap.add_argument("--no-secondary", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32, help="decode tokens in the CPU sample")
    ap.add_argument("--cpu-prefill-tokens", type=int, default=256, help="prefill tokens in the CPU sample")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="fp8 (E4M3) vs bf16 expert weights at decode and prefill, one JSON line each")
    ap.add_argument("--ep-share", action="store_true",
                    help="one GPU's expert-parallel share (36 experts, 8 ranks x 8192 tokens), one JSON line")
    ap.add_argument("--dynamic-k", action="store_true",
                    help="dynamic top-k (4 or 8 per token) vs fixed top-8 at decode and prefill, one JSON line each")
    ap.add_argument("--sweep", action="store_true",
                    help="token-count sweep T = 1 .. 16384 at the decode/prefill shape (one JSON line per T)")
    ap.add_argument("--layout", default="packed", choices=["packed", "rows"],
                    help="weight layout the timed steps read (bf16 layers; converted once before timing)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 1 GiB device-to-device copy: the known-size reference for HBM byte counters")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the markdown summary of a rocprofv3 --kernel-trace --stats run (csv, -o run) in DIR "
                         "to --out, with --title and --command; no GPU needed")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="write the gate/up HBM traffic summary from rocprofv3 --pmc runs in DIR/pmc_<workload>_"
                         "<FETCH_SIZE|WRITE_SIZE> (csv, -o run) to --out; no GPU needed")
    ap.add_argument("--counters-workload", default="prefill", choices=["prefill", "decode"],
                    help="which expert GEMM kernels --summarize-counters reports")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write the SQ / L2 counter summary of the 256x256 expert GEMMs from rocprofv3 --pmc runs "
                         "in DIR/<pass> (csv, -o run; passes listed in COUNTER_PASSES) and the kernel trace in "
                         "DIR/trace to --out; no GPU needed")
    ap.add_argument("--out")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="")
    return ap.parse_args()


class Flusher:
    def __init__(self, enabled: bool):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if enabled else None
        self.i = 0

    def __call__(self):
        if self.buf is not None:
            self.i += 1
            self.buf.fill_(float(self.i))


def timed(fn, steps: int, warmup: int, flush: Flusher):
    """Run fn warmup times, then time `steps` calls with HIP events; returns per-call ms list and wall s."""
    import torch
    for _ in range(warmup):
        flush()
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall


def layer_flops_bytes(spec, counts):
    """Algorithmic flops and HBM bytes of one layer call (touched experts only)."""
    import numpy as np
    T, D, E, K, F, Fs = spec.T, spec.D, spec.E, spec.K, spec.F, spec.Fs
    es = 2 if spec.dtype == "bf16" else 4
    touched = int((np.asarray(counts) > 0).sum())
    pairs = int(np.asarray(counts).sum())  # T*K, or fewer under dynamic top-k
    flops = 2 * T * D * E + 2 * pairs * 3 * D * F + 2 * T * 3 * D * Fs
    wbytes = (touched * 3 * D * F + 3 * D * Fs + E * D) * es
    abytes = T * D * es * 2  # x in, out
    return flops, wbytes + abytes, touched


# tile-height thresholds of the expert GEMMs, in mean rows per group (as gemm_block_rows in
# csrc/grouped_gemm.hip and the 256x256 launcher in csrc/grouped_gemm_big8.hip)
ROWS_32, ROWS_256, ROWS_256_SKIP = 24, 48, 160


def gate_up_kernel(rows: int, groups: int, packed: bool) -> str:
    """Name of the gate/up kernel the library picks for `rows` rows over `groups` groups (bf16)."""
    if rows <= ROWS_32 * groups:
        return "gemm_bf16_mfma<EPI_SWIGLU>, 32-row tiles"
    if rows >= ROWS_256 * groups:
        skip = packed and rows < ROWS_256_SKIP * groups
        return "gemm_bf16_big8<EPI_SWIGLU%s>, 256x256 tiles, 8 waves" % (", skipping empty half items" if skip else "")
    return "gemm_bf16_mfma<EPI_SWIGLU>, 64-row tiles"


def roofline(k_bytes: int, k_flops: int, k_ms: float, peak_tf: float, prefer: str | None = None) -> dict:
    """Roofline entry of one kernel: bound = the larger roofline time (or `prefer`), both fractions reported."""
    gbs = k_bytes / (k_ms * 1e-3) / 1e9
    tfs = k_flops / (k_ms * 1e-3) / 1e12
    bound = prefer or ("hbm" if k_bytes / (HBM_PEAK_GBS * 1e9) >= k_flops / (peak_tf * 1e12) else "mfma")
    if bound == "hbm":
        r = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        r = dict(bound="mfma", achieved=round(tfs, 1), peak=peak_tf, unit="TFLOP/s", frac=round(tfs / peak_tf, 4))
    r.update(launch_ms=round(k_ms, 4), algorithmic_bytes=int(k_bytes), algorithmic_flops=int(k_flops),
             intensity_flop_per_byte=round(k_flops / k_bytes, 1), mfma_frac=round(tfs / peak_tf, 4),
             hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
    return r


def measure(spec, steps, warmup, flush_on, packed=True):
    """The layer and its dominant kernel on one workload: a dict with the layer's timing, the work
    accounting of this batch's routing, and the gate/up kernel's roofline entry."""
    import numpy as np
    import torch

    import synth
    import top_routed_expert_amd as moe

    L = synth.make_layer(spec, "cuda")
    packed = packed and spec.dtype == "bf16"
    cfg = moe.config_for(spec, packed=packed)
    # weights are converted once, as at load time; the timed steps read only the packed copy
    W = moe.pack_layer(L) if packed else L
    torch.cuda.synchronize()
    flush = Flusher(flush_on)
    dev = L["x"].device
    T, D, E, K, F = spec.T, spec.D, spec.E, spec.K, spec.F
    # --- whole layer -------------------------------------------------------
    ws = moe.Workspace(cfg, T, dev)
    wt = moe.weights_struct(cfg, W)
    out = torch.empty((T, D), dtype=cfg.odtype, device=dev)
    layer = lambda: moe.layer_forward(cfg, L["x"], W, out=out, workspace=ws, weights=wt)
    ms, wall = timed(layer, steps, warmup, flush)
    ms_step = float(np.mean(ms))
    # routing of this batch (outside the timed region) for the work accounting
    idx, prob = moe.route(cfg, L["x"], W["w_router"], L["bias"])
    offs, st, dest = moe.permute(cfg, idx)
    counts = np.diff(offs.cpu().numpy())
    flops, nbytes, touched = layer_flops_bytes(spec, counts)
    es = 2 if spec.dtype == "bf16" else 4
    peak_tf = MFMA_BF16_PEAK_TFLOPS if spec.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    res = dict(ms=ms_step, ms_min=float(np.min(ms)), wall=wall, tokens_per_s=T / (ms_step * 1e-3),
               touched=touched, layer_tflops=flops / (ms_step * 1e-3) / 1e12,
               layer_gbs=nbytes / (ms_step * 1e-3) / 1e9, skew=float(counts.max() / counts.mean()),
               layer_flops=flops, layer_bytes=nbytes, counts=counts, peak_tf=peak_tf)
    # --- dominant kernel: expert gate/up + SwiGLU, the layer's own arguments -
    P = T * K
    fused = spec.Fs == spec.F and spec.Fs > 0
    offs_ext = torch.cat([offs, torch.tensor([P + T], dtype=torch.int32, device=dev)]) if fused else offs
    n_rows = P + (T if fused else 0)
    h = torch.empty((n_rows, F), dtype=cfg.dtype, device=dev)
    gws = torch.empty(moe.lib().moe_expert_workspace_bytes(
        __import__("ctypes").byref(cfg.c()), E + (1 if fused else 0), n_rows, F), dtype=torch.uint8, device=dev)
    gate_up = lambda: moe.expert_gate_up(cfg, offs_ext, L["x"], W["w_gate"], W["w_up"], gather=st, n_rows=n_rows,
                                         s_gate=W["s_gate"] if fused else None, s_up=W["s_up"] if fused else None,
                                         h=h, ws=gws)
    kms, _ = timed(gate_up, steps, warmup, flush)
    k_ms = float(np.mean(kms))
    k_experts = touched + (1 if fused else 0)
    k_bytes = k_experts * 2 * F * D * es + T * D * es + n_rows * F * es
    k_flops = 2 * n_rows * 2 * F * D
    # the prefill-shaped workloads are judged by their matrix-core fraction (their gate/up intensity,
    # 245-500 flop/B, sits near or above the 312 flop/B ridge); decode by its HBM fraction
    prefer = "mfma" if spec.dtype == "bf16" and n_rows >= ROWS_256 * k_experts else None
    roof = roofline(k_bytes, k_flops, k_ms, peak_tf, prefer)
    kname = gate_up_kernel(n_rows, k_experts, packed) if spec.dtype == "bf16" else "gemm_generic<EPI_SWIGLU>"
    roof.update(traffic=measured_traffic(spec.name), kernel=kname + " (expert gate/up + SwiGLU)",
                experts_read=k_experts)
    res["roofline"] = roof
    res["L"] = L
    res["layout"] = "packed" if packed else "rows"
    del W
    return res


def workload_entry(spec, r: dict) -> dict:
    """JSON entry of one workload's measurement (everything but the headline fields)."""
    import numpy as np

    e = {"workload": spec.name, "tokens": spec.T, "d_model": spec.D, "routed_experts": spec.E, "top_k": spec.K,
         "d_expert": spec.F, "d_shared": spec.Fs, "dtype": "bf16" if spec.dtype == "bf16" else "f32",
         "router_bias": "zipf" if spec.skew else "none", "weight_layout": r["layout"],
         "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "ms_per_step": round(r["ms"], 5),
         "ms_min": round(r["ms_min"], 5), "layer_tflops": round(r["layer_tflops"], 2),
         "layer_mfma_frac": round(r["layer_tflops"] / r["peak_tf"], 4), "layer_gbs": round(r["layer_gbs"], 1),
         "layer_hbm_frac": round(r["layer_gbs"] / HBM_PEAK_GBS, 4), "experts_touched": r["touched"],
         "roofline": r["roofline"]}
    # Expert Activation Skew: the largest expert's pair count over the mean count of all E experts
    c = np.asarray(r["counts"], dtype=np.int64)
    e["expert_activation_skew"] = round(float(c.max() / c.mean()), 3)
    if spec.groups:  # pairs per group of E/G consecutive experts
        e["group_counts"] = [int(v) for v in c.reshape(spec.groups, -1).sum(axis=1)]
    return e


SWEEP_T = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]


def tile_kernel(T, spec):
    """Row tiles the expert GEMMs use for T tokens (mean rows per group decides), as the library picks."""
    rows, groups = T * spec.K + (T if spec.Fs == spec.F else 0), spec.E + (1 if spec.Fs == spec.F else 0)
    if rows <= ROWS_32 * groups:
        return 32
    return 256 if rows >= ROWS_256 * groups else 64


def sweep(steps, warmup, flush_on):
    """Token-count sweep of the layer at the decode/prefill shape (same weights): one JSON line per T."""
    import dataclasses

    import numpy as np
    import torch

    import synth
    import top_routed_expert_amd as moe

    base = synth.spec("prefill", T=max(SWEEP_T))
    L = synth.make_layer(base, "cuda")
    cfg = moe.config_for(base, packed=True)
    W = moe.pack_layer(L)
    dev = L["x"].device
    ws = moe.Workspace(cfg, max(SWEEP_T), dev)
    wt = moe.weights_struct(cfg, W)
    flush = Flusher(flush_on)
    for T in SWEEP_T:
        spec = dataclasses.replace(base, T=T)
        x = L["x"][:T]
        out = torch.empty((T, base.D), dtype=cfg.odtype, device=dev)
        ms, _ = timed(lambda: moe.layer_forward(cfg, x, W, out=out, workspace=ws, weights=wt), steps, warmup, flush)
        ms_step = float(np.mean(ms))
        idx, _ = moe.route(cfg, x, W["w_router"], L["bias"])
        offs, _, _ = moe.permute(cfg, idx)
        counts = np.diff(offs.cpu().numpy())
        flops, nbytes, touched = layer_flops_bytes(spec, counts)
        print(json.dumps({"T": T, "ms_per_step": round(ms_step, 5), "ms_min": round(float(np.min(ms)), 5),
                          "tokens_per_s": round(T / (ms_step * 1e-3), 1),
                          "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
                          "mfma_frac": round(flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
                          "hbm_frac": round(nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "experts_touched": touched, "tile_rows": tile_kernel(T, spec)}), flush=True)


def fp8_weights(steps, warmup, flush_on):
    """FP8 (E4M3, per-row scales) expert weights against bf16 at the decode and prefill workloads: one
    JSON line per (workload, weights), whole-layer figures; bytes count the weights as stored."""
    import numpy as np
    import torch

    import synth
    import top_routed_expert_amd as moe

    for name in ("decode", "prefill"):
        spec = synth.spec(name)
        L = synth.make_layer(spec, "cuda")
        dev = L["x"].device
        T, D, E, F, Fs = spec.T, spec.D, spec.E, spec.F, spec.Fs
        for mode in ("bf16", "fp8"):
            cfg = moe.config_for(spec, packed=True, fp8=(mode == "fp8"))
            W = moe.quantize_layer(L) if mode == "fp8" else moe.pack_layer(L)
            ws = moe.Workspace(cfg, T, dev)
            wt = moe.weights_struct(cfg, W)
            out = torch.empty((T, D), dtype=cfg.odtype, device=dev)
            ms, _ = timed(lambda: moe.layer_forward(cfg, L["x"], W, out=out, workspace=ws, weights=wt),
                          steps, warmup, Flusher(flush_on))
            ms_step = float(np.mean(ms))
            idx, _ = moe.route(cfg, L["x"], W["w_router"], L["bias"])
            offs, _, _ = moe.permute(cfg, idx)
            counts = np.diff(offs.cpu().numpy())
            flops, nbytes, touched = layer_flops_bytes(spec, counts)
            if mode == "fp8":  # expert matrices at 1 byte per weight plus one fp32 scale per row
                ex = touched * (2 * F + D) + (2 * Fs + D)
                nbytes -= (touched * 3 * D * F + 3 * D * Fs) * 2
                nbytes += (touched * 3 * D * F + 3 * D * Fs) + ex * 4
            print(json.dumps({"workload": name, "T": T, "weights": mode, "ms_per_step": round(ms_step, 5),
                              "tokens_per_s": round(T / (ms_step * 1e-3), 1), "experts_touched": touched,
                              "bytes": int(nbytes), "gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
                              "hbm_frac": round(nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "mfma_frac": round(flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}),
                  flush=True)
            del W, ws, wt
            torch.cuda.empty_cache()
        del L
        torch.cuda.empty_cache()


def dynamic_topk(steps, warmup, flush_on):
    """Dynamic top-k (4 or 8 experts per token, seeded, about half each) against fixed top-8 at the
    decode and prefill workloads: one JSON line per (workload, mode), whole-layer figures."""
    import numpy as np
    import torch

    import synth
    import top_routed_expert_amd as moe

    for name in ("decode", "prefill"):
        spec = synth.spec(name)
        L = synth.make_layer(spec, "cuda")
        cfg = moe.config_for(spec, packed=True)
        W = moe.pack_layer(L)
        del L["w_gate"], L["w_up"], L["w_down"]
        dev = L["x"].device
        ws = moe.Workspace(cfg, spec.T, dev)
        wt = moe.weights_struct(cfg, W)
        out = torch.empty((spec.T, spec.D), dtype=cfg.odtype, device=dev)
        flush = Flusher(flush_on)
        k_dyn = synth.dynamic_k(spec, device=dev)
        for mode, k in (("fixed top-8", None), ("dynamic top-4/8", k_dyn)):
            ms, _ = timed(lambda: moe.layer_forward(cfg, L["x"], W, out=out, workspace=ws, weights=wt,
                                                    k_per_token=k), steps, warmup, flush)
            ms_step = float(np.mean(ms))
            idx, _ = moe.route(cfg, L["x"], W["w_router"], L["bias"], k_per_token=k)
            offs, _, _ = moe.permute(cfg, idx)
            counts = np.diff(offs.cpu().numpy())
            flops, nbytes, touched = layer_flops_bytes(spec, counts)
            print(json.dumps({"workload": name, "T": spec.T, "mode": mode, "pairs": int(counts.sum()),
                              "ms_per_step": round(ms_step, 5), "tokens_per_s": round(spec.T / (ms_step * 1e-3), 1),
                              "experts_touched": touched,
                              "mfma_frac": round(flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "hbm_frac": round(nbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
        del W, L, ws
        torch.cuda.empty_cache()


def ep_share(steps, warmup, flush_on, n_src=8, n_groups=8, group=0):
    """One GPU's share under expert parallelism at the prefill shape: 8 source ranks x 8192 tokens
    route and permute their own tokens; group 0's 36 experts run on the rows they would send it
    (receive plan, gate/up on the receive buffer in place, down, outputs back in receive order).
    One JSON line; the per-group balance statistics of the same routing are reported beside it."""
    import numpy as np
    import torch

    import synth
    import top_routed_expert_amd as moe

    spec = synth.spec("prefill", T=n_src * 8192)
    L = synth.make_layer(spec, "cuda")
    cfg = moe.config_for(spec, packed=True)
    W = moe.pack_layer(L)
    del L["w_gate"], L["w_up"], L["w_down"]
    Tl, El = spec.T // n_src, spec.E // n_groups
    idx, _, stats = moe.route_group_stats(cfg, L["x"], W["w_router"], n_groups, L["bias"])
    chunks, counts = [], []
    for r in range(n_src):
        sl = slice(r * Tl, (r + 1) * Tl)
        offs, _, _, xp = moe.permute(cfg, idx[sl].contiguous(), L["x"][sl].contiguous())
        oh = offs.cpu().numpy().astype(np.int64)
        chunks.append(xp[oh[group * El]:oh[(group + 1) * El]])
        counts.append(np.diff(oh)[group * El:(group + 1) * El])
        del xp
    recv = torch.cat(chunks).contiguous()
    del chunks
    n = recv.shape[0]
    cnt = torch.from_numpy(np.stack(counts).astype(np.int32)).cuda()
    local = moe.Config(spec.D, El, spec.K, spec.F, 0, cfg.dtype, cfg.out_dtype, True)
    sl = slice(group * El, (group + 1) * El)
    wg, wu, wd = W["w_gate"][sl], W["w_up"][sl], W["w_down"][sl]
    h = torch.empty((n, spec.F), dtype=cfg.dtype, device="cuda")
    y = torch.empty((n, spec.D), dtype=torch.float32, device="cuda")
    y_recv = torch.empty_like(y)
    gws = torch.empty(moe.lib().moe_expert_workspace_bytes(__import__("ctypes").byref(local.c()), El, n, spec.F),
                      dtype=torch.uint8, device="cuda")
    plan = {}

    def share():
        plan["p"] = moe.ep_receive_plan(cnt, n)
        offsets, gather, scatter = plan["p"]
        moe.expert_gate_up(local, offsets, recv, wg, wu, gather=gather, n_rows=n, h=h, ws=gws)
        moe.expert_down(local, offsets, h, wd, y=y, ws=gws)
        moe.gather_rows(y, scatter, out=y_recv)

    flush = Flusher(flush_on)
    ms, _ = timed(share, steps, warmup, flush)
    offsets, gather, _ = plan["p"]
    gemm = lambda: (moe.expert_gate_up(local, offsets, recv, wg, wu, gather=gather, n_rows=n, h=h, ws=gws),
                    moe.expert_down(local, offsets, h, wd, y=y, ws=gws))
    gms, _ = timed(gemm, steps, warmup, flush)
    ms_step, g_ms = float(np.mean(ms)), float(np.mean(gms))
    flops = 2 * n * 3 * spec.D * spec.F
    st = stats.cpu().numpy()
    f, pg = st[n_groups:] / st[n_groups:].sum(), st[:n_groups] / spec.T
    return dict(workload=f"ep share: group {group} of {n_groups} ({El} experts), {n_src} ranks x {Tl} tokens",
                rows=n, rows_per_expert=round(n / El, 1), ms_per_step=round(ms_step, 5),
                rows_per_s=round(n / (ms_step * 1e-3), 1), gemm_ms=round(g_ms, 5),
                gemm_tflops=round(flops / (g_ms * 1e-3) / 1e12, 1),
                gemm_mfma_frac=round(flops / (g_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                share_mfma_frac=round(flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                l_ep=round(float(n_groups * np.sum(f * pg)), 5),
                group_pair_fraction=[round(float(v), 5) for v in f])


CPU_BASELINE_MIN_S = 10.0  # repeat whole passes over a sample until at least this much CPU time


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_rate(spec, L, x, label: str) -> dict:
    """The oracle, as it stands, on the host tokens x (single thread), repeated pass by pass until
    CPU_BASELINE_MIN_S seconds have accumulated. The expert weights the sample routes to are copied to
    host memory before timing (the oracle's own float64 conversion of them is part of its time)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import top_routed_expert_amd as moe
    from oracle import moe_oracle as O

    n = x.shape[0]
    # experts the sample uses (the library's routing of the same tokens decides what to copy; any
    # other expert the oracle asks for is copied when asked, inside the timed region)
    cfg = moe.config_for(spec)
    idx, _ = moe.route(cfg, x.to(L["x"].device), L["w_router"], L.get("bias"))
    used = sorted(set(int(e) for e in idx.cpu().numpy().reshape(-1).tolist() if e >= 0))
    host = {e: (L["w_gate"][e].cpu(), L["w_up"][e].cpu(), L["w_down"][e].cpu()) for e in used}
    expert = lambda e: host[e] if e in host else (L["w_gate"][e].cpu(), L["w_up"][e].cpu(), L["w_down"][e].cpu())
    sh = (L["s_gate"].cpu(), L["s_up"].cpu(), L["s_down"].cpu()) if spec.Fs else None
    bias = L.get("bias")
    W = O.LayerWeights(L["w_router"].cpu(), expert, (lambda: sh) if sh else None,
                       None if bias is None else bias.cpu())
    prev = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            passes, dt = 0, 0.0
            while passes == 0 or dt < CPU_BASELINE_MIN_S:
                t0 = time.perf_counter()
                r = O.layer_forward(x, W, spec.K)
                dt += time.perf_counter() - t0
                passes += 1
                assert np.all(np.isfinite(r["out"]))
    finally:
        torch.set_num_threads(prev)
    return dict(value=round(passes * n / dt, 3), unit="tokens/s",
                sample=f"{passes} pass(es) over the first {n} tokens of the {label} batch ({len(used)} experts), "
                       f"whole layer, numpy float64, {dt:.1f} s")


def cpu_baseline(L, decode_tokens: int, prefill_tokens: int) -> dict:
    """The oracle on the decode batch's first tokens (the headline unit) and on a slice of the prefill
    batch (more rows per expert, so its per-expert weight conversion is shared by more tokens).
    Decode and prefill use the same weights (same shape and seed); L holds them."""
    import synth

    d, p = synth.spec("decode"), synth.spec("prefill")
    r_d = oracle_rate(d, L, synth.make_x(d, "cpu", tokens=slice(0, min(decode_tokens, d.T))), "decode")
    r_p = oracle_rate(p, L, synth.make_x(p, "cpu", tokens=slice(0, min(prefill_tokens, p.T))), "prefill")
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return dict(value=r_d["value"], unit="tokens/s", cores=1, kind="oracle", sample=r_d["sample"],
                nproc=os.cpu_count(), cpus_available=aff, cpu_model=cpu_model(),
                prefill=dict(value=r_p["value"], unit="tokens/s", sample=r_p["sample"]))


# ---------------------------------------------------------- profile summaries ---

def _short_kernel(n: str) -> str:
    import re
    n = re.sub(r"\(anonymous namespace\)::", "", n).replace("void ", "")
    return n.split("(")[0]


def summarize_trace(d: str, title: str, command: str, out: str) -> None:
    """Markdown summary of a kernel-trace run: per (kernel, grid) average and minimum duration."""
    import collections
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_trace.csv"))))
    agg = collections.OrderedDict()
    for r in rows:
        if "moe::" not in r["Kernel_Name"]:
            continue
        gx = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        gy = int(r["Grid_Size_Y"]) // int(r["Workgroup_Size_Y"])
        k = (_short_kernel(r["Kernel_Name"]), f"{gx} x {gy}")
        agg.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000)
    L = [f"# {title}\n", "Command (repo root, one MI355X, `TMPDIR=/tmp`):\n", "```", command, "```\n",
         "Durations per dispatch from the kernel trace, grouped by kernel and grid (blocks x slices). "
         "Written by `python bench.py --summarize-trace <dir>`.\n",
         "| kernel | grid (blocks x y) | calls | avg us | min us |", "|---|---|---|---|---|"]
    for (n, g), v in agg.items():
        L.append(f"| `{n}` | {g} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} |")
    st = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    L += ["", "rocprofv3 --stats totals of the library's kernels over the whole run:", "",
          "| kernel | calls | total ms | avg us |", "|---|---|---|---|"]
    for r in st:
        if "moe::" in r["Name"]:
            L.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {int(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} |")
    open(out, "w").write("\n".join(L) + "\n")


def measured_peaks(reps: int = 10) -> dict:
    """Rates this GPU reaches with plain library work, beside the published peaks: a 2 GiB
    device-to-device copy (HBM read and write, counted both ways) and one 8192^3 bf16 matrix
    product (torch.matmul, the vendor GEMM library). Timed with HIP events on the current stream."""
    import torch

    ev = lambda: torch.cuda.Event(enable_timing=True)
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = ev(), ev()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(2):
        torch.matmul(x, y)
    a, b = ev(), ev()
    a.record()
    for _ in range(reps):
        torch.matmul(x, y)
    b.record()
    torch.cuda.synchronize()
    tflops = 2 * m ** 3 * reps / (a.elapsed_time(b) * 1e-3) / 1e12
    del x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_gbs": round(copy_gbs, 1), "bf16_matmul_tflops": round(tflops, 1),
            "how": "2 GiB device copy (read + write bytes); torch.matmul bf16 8192x8192x8192; 10 runs each"}


def of_measured(roof: dict, peaks: dict):
    """An MFMA-bound roofline's achieved rate as a fraction of the vendor GEMM's measured rate.
    HBM-bound ones get none: no plain library kernel reads HBM as fast as the expert GEMMs do (a
    device copy moves about 4.8 TB/s of reads and writes together, torch's reductions read at
    about 4 TB/s), so such a fraction would say nothing about the kernel."""
    if roof.get("bound") != "mfma" or not peaks["bf16_matmul_tflops"]:
        return None
    return round(roof["achieved"] / peaks["bf16_matmul_tflops"], 4)


# counter passes of the 256x256 expert GEMMs (each within one run's per-block limits)
COUNTER_PASSES = {
    "sq_a": "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT "
            "SQ_ACTIVE_INST_LDS SQ_WAVE_CYCLES SQ_WAIT_ANY",
    "sq_b": "SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_LDS_IDX_ACTIVE SQ_LDS_ADDR_CONFLICT SQ_LDS_UNALIGNED_STALL "
            "SQ_INSTS_LDS SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VMEM",
    "sq_c": "SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_INSTS_VMEM_RD "
            "SQ_WAVES SQ_CYCLES TA_BUSY_avr",
    "tcc": "TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum",
    "tcp": "TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum TCP_TCR_TCP_STALL_CYCLES_sum "
           "TA_ADDR_STALLED_BY_TC_CYCLES_sum TA_DATA_STALLED_BY_TC_CYCLES_sum TD_TC_STALL_sum TD_TD_BUSY_sum",
}


def synth_tokens(workload: str) -> int:
    import synth
    return synth.spec(workload).T


# expert GEMM kernels whose counters summarize_counters reports, by workload: the 256x256 kernel at
# prefill, the 32-row-tile kernel (weights streamed non-temporally) at decode
COUNTER_KERNELS = {
    "prefill": {"gate/up": "gemm_bf16_big8<0", "down": "gemm_bf16_big8<1"},
    "decode": {"gate/up": "gemm_bf16_mfma<0, 2, 1, 2, 4, true, true", "down": "gemm_bf16_mfma<1, 2, 1, 2, 4, true, true"},
}


def summarize_counters(d: str, out: str, workload: str = "prefill") -> None:
    """Per-dispatch averages of the counter passes for the expert gate/up and down kernels of a run of
    `workload`, with the derived clock, matrix-core utilisation, wait fractions, L2 hit rate and vector L1
    read latency."""
    import collections
    import csv
    kinds = COUNTER_KERNELS[workload]
    tiles = "256x256 expert GEMMs" if workload == "prefill" else "32-row-tile expert GEMMs"
    T = synth_tokens(workload)
    vals = {k: collections.OrderedDict() for k in kinds}
    for name in COUNTER_PASSES:
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(os.path.join(d, name, "run_counter_collection.csv"))):
            for k, pat in kinds.items():
                if pat in r["Kernel_Name"]:
                    per[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k in kinds:
            for c, v in per[k].items():
                vals[k][c] = sum(v) / len(v)
    dur = {}
    for r in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_trace.csv"))):
        for k, pat in kinds.items():
            if pat in r["Kernel_Name"]:
                dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9)
    wl = "" if workload == "prefill" else f" --counters-workload {workload}"
    L = [f"# SQ / LDS / matrix-core / L1 / L2 counters of the {tiles}, {workload} (T={T}), MI355X\n",
         "Commands (repo root, one MI355X, `TMPDIR=/tmp`), one pass each under `timeout -s KILL 120`, then "
         f"`python bench.py --summarize-counters <dir>{wl} --out {out}`:\n", "```"]
    for name, cs in COUNTER_PASSES.items():
        L.append(f"rocprofv3 --pmc {cs} --output-format csv -d <dir>/{name} -o run -- python bench.py --workload "
                 f"{workload} --steps 2 --warmup 1 --no-cpu-baseline --no-secondary")
    L += ["rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o run -- python bench.py --workload "
          f"{workload} --steps 2 --warmup 1 --no-cpu-baseline --no-secondary", "```\n",
          "Per dispatch, averaged over the dispatches of each kernel in the run (the layer steps and the gate/up "
          "kernel alone). rocprofv3 reports each counter summed over its hardware instances: GRBM_GUI_ACTIVE over "
          "the 8 XCDs, SQ_CYCLES over the 32 shader engines.\n",
          f"| counter | gate/up `{kinds['gate/up']}…>` | down `{kinds['down']}…>` |", "|---|---|---|"]
    names = sorted(set(vals["gate/up"]) | set(vals["down"]))
    for c in names:
        L.append(f"| {c} | {vals['gate/up'].get(c, float('nan')):.0f} | {vals['down'].get(c, float('nan')):.0f} |")
    L += ["", "Derived:", ""]
    for k in kinds:
        v = vals[k]
        cyc = v.get("GRBM_GUI_ACTIVE", 0.0) / 8
        t = sum(dur.get(k, [0.0])) / max(1, len(dur.get(k, [])))
        line = f"- {k}: {cyc / 1e6:.2f}M cycles per XCD"
        if t > 0:
            line += f" in {t * 1e3:.3f} ms (trace average), so about {cyc / t / 1e9:.2f} GHz"
        if cyc > 0:
            line += (f"; matrix cores busy {100 * v.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (cyc * 1024):.1f}% of "
                     "cycles (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs))")
        wc = v.get("SQ_WAVE_CYCLES", 0.0)
        if wc > 0:
            line += (f"; waves waiting on a counter {100 * v.get('SQ_WAIT_ANY', 0) / wc:.0f}% and to issue "
                     f"{100 * v.get('SQ_WAIT_INST_ANY', 0) / wc:.0f}% of wave cycles")
        la = v.get("SQ_LDS_IDX_ACTIVE", 0.0)
        if la > 0:
            line += f"; LDS bank conflicts {100 * v.get('SQ_LDS_BANK_CONFLICT', 0) / la:.2f}% of LDS-active cycles"
        req = v.get("TCC_REQ_sum", 0.0)
        if req > 0:
            line += (f"; L2 {req / 1e6:.1f}M requests ({req * 128 / 1e9:.2f} GB in 128-byte lines), hit rate "
                     f"{100 * v.get('TCC_HIT_sum', 0) / req:.1f}%")
        if v.get("SQ_INSTS_MFMA"):
            line += f"; {v['SQ_INSTS_MFMA'] / 1e6:.1f}M MFMA instructions"
        rq = v.get("TCP_TCC_READ_REQ_sum", 0.0)
        if rq > 0 and cyc > 0:
            lat = v.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / rq  # cycles from a vector L1 miss to its L2 data
            per_cu = rq / 256 / cyc  # requests per cycle per compute unit
            line += (f"; vector L1 to L2 reads {rq / 1e6:.1f}M ({rq * 128 / 1e9:.2f} GB), average latency "
                     f"{lat:.0f} cycles, so about {per_cu * lat:.0f} reads in flight per compute unit on average "
                     f"({per_cu * 128:.1f} bytes per cycle per compute unit); the vector L1 waits on pending L2 "
                     f"data {100 * v.get('TCP_PENDING_STALL_CYCLES_sum', 0) / (256 * cyc):.0f}% of cycles and the "
                     f"texture data unit on the cache {100 * v.get('TD_TC_STALL_sum', 0) / (256 * cyc):.0f}%")
        L.append(line)
    open(out, "w").write("\n".join(L) + "\n")


PMC_WORKLOADS = ("decode", "prefill", "skew", "full")


def summarize_pmc(d: str, out: str) -> None:
    """Gate/up HBM traffic per launch from FETCH_SIZE / WRITE_SIZE runs, each counter scaled by what it
    reads for the run's 1 GiB device copy (bench.py --copy-calibration), against the algorithmic bytes."""
    import collections
    import csv

    import synth

    def load(w, c):
        agg = collections.OrderedDict()
        for r in csv.DictReader(open(os.path.join(d, f"pmc_{w}_{c}", "run_counter_collection.csv"))):
            if r["Counter_Name"] == c:
                agg.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return agg

    L = ["# HBM traffic of the expert gate/up kernel (PMC), MI355X, packed weights\n",
         "Commands (repo root), one counter per run, each under `timeout -s KILL 240`; summary written by "
         f"`python bench.py --summarize-pmc <dir> --out {out}`:\n", "```"]
    for w in PMC_WORKLOADS:
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            L.append(f"rocprofv3 --pmc {c} --output-format csv -d <dir>/pmc_{w}_{c} -o run -- python bench.py "
                     f"--workload {w} --steps 3 --warmup 1 --no-cpu-baseline --no-secondary --copy-calibration "
                     f"> <dir>/pmc_{w}_{c}/bench.log")
    L += ["```\n",
          "`--copy-calibration` copies 1 GiB device to device first (`__amd_rocclr_copyBuffer`, grid 131072), a "
          "kernel of known traffic: 1048576 KiB read and 1048576 KiB written. Each counter is scaled by "
          "1048576 / (its value for that copy), then x 1024 to bytes. The gate/up kernel is the one with the "
          "most FETCH_SIZE per dispatch among the expert gate/up launches (the layer's own and the standalone "
          "one are the same kernel and grid). Per dispatch, in KiB:\n",
          "| workload | gate/up kernel | FETCH (copy) | FETCH (kernel) | WRITE (copy) | WRITE (kernel) | dispatches |",
          "|---|---|---|---|---|---|---|"]
    lines, other = [], []
    for w in PMC_WORKLOADS:
        f, wr = load(w, "FETCH_SIZE"), load(w, "WRITE_SIZE")
        ck = [k for k in f if k[0] == "__amd_rocclr_copyBuffer" and k[1] == 131072]
        cf, cw = f[ck[0]][0], wr[ck[0]][0]
        ff, fw = 1048576.0 / cf, 1048576.0 / cw
        # the gate/up launch: EPI_SWIGLU (template argument 0) of the expert GEMMs
        gu = [k for k in f if ("gemm_bf16_big8<0" in k[0] or "gemm_bf16_mfma<0" in k[0])]
        key = max(gu, key=lambda k: sum(f[k]) / len(f[k]))
        fv = sum(f[key]) / len(f[key])
        wv = sum(wr.get(key, [0.0])) / max(1, len(wr.get(key, [0.0])))
        L.append(f"| {w} | `{_short_kernel(key[0])}` | {cf:.1f} | {fv:.1f} | {cw:.1f} | {wv:.1f} | {len(f[key])} |")
        spec = synth.spec(w)
        traffic = fv * ff * 1024 + wv * fw * 1024
        lines.append((w, traffic, key))
        for k in f:
            if "moe::" not in k[0] or "pack_kernel" in k[0] or k == key:
                continue
            fb = sum(f[k]) / len(f[k]) * ff * 1024
            wb = sum(wr.get(k, [0.0])) / max(1, len(wr.get(k, [0.0]))) * fw * 1024
            if fb + wb >= 1e6:
                other.append(f"- {w}: `{_short_kernel(k[0])}` (grid {k[1]}): {fb / 1e9:.3f} GB fetched, "
                             f"{wb / 1e9:.3f} GB written")
    L.append("")
    for w, t, _ in lines:
        L.append(f"traffic_bytes[{w}]: {int(t)}")
    L.append("")
    L.append("Against the algorithmic bytes of the same launch (touched experts' gate and up weights, the token "
             "rows once, the SwiGLU output: `roofline.algorithmic_bytes` of the bench line each run printed to "
             "`<dir>/pmc_<workload>_FETCH_SIZE/bench.log`):\n")
    for w, t, _ in lines:
        log = os.path.join(d, f"pmc_{w}_FETCH_SIZE", "bench.log")
        alg = None
        if os.path.exists(log):
            for ln in open(log).read().splitlines()[::-1]:
                if ln.startswith("{"):
                    alg = json.loads(ln)["roofline"]["algorithmic_bytes"]
                    break
        if alg:
            L.append(f"- {w}: {t / 1e9:.3f} GB measured vs {alg / 1e9:.3f} GB algorithmic ({t / alg:.3f}x)")
    L.append("")
    L.append("Other kernels in the same runs (per launch, scaled):\n")
    L += other
    L += ["", "Kernel sources these counters belong to (bench.py reports the traffic only while they hash the same):",
          "", f"source_sha256: {kernel_source_hash()}"]
    open(out, "w").write("\n".join(L) + "\n")


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.title, args.command, args.out)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.out)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.counters_workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth

    if args.fp8:
        print(f"[bench] fp8 vs bf16 expert weights, steps={args.steps} warmup={args.warmup}", file=sys.stderr,
              flush=True)
        fp8_weights(args.steps, args.warmup, not args.no_flush)
        return
    if args.ep_share:
        print(f"[bench] expert-parallel share, steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
        print(json.dumps(ep_share(args.steps, args.warmup, not args.no_flush)), flush=True)
        return
    if args.dynamic_k:
        print(f"[bench] dynamic top-k vs fixed top-8, steps={args.steps} warmup={args.warmup}", file=sys.stderr,
              flush=True)
        dynamic_topk(args.steps, args.warmup, not args.no_flush)
        return
    if args.sweep:
        print(f"[bench] token-count sweep {SWEEP_T} at the prefill shape, steps={args.steps} warmup={args.warmup}",
              file=sys.stderr, flush=True)
        sweep(args.steps, args.warmup, not args.no_flush)
        return
    spec = synth.spec(args.workload)
    print(f"[bench] workload={spec.name} T={spec.T} steps={args.steps} warmup={args.warmup}", file=sys.stderr,
          flush=True)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = measure(spec, args.steps, args.warmup, not args.no_flush, args.layout == "packed")
    print(f"[bench] layer {res['ms']:.4f} ms/step; gate/up kernel {res['roofline']['launch_ms']:.4f} ms",
          file=sys.stderr, flush=True)
    line = {
        "metric": METRIC, "value": round(res["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": spec.name, "tokens": spec.T, "d_model": spec.D, "routed_experts": spec.E,
                   "top_k": spec.K, "d_expert": spec.F, "shared_experts": 1 if spec.Fs else 0,
                   "d_shared": spec.Fs, "router_bias": "zipf" if spec.skew else "none",
                   "weight_layout": res["layout"], "parallelism": "single-gpu"},
        "roofline": res["roofline"],
        "layer": {"ms_min": round(res["ms_min"], 5), "experts_touched": res["touched"],
                  "expert_load_skew": round(res["skew"], 3), "tflops": round(res["layer_tflops"], 2),
                  "gbs": round(res["layer_gbs"], 1),
                  "mfma_frac": round(res["layer_tflops"] / res["peak_tf"], 4),
                  "hbm_frac": round(res["layer_gbs"] / HBM_PEAK_GBS, 4), "timed_wall_s": round(res["wall"], 3),
                  "cache_flush_between_steps": not args.no_flush},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        same = lambda a, b: (a.D, a.E, a.F, a.Fs, a.dtype, a.seed) == (b.D, b.E, b.F, b.Fs, b.dtype, b.seed)
        if same(spec, synth.spec("decode")):
            line["cpu_baseline"] = cpu_baseline(res["L"], args.cpu_sample_tokens, args.cpu_prefill_tokens)
        else:
            del res["L"]
            torch.cuda.empty_cache()
            Ld = synth.make_layer(synth.spec("decode"), "cuda")
            line["cpu_baseline"] = cpu_baseline(Ld, args.cpu_sample_tokens, args.cpu_prefill_tokens)
            del Ld
    res.pop("L", None)
    if not args.no_secondary:
        others = {}
        for name in ("tiny", "decode", "prefill", "skew", "full"):
            if name == spec.name:
                continue
            torch.cuda.empty_cache()
            sp = synth.spec(name)
            print(f"[bench] workload={sp.name} T={sp.T}", file=sys.stderr, flush=True)
            r2 = measure(sp, args.steps, args.warmup, not args.no_flush, args.layout == "packed")
            del r2["L"]
            others[name] = workload_entry(sp, r2)
            print(f"[bench] {name}: layer {r2['ms']:.4f} ms/step; gate/up kernel "
                  f"{r2['roofline']['launch_ms']:.4f} ms", file=sys.stderr, flush=True)
        line["workloads"] = others
        torch.cuda.empty_cache()
        peaks = measured_peaks()
        print(f"[bench] measured: copy {peaks['hbm_copy_gbs']:.0f} GB/s, bf16 matmul "
              f"{peaks['bf16_matmul_tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
        line["measured_peaks"] = peaks
        for r in [line["roofline"]] + [e["roofline"] for e in others.values()]:
            f = of_measured(r, peaks)
            if f is not None:
                r["frac_of_vendor_gemm"] = f
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
