"""Seeded synthetic inputs for one sparse-MoE FFN layer (test and bench infrastructure).

This module holds no part of the layer's arithmetic. It only draws the
inputs (activations, router weights, router bias, expert weights) that both
the CPU oracle and the HIP library consume, so both sides see bit-identical
values.

Generator
---------
Every tensor is a counter-based stream: element ``i`` of tensor ``tid`` under
``seed`` is

    z   = SplitMix64_mix(key(seed, tid) + (i + 1) * GAMMA)   (mod 2**64)
    q   = z >> 48                                             (16-bit level)
    val = round_to_dtype(float32(std * Phi^-1((q + 0.5) / 65536)))

``SplitMix64_mix`` and ``GAMMA`` are the output mix and increment of
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014). ``Phi^-1`` is the standard normal quantile, so the
values follow N(0, std**2) discretised to 65536 equiprobable levels
(|value| <= 4.17 std). The quantile table is built once in float64 on the
host and rounded to float32, then to bfloat16 with round-to-nearest-even
when the layer is bf16.

The stream uses only 64-bit integer arithmetic and one table gather, so the
same code run by torch on the CPU or on a GPU yields the same bits, and any
element, e.g. one expert's weight matrix, can be regenerated on its own.

Shapes and distributions follow the layer the pages state (Step 3.5 Flash:
288 routed experts + 1 shared, top-8, d_model 4096; page "Step3.5 Flash 大模型
技术深度解析", section 3.2.1 and 3.2.2): x ~ N(0, 1), router weights
~ N(0, 0.02), expert weights ~ N(0, 1/sqrt(fan_in)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from statistics import NormalDist

import torch

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
LEVELS = 1 << 16


def _s64(u: int) -> int:
    """Unsigned 64-bit constant as the signed int64 torch stores."""
    u &= MASK64
    return u - (1 << 64) if u >= (1 << 63) else u


def _srl(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 lanes (torch's >> is arithmetic)."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _s64(MIX1)
    z = (z ^ _srl(z, 27)) * _s64(MIX2)
    return z ^ _srl(z, 31)


def _mix_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tid: int) -> int:
    return _mix_int(((seed & 0xFFFFFFFF) << 32) + tid + 1)


_TABLES: dict = {}


def quantile_table(std: float) -> torch.Tensor:
    """float32 table: std * Phi^-1((q+0.5)/65536), computed in float64."""
    key = float(std)
    if key not in _TABLES:
        nd = NormalDist()
        vals = [std * nd.inv_cdf((q + 0.5) / LEVELS) for q in range(LEVELS)]
        _TABLES[key] = torch.tensor(vals, dtype=torch.float64).to(torch.float32)
    return _TABLES[key]


def levels(seed: int, tid: int, start: int, count: int, device) -> torch.Tensor:
    """16-bit quantile levels of elements [start, start+count) of stream tid."""
    i = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    z = i * _s64(GAMMA) + _s64(stream_key(seed, tid))
    return _srl(_mix(z), 48)


def fill_(out: torch.Tensor, seed: int, tid: int, std: float, start: int = 0,
          chunk: int = 1 << 24) -> torch.Tensor:
    """Fill a contiguous tensor with elements [start, start+numel) of stream tid."""
    flat = out.view(-1)
    table = quantile_table(std).to(out.device)
    n = flat.numel()
    for c0 in range(0, n, chunk):
        c = min(chunk, n - c0)
        q = levels(seed, tid, start + c0, c, out.device)
        flat[c0:c0 + c].copy_(table[q].to(out.dtype))
    return out


def draw(shape, seed: int, tid: int, std: float, dtype, device="cpu", start: int = 0):
    out = torch.empty(shape, dtype=dtype, device=device)
    return fill_(out, seed, tid, std, start)


# ---------------------------------------------------------------------------
# Layer workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerSpec:
    """Shape and input recipe of one MoE FFN layer workload."""
    name: str
    T: int           # tokens
    D: int           # d_model
    E: int           # routed experts
    K: int           # experts chosen per token
    F: int           # routed expert SwiGLU width
    Fs: int          # shared expert width (0 = no shared expert)
    dtype: str       # "bf16" or "f32": x and all weights
    skew: bool = False   # Zipf-like router bias b_e = 2 ln(1/(e+1))
    groups: int = 0      # report per-group counts over this many expert groups
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def out_dtype(self):
        return self.torch_dtype


WORKLOADS = {
    "tiny": LayerSpec("tiny", T=128, D=256, E=32, K=8, F=128, Fs=128, dtype="f32"),
    "decode": LayerSpec("decode", T=32, D=4096, E=288, K=8, F=1280, Fs=1280, dtype="bf16"),
    "prefill": LayerSpec("prefill", T=8192, D=4096, E=288, K=8, F=1280, Fs=1280, dtype="bf16"),
    "skew": LayerSpec("skew", T=4096, D=4096, E=288, K=8, F=1280, Fs=1280, dtype="bf16", skew=True),
    "full": LayerSpec("full", T=16384, D=4096, E=288, K=8, F=4096, Fs=4096, dtype="bf16", groups=8),
}


def spec(name: str, **over) -> LayerSpec:
    return replace(WORKLOADS[name], **over) if over else WORKLOADS[name]


# stream ids: one per tensor, one per expert matrix, so any expert regenerates alone
TID_X, TID_ROUTER, TID_KDYN = 0, 1, 2


def tid_expert(e: int, which: int) -> int:
    """which: 0 gate, 1 up, 2 down. e == E addresses the shared expert."""
    return 16 + 3 * e + which


def router_bias(s: LayerSpec) -> torch.Tensor | None:
    """Zipf-like bias b_e = 2 ln(1/(rank_e+1)) with rank_e = e, float32."""
    if not s.skew:
        return None
    return torch.tensor([2.0 * math.log(1.0 / (e + 1)) for e in range(s.E)],
                        dtype=torch.float64).to(torch.float32)


def make_x(s: LayerSpec, device="cpu", tokens: slice | None = None) -> torch.Tensor:
    t0 = 0 if tokens is None else tokens.start
    t1 = s.T if tokens is None else tokens.stop
    return draw((t1 - t0, s.D), s.seed, TID_X, 1.0, s.torch_dtype, device, start=t0 * s.D)


def make_router(s: LayerSpec, device="cpu") -> torch.Tensor:
    return draw((s.E, s.D), s.seed, TID_ROUTER, 0.02, s.torch_dtype, device)


def make_expert(s: LayerSpec, e: int, device="cpu"):
    """(gate [F,D], up [F,D], down [D,F]) of routed expert e, or the shared one if e == E."""
    F = s.Fs if e == s.E else s.F
    g = draw((F, s.D), s.seed, tid_expert(e, 0), 1.0 / math.sqrt(s.D), s.torch_dtype, device)
    u = draw((F, s.D), s.seed, tid_expert(e, 1), 1.0 / math.sqrt(s.D), s.torch_dtype, device)
    d = draw((s.D, F), s.seed, tid_expert(e, 2), 1.0 / math.sqrt(F), s.torch_dtype, device)
    return g, u, d


def dynamic_k(s: LayerSpec, choices=None, device="cpu") -> torch.Tensor:
    """Per-token expert counts of a dynamic top-k run, int32 [T].

    Token t takes choices[q_t % len(choices)], q_t being element t of the
    level stream (seed, TID_KDYN). Default choices (K // 2, K): the pages'
    simple and complex inputs (4 and 8 experts at K = 8; page "Step3.5 Flash
    大模型技术深度解析", section 8.2), in about equal numbers.
    """
    choices = tuple(choices) if choices is not None else (s.K // 2, s.K)
    q = levels(s.seed, TID_KDYN, 0, s.T, "cpu")
    return torch.tensor(choices, dtype=torch.int32)[q % len(choices)].to(device)


def make_layer(s: LayerSpec, device="cpu") -> dict:
    """All inputs of the layer as contiguous tensors on `device`.

    Routed expert weights are stacked: w_gate, w_up [E, F, D]; w_down [E, D, F].
    Shared expert: s_gate, s_up [Fs, D]; s_down [D, Fs] (None when Fs == 0).
    """
    dt = s.torch_dtype
    w_gate = torch.empty((s.E, s.F, s.D), dtype=dt, device=device)
    w_up = torch.empty_like(w_gate)
    w_down = torch.empty((s.E, s.D, s.F), dtype=dt, device=device)
    sd_in, sd_out = 1.0 / math.sqrt(s.D), 1.0 / math.sqrt(s.F)
    for e in range(s.E):
        fill_(w_gate[e], s.seed, tid_expert(e, 0), sd_in)
        fill_(w_up[e], s.seed, tid_expert(e, 1), sd_in)
        fill_(w_down[e], s.seed, tid_expert(e, 2), sd_out)
    layer = dict(x=make_x(s, device), w_router=make_router(s, device),
                 w_gate=w_gate, w_up=w_up, w_down=w_down,
                 s_gate=None, s_up=None, s_down=None, bias=None)
    b = router_bias(s)
    if b is not None:
        layer["bias"] = b.to(device)
    if s.Fs:
        g, u, d = make_expert(s, s.E, device)
        layer.update(s_gate=g, s_up=u, s_down=d)
    return layer
