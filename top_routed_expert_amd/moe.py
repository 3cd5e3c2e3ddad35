"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every computation runs in the HIP kernels of libmoe.so. Torch supplies the
device memory (inputs, outputs, workspace) and the current HIP stream. The
functions check dtype, device, contiguity and shape of the tensors, allocate
outputs and workspace with torch, and raise MoeError when the library
returns a non-zero status. There is no fallback: if libmoe.so is missing or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

F32, BF16 = 0, 1
LAYOUT_ROWS, LAYOUT_PACKED, LAYOUT_FP8 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16}
SIZE_MAX = ctypes.c_size_t(-1).value


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn} failed with status {status} ({status_string(status)}): {detail}")
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("d_shared", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("weight_layout", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "router_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                 "w_gate_scale", "w_up_scale", "w_down_scale", "s_gate_scale", "s_up_scale", "s_down_scale")]


_lib = None
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_CFG = ctypes.POINTER(MoeConfig)
_SIGS = {
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_route_workspace_bytes": ([_CFG, _I64], _SZ),
    "moe_permute_workspace_bytes": ([_CFG, _I64], _SZ),
    "moe_grouped_ffn_workspace_bytes": ([_CFG, _I32, _I64, _I32], _SZ),
    "moe_layer_workspace_bytes": ([_CFG, _I64], _SZ),
    "moe_route": ([_CFG, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_route_dynamic": ([_CFG, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_permute": ([_CFG, _I64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_grouped_ffn": ([_CFG, _I32, _I64, _P, _P, _I64, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_expert_workspace_bytes": ([_CFG, _I32, _I64, _I32], _SZ),
    "moe_expert_gate_up": ([_CFG, _I32, _I64, _P, _P, _I64, _P, _I64, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P],
                           ctypes.c_int),
    "moe_expert_down": ([_CFG, _I32, _I64, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_combine": ([_CFG, _I64, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "moe_layer_forward": ([_CFG, _I64, _P, ctypes.POINTER(MoeWeights), _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_layer_forward_dynamic": ([_CFG, _I64, _P, ctypes.POINTER(MoeWeights), _P, _P, _P, _P, _P, _P, _SZ, _P],
                                  ctypes.c_int),
    "moe_route_group_stats_workspace_bytes": ([_CFG, _I64, _I32], _SZ),
    "moe_route_group_stats": ([_CFG, _I64, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_ep_receive_plan": ([_I32, _I32, _P, _I64, _P, _P, _P, _P], ctypes.c_int),
    "moe_gather_rows": ([_P, _I64, _I64, _P, _I64, _P, _P], ctypes.c_int),
    "moe_packed_weights_bytes": ([_I64, _I64, _I64], _SZ),
    "moe_fp8_weights_bytes": ([_I64, _I64, _I64], _SZ),
    "moe_quantize_fp8": ([_I64, _I64, _I64, _P, _P, _SZ, _P, _P], ctypes.c_int),
    "moe_pack_weights": ([_I64, _I64, _I64, _P, _P, _SZ, _P], ctypes.c_int),
    "moe_noalloc_scratch_bytes": ([], _SZ),
    "moe_layer_forward_noalloc": ([_CFG, _I64, _P, ctypes.POINTER(MoeWeights), _P, _P, _P, _P, _P], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m top_routed_expert_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise MoeError(status, fn, lib().moe_last_error().decode())


@dataclass(frozen=True)
class Config:
    """Layer shape (moe_config): d_model, routed experts, top-k, expert and shared widths."""
    d_model: int
    n_experts: int
    top_k: int
    d_expert: int
    d_shared: int
    dtype: torch.dtype = torch.bfloat16
    out_dtype: torch.dtype | None = None
    packed: bool = False  # weight matrices in the packed fragment layout (pack_weights)
    fp8: bool = False     # expert matrices FP8 E4M3 (quantize_fp8) with per-row scales; router packed bf16

    def c(self) -> MoeConfig:
        out = self.out_dtype if self.out_dtype is not None else self.dtype
        layout = LAYOUT_FP8 if self.fp8 else (LAYOUT_PACKED if self.packed else LAYOUT_ROWS)
        return MoeConfig(self.d_model, self.n_experts, self.top_k, self.d_expert, self.d_shared,
                         _DT[self.dtype], _DT[out], layout)

    def wshape(self, *shape: int) -> tuple:
        """Shape of a weight tensor whose row-major shape is `shape` (rows rounded up to 16 when packed)."""
        if not (self.packed or self.fp8):
            return tuple(shape)
        return (*shape[:-2], (shape[-2] + 15) // 16 * 16, shape[-1])

    @property
    def odtype(self) -> torch.dtype:
        return self.out_dtype if self.out_dtype is not None else self.dtype


def _ptr(t: torch.Tensor | None, name: str, dtype=None, shape=None, device=None) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() and t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")
    return t.data_ptr() if t.numel() else None


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    if nbytes == SIZE_MAX:
        raise ValueError("invalid configuration (workspace query returned SIZE_MAX)")
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def route(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor | None = None,
          want_gap: bool = False, k_per_token: torch.Tensor | None = None):
    """moe_route (moe_route_dynamic with k_per_token [T] int32): returns
    (topk_idx [T,K] int32, topk_prob [T,K] fp32[, gap [T] fp32])."""
    T = x.shape[0]
    dev = x.device
    c = cfg.c()
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    prob = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    gap = torch.empty((T,), dtype=torch.float32, device=dev) if want_gap else None
    ws = _workspace(lib().moe_route_workspace_bytes(ctypes.byref(c), T), dev)
    _check(lib().moe_route_dynamic(ctypes.byref(c), T, _ptr(x, "x", cfg.dtype, (T, cfg.d_model)),
                                   _ptr(w_router, "w_router", cfg.dtype, cfg.wshape(cfg.n_experts, cfg.d_model), dev),
                                   _ptr(bias, "bias", torch.float32, (cfg.n_experts,), dev),
                                   _ptr(k_per_token, "k_per_token", torch.int32, (T,), dev),
                                   _ptr(idx, "idx"), _ptr(prob, "prob"), _ptr(gap, "gap"),
                                   ws.data_ptr(), ws.numel(), _stream(dev)), "moe_route")
    return (idx, prob, gap) if want_gap else (idx, prob)


def permute(cfg: Config, topk_idx: torch.Tensor, x: torch.Tensor | None = None):
    """moe_permute: returns (offsets [E+1], sorted_token [T*K], dest [T*K][, x_perm [T*K, D]])."""
    T = topk_idx.shape[0]
    dev = topk_idx.device
    c = cfg.c()
    P = T * cfg.top_k
    offsets = torch.zeros((cfg.n_experts + 1,), dtype=torch.int32, device=dev)
    sorted_token = torch.empty((P,), dtype=torch.int32, device=dev)
    dest = torch.empty((P,), dtype=torch.int32, device=dev)
    x_perm = torch.empty((P, cfg.d_model), dtype=cfg.dtype, device=dev) if x is not None else None
    ws = _workspace(lib().moe_permute_workspace_bytes(ctypes.byref(c), T), dev)
    _check(lib().moe_permute(ctypes.byref(c), T, _ptr(topk_idx, "topk_idx", torch.int32, (T, cfg.top_k)),
                             _ptr(offsets, "offsets"), _ptr(sorted_token, "sorted_token"), _ptr(dest, "dest"),
                             _ptr(x, "x", cfg.dtype, (T, cfg.d_model), dev), _ptr(x_perm, "x_perm"),
                             ws.data_ptr(), ws.numel(), _stream(dev)), "moe_permute")
    return (offsets, sorted_token, dest, x_perm) if x is not None else (offsets, sorted_token, dest)


def grouped_ffn(cfg: Config, offsets: torch.Tensor, x: torch.Tensor, w_gate: torch.Tensor, w_up: torch.Tensor,
                w_down: torch.Tensor, gather: torch.Tensor | None = None, n_rows: int | None = None,
                y: torch.Tensor | None = None) -> torch.Tensor:
    """moe_grouped_ffn: y [n_rows, D] fp32, group g = rows offsets[g]:offsets[g+1] with expert g's weights.

    w_gate, w_up: [G, d_ff, D]; w_down: [G, D, d_ff]. n_rows defaults to
    len(gather) if given, else x.shape[0].
    """
    dev = x.device
    G, d_ff, D = w_gate.shape
    if n_rows is None:
        n_rows = gather.shape[0] if gather is not None else x.shape[0]
    c = cfg.c()
    if y is None:
        y = torch.empty((n_rows, D), dtype=torch.float32, device=dev)
    ws = _workspace(lib().moe_grouped_ffn_workspace_bytes(ctypes.byref(c), G, n_rows, d_ff), dev)
    _check(lib().moe_grouped_ffn(ctypes.byref(c), G, n_rows, _ptr(offsets, "offsets", torch.int32, (G + 1,), dev),
                                 _ptr(x, "x", cfg.dtype), x.shape[0],
                                 _ptr(gather, "gather", torch.int32, (n_rows,), dev),
                                 _ptr(w_gate, "w_gate", cfg.dtype, (G, d_ff, D), dev),
                                 _ptr(w_up, "w_up", cfg.dtype, (G, d_ff, D), dev),
                                 _ptr(w_down, "w_down", cfg.dtype, (G, D, d_ff), dev), d_ff,
                                 _ptr(y, "y", torch.float32, (n_rows, D), dev),
                                 ws.data_ptr(), ws.numel(), _stream(dev)), "moe_grouped_ffn")
    return y


def expert_gate_up(cfg: Config, offsets: torch.Tensor, x: torch.Tensor, w_gate: torch.Tensor,
                   w_up: torch.Tensor, gather: torch.Tensor | None = None, n_rows: int | None = None,
                   s_gate: torch.Tensor | None = None, s_up: torch.Tensor | None = None,
                   h: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """moe_expert_gate_up: h [n_rows, d_ff] = silu(x W_g^T) * (x W_u^T) per group (dtype).

    Rows r < len(gather) read x[gather[r]], later rows read x[r - len(gather)].
    With s_gate/s_up, one more group (offsets has G+2 entries) uses them.
    """
    dev = x.device
    G, d_ff, D = w_gate.shape
    n_gather = gather.shape[0] if gather is not None else 0
    if n_rows is None:
        n_rows = n_gather if gather is not None else x.shape[0]
    extra = 1 if s_gate is not None else 0
    c = cfg.c()
    if h is None:
        h = torch.empty((n_rows, d_ff), dtype=cfg.dtype, device=dev)
    if ws is None:
        ws = _workspace(lib().moe_expert_workspace_bytes(ctypes.byref(c), G + extra, n_rows, d_ff), dev)
    _check(lib().moe_expert_gate_up(
        ctypes.byref(c), G, n_rows, _ptr(offsets, "offsets", torch.int32, (G + 1 + extra,), dev),
        _ptr(x, "x", cfg.dtype), x.shape[0], _ptr(gather, "gather", torch.int32, None, dev), n_gather,
        _ptr(w_gate, "w_gate", cfg.dtype, (G, d_ff, D), dev), _ptr(w_up, "w_up", cfg.dtype, (G, d_ff, D), dev),
        _ptr(s_gate, "s_gate", cfg.dtype, (d_ff, D), dev), _ptr(s_up, "s_up", cfg.dtype, (d_ff, D), dev), d_ff,
        _ptr(h, "h", cfg.dtype, (n_rows, d_ff), dev), ws.data_ptr(), ws.numel(), _stream(dev)), "moe_expert_gate_up")
    return h


def expert_down(cfg: Config, offsets: torch.Tensor, h: torch.Tensor, w_down: torch.Tensor,
                s_down: torch.Tensor | None = None, y: torch.Tensor | None = None,
                ws: torch.Tensor | None = None) -> torch.Tensor:
    """moe_expert_down: y [n_rows, D] fp32 = h W_d^T per group (s_down: one more group)."""
    dev = h.device
    G, D, d_ff = w_down.shape
    n_rows = h.shape[0]
    extra = 1 if s_down is not None else 0
    c = cfg.c()
    if y is None:
        y = torch.empty((n_rows, D), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(lib().moe_expert_workspace_bytes(ctypes.byref(c), G + extra, n_rows, d_ff), dev)
    _check(lib().moe_expert_down(
        ctypes.byref(c), G, n_rows, _ptr(offsets, "offsets", torch.int32, (G + 1 + extra,), dev),
        _ptr(h, "h", cfg.dtype, (n_rows, d_ff), dev), _ptr(w_down, "w_down", cfg.dtype, (G, D, d_ff), dev),
        _ptr(s_down, "s_down", cfg.dtype, (D, d_ff), dev), d_ff, _ptr(y, "y", torch.float32, (n_rows, D), dev),
        ws.data_ptr(), ws.numel(), _stream(dev)), "moe_expert_down")
    return y


def combine(cfg: Config, y_perm: torch.Tensor, dest: torch.Tensor, topk_prob: torch.Tensor,
            y_shared: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """moe_combine: out[t] = y_shared[t] + sum_k prob[t,k] * y_perm[dest[t*K+k]]."""
    T = topk_prob.shape[0]
    dev = topk_prob.device
    c = cfg.c()
    if out is None:
        out = torch.empty((T, cfg.d_model), dtype=cfg.odtype, device=dev)
    _check(lib().moe_combine(ctypes.byref(c), T, _ptr(y_perm, "y_perm", torch.float32, (T * cfg.top_k, cfg.d_model), dev),
                             _ptr(dest, "dest", torch.int32, (T * cfg.top_k,), dev),
                             _ptr(topk_prob, "topk_prob", torch.float32, (T, cfg.top_k), dev),
                             _ptr(y_shared, "y_shared", torch.float32, (T, cfg.d_model), dev),
                             _ptr(out, "out", cfg.odtype, (T, cfg.d_model), dev), _stream(dev)), "moe_combine")
    return out


def weights_struct(cfg: Config, w: dict) -> MoeWeights:
    """Validate a weight dict (keys as synth.make_layer) and pack it into moe_weights."""
    E, D, F, Fs = cfg.n_experts, cfg.d_model, cfg.d_expert, cfg.d_shared
    dev = w["w_router"].device
    s = MoeWeights()
    s.w_router = _ptr(w["w_router"], "w_router", cfg.dtype, cfg.wshape(E, D), dev)
    s.router_bias = _ptr(w.get("bias"), "bias", torch.float32, (E,), dev)
    ed = torch.uint8 if cfg.fp8 else cfg.dtype   # fp8: E4M3 codes, rows rounded up to 16
    r16 = (lambda n: (n + 15) // 16 * 16) if cfg.fp8 else (lambda n: n)
    s.w_gate = _ptr(w["w_gate"], "w_gate", ed, (E, r16(F), D), dev)
    s.w_up = _ptr(w["w_up"], "w_up", ed, (E, r16(F), D), dev)
    s.w_down = _ptr(w["w_down"], "w_down", ed, (E, r16(D), F), dev)
    if cfg.fp8:
        s.w_gate_scale = _ptr(w["w_gate_scale"], "w_gate_scale", torch.float32, (E, F), dev)
        s.w_up_scale = _ptr(w["w_up_scale"], "w_up_scale", torch.float32, (E, F), dev)
        s.w_down_scale = _ptr(w["w_down_scale"], "w_down_scale", torch.float32, (E, D), dev)
    if Fs:
        s.s_gate = _ptr(w["s_gate"], "s_gate", ed, (r16(Fs), D), dev)
        s.s_up = _ptr(w["s_up"], "s_up", ed, (r16(Fs), D), dev)
        s.s_down = _ptr(w["s_down"], "s_down", ed, (r16(D), Fs), dev)
        if cfg.fp8:
            s.s_gate_scale = _ptr(w["s_gate_scale"], "s_gate_scale", torch.float32, (Fs,), dev)
            s.s_up_scale = _ptr(w["s_up_scale"], "s_up_scale", torch.float32, (Fs,), dev)
            s.s_down_scale = _ptr(w["s_down_scale"], "s_down_scale", torch.float32, (D,), dev)
    return s


class Workspace:
    """A reusable device workspace for moe_layer_forward at up to T tokens."""

    def __init__(self, cfg: Config, T: int, device):
        c = cfg.c()
        self.nbytes = lib().moe_layer_workspace_bytes(ctypes.byref(c), T)
        self.buf = _workspace(self.nbytes, device)


def route_group_stats(cfg: Config, x: torch.Tensor, w_router: torch.Tensor, n_groups: int,
                      bias: torch.Tensor | None = None, k_per_token: torch.Tensor | None = None):
    """moe_route_group_stats: (topk_idx, topk_prob, stats [2G] fp64: group probability mass, pair counts)."""
    T = x.shape[0]
    dev = x.device
    c = cfg.c()
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
    prob = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
    stats = torch.empty((2 * n_groups,), dtype=torch.float64, device=dev)
    ws = _workspace(lib().moe_route_group_stats_workspace_bytes(ctypes.byref(c), T, n_groups), dev)
    _check(lib().moe_route_group_stats(
        ctypes.byref(c), T, _ptr(x, "x", cfg.dtype, (T, cfg.d_model)),
        _ptr(w_router, "w_router", cfg.dtype, cfg.wshape(cfg.n_experts, cfg.d_model), dev),
        _ptr(bias, "bias", torch.float32, (cfg.n_experts,), dev),
        _ptr(k_per_token, "k_per_token", torch.int32, (T,), dev), n_groups, _ptr(idx, "idx"), _ptr(prob, "prob"),
        _ptr(stats, "stats"), ws.data_ptr(), ws.numel(), _stream(dev)), "moe_route_group_stats")
    return idx, prob, stats


def ep_receive_plan(counts: torch.Tensor, max_rows: int):
    """moe_ep_receive_plan: counts [n_src, n_local] int32 -> (offsets [n_local+1], gather, scatter [max_rows])."""
    n_src, n_local = counts.shape
    dev = counts.device
    offsets = torch.empty((n_local + 1,), dtype=torch.int32, device=dev)
    gather = torch.empty((max(max_rows, 1),), dtype=torch.int32, device=dev)
    scatter = torch.empty((max(max_rows, 1),), dtype=torch.int32, device=dev)
    _check(lib().moe_ep_receive_plan(n_src, n_local, _ptr(counts.contiguous(), "counts", torch.int32), max_rows,
                                     _ptr(offsets, "offsets"), _ptr(gather, "gather"), _ptr(scatter, "scatter"),
                                     _stream(dev)), "moe_ep_receive_plan")
    return offsets, gather[:max_rows], scatter[:max_rows]


def gather_rows(src: torch.Tensor, index: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """moe_gather_rows: out[i] = src[index[i]] (rows of src's trailing dimensions)."""
    n = index.shape[0]
    dev = src.device
    if out is None:
        out = torch.empty((n, *src.shape[1:]), dtype=src.dtype, device=dev)
    row_bytes = src[0].numel() * src.element_size() if src.shape[0] else out[0].numel() * out.element_size()
    _check(lib().moe_gather_rows(_ptr(src, "src", None, None, dev), src.shape[0], row_bytes,
                                 _ptr(index, "index", torch.int32, (n,), dev), n,
                                 _ptr(out, "out", src.dtype, (n, *src.shape[1:]), dev), _stream(dev)),
           "moe_gather_rows")
    return out


def layer_forward(cfg: Config, x: torch.Tensor, w: dict, out: torch.Tensor | None = None,
                  routing: bool = False, workspace: Workspace | None = None, weights: MoeWeights | None = None,
                  k_per_token: torch.Tensor | None = None):
    """moe_layer_forward (moe_layer_forward_dynamic with k_per_token [T] int32): out [T, D];
    with routing=True also (topk_idx, topk_prob, offsets)."""
    T = x.shape[0]
    dev = x.device
    c = cfg.c()
    if out is None:
        out = torch.empty((T, cfg.d_model), dtype=cfg.odtype, device=dev)
    ws = workspace.buf if workspace is not None else \
        _workspace(lib().moe_layer_workspace_bytes(ctypes.byref(c), T), dev)
    wt = weights if weights is not None else weights_struct(cfg, w)
    idx = prob = offs = None
    if routing:
        idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=dev)
        prob = torch.empty((T, cfg.top_k), dtype=torch.float32, device=dev)
        offs = torch.empty((cfg.n_experts + 1,), dtype=torch.int32, device=dev)
    if k_per_token is None:
        _check(lib().moe_layer_forward(ctypes.byref(c), T, _ptr(x, "x", cfg.dtype, (T, cfg.d_model), dev),
                                       ctypes.byref(wt), _ptr(out, "out", cfg.odtype, (T, cfg.d_model), dev),
                                       _ptr(idx, "idx"), _ptr(prob, "prob"), _ptr(offs, "offsets"),
                                       ws.data_ptr(), ws.numel(), _stream(dev)), "moe_layer_forward")
    else:
        _check(lib().moe_layer_forward_dynamic(
            ctypes.byref(c), T, _ptr(x, "x", cfg.dtype, (T, cfg.d_model), dev), ctypes.byref(wt),
            _ptr(k_per_token, "k_per_token", torch.int32, (T,), dev),
            _ptr(out, "out", cfg.odtype, (T, cfg.d_model), dev), _ptr(idx, "idx"), _ptr(prob, "prob"),
            _ptr(offs, "offsets"), ws.data_ptr(), ws.numel(), _stream(dev)), "moe_layer_forward_dynamic")
    return (out, idx, prob, offs) if routing else out


def noalloc_scratch_bytes() -> int:
    """moe_noalloc_scratch_bytes: size of the library's static device scratch."""
    return lib().moe_noalloc_scratch_bytes()


def layer_forward_noalloc(cfg: Config, x: torch.Tensor, out: torch.Tensor, weights: MoeWeights,
                          topk_idx: torch.Tensor | None = None, topk_prob: torch.Tensor | None = None,
                          offsets: torch.Tensor | None = None) -> torch.Tensor:
    """moe_layer_forward_noalloc: the layer with the library's static scratch as its workspace.

    The caller passes every output (out [T, D]; optionally topk_idx [T,K], topk_prob [T,K],
    offsets [E+1]) and a prepared weights_struct, so nothing is allocated on this path."""
    T = x.shape[0]
    dev = x.device
    c = cfg.c()
    _check(lib().moe_layer_forward_noalloc(
        ctypes.byref(c), T, _ptr(x, "x", cfg.dtype, (T, cfg.d_model), dev), ctypes.byref(weights),
        _ptr(out, "out", cfg.odtype, (T, cfg.d_model), dev),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, cfg.top_k), dev),
        _ptr(topk_prob, "topk_prob", torch.float32, (T, cfg.top_k), dev),
        _ptr(offsets, "offsets", torch.int32, (cfg.n_experts + 1,), dev), _stream(dev)), "moe_layer_forward_noalloc")
    return out


def packed_weights_bytes(n_mats: int, rows: int, cols: int) -> int:
    """moe_packed_weights_bytes: bytes of n_mats packed [rows, cols] bf16 matrices."""
    return lib().moe_packed_weights_bytes(n_mats, rows, cols)


def pack_weights(w: torch.Tensor) -> torch.Tensor:
    """moe_pack_weights: a bf16 [rows, cols] or [n, rows, cols] device tensor in the packed fragment
    layout, returned as a tensor of shape [..., ceil(rows/16)*16, cols] (its bytes are the packed form)."""
    if w.dim() not in (2, 3):
        raise ValueError("pack_weights takes a [rows, cols] or [n, rows, cols] tensor")
    n = w.shape[0] if w.dim() == 3 else 1
    rows, cols = w.shape[-2], w.shape[-1]
    nbytes = packed_weights_bytes(n, rows, cols)
    if nbytes == SIZE_MAX:
        raise ValueError(f"cannot pack [{rows}, {cols}]: cols must be a multiple of 32")
    out = torch.empty((*w.shape[:-2], (rows + 15) // 16 * 16, cols), dtype=torch.bfloat16, device=w.device)
    _check(lib().moe_pack_weights(n, rows, cols, _ptr(w, "w", torch.bfloat16), _ptr(out, "out"),
                                  out.numel() * 2, _stream(w.device)), "moe_pack_weights")
    return out


def fp8_weights_bytes(n_mats: int, rows: int, cols: int) -> int:
    return lib().moe_fp8_weights_bytes(n_mats, rows, cols)


def quantize_fp8(w: torch.Tensor):
    """moe_quantize_fp8: bf16 [rows, cols] or [n, rows, cols] -> (E4M3 codes uint8 [..., ceil(rows/16)*16, cols]
    in the packed fp8 layout, per-row fp32 scales [..., rows])."""
    if w.dim() not in (2, 3):
        raise ValueError("quantize_fp8 takes a [rows, cols] or [n, rows, cols] tensor")
    n = w.shape[0] if w.dim() == 3 else 1
    rows, cols = w.shape[-2], w.shape[-1]
    nbytes = fp8_weights_bytes(n, rows, cols)
    if nbytes == SIZE_MAX:
        raise ValueError(f"cannot quantise [{rows}, {cols}]: cols must be a multiple of 64")
    codes = torch.empty((*w.shape[:-2], (rows + 15) // 16 * 16, cols), dtype=torch.uint8, device=w.device)
    scales = torch.empty((*w.shape[:-2], rows), dtype=torch.float32, device=w.device)
    _check(lib().moe_quantize_fp8(n, rows, cols, _ptr(w, "w", torch.bfloat16), _ptr(codes, "codes"), codes.numel(),
                                  _ptr(scales, "scales"), _stream(w.device)), "moe_quantize_fp8")
    return codes, scales


def quantize_layer(w: dict) -> dict:
    """A copy of a layer's weight dict for a Config with fp8=True: expert matrices as E4M3 codes with
    *_scale entries, the router packed (bf16)."""
    out = dict(w)
    out["w_router"] = pack_weights(w["w_router"])
    for k in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down"):
        if w.get(k) is not None:
            out[k], out[k + "_scale"] = quantize_fp8(w[k])
    return out


_WEIGHT_KEYS = ("w_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down")


def pack_layer(w: dict) -> dict:
    """A copy of a layer's weight dict with every weight matrix packed (for a Config with packed=True)."""
    return {k: (pack_weights(v) if k in _WEIGHT_KEYS and v is not None else v) for k, v in w.items()}
