"""CPU oracle for one sparse-MoE FFN layer (Step 3.5 Flash style).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the
HIP library is checked against. Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the library never calls
it and it calls nothing in the library.

Source: page "Step3.5 Flash 大模型技术深度解析：稀疏 MoE、混合注意力与 MTP 的
高效推理革命", section 3.2.1 (expert configuration: 288 routed experts per
layer, each an independent FFN, plus 1 always-active shared expert; d_model
4096) and section 3.2.2 (Top-8 routing: a linear layer plus softmax gives
each expert a probability; the 8 most probable routed experts and the shared
expert, 9 in all, run; their outputs are summed with weights).

Everything is float64 (inputs are converted exactly: bf16 and fp32 values and
their pairwise products are exact in float64). Library primitives used as
single steps: numpy matmul, exp, argsort (stable), bincount, cumsum.

Readings where the pages leave a step open (R8 to R11 are readings about the
workload shapes, the initialisation and training-time terms, not about the
steps below):
  R1 softmax runs over all E routed experts before selection (3.2.2 computes
     the probabilities, then selects the 8 most probable);
  R2 the selected probabilities weight the routed outputs as they are, with
     no renormalisation over the 8;
  R3 the shared expert has weight 1 (it is always active and has no router
     score);
  R4 each expert is a bias-free SwiGLU FFN: y = W_d (silu(W_g x) * (W_u x));
  R5 selection compares probabilities rounded to float32; equal float32
     probabilities go to the lower expert index; the returned probabilities
     are those float32 values;
  R6 no capacity limit: every (token, choice) pair is processed (dropless);
  R7 an optional per-expert router bias is added to the logits before the
     softmax;
  R12 dynamic top-k (page "Step3.5 Flash
     大模型技术深度解析", section 8.2: 4 experts for simple inputs, 8 for
     complex ones; page "Step 3.5 Flash动态稀疏MoE架构解析与优化实践", section
     2.1: fewer experts for short texts, up to 8 for long ones): token t keeps
     the first k_t of its choices in the same order (k_t clamped to [0, K]),
     with the same unrenormalised probabilities; its remaining slots hold
     expert -1 with probability 0 and contribute nothing; the shared expert
     is unchanged;
  R13 expert-parallel balance (page "Step3.5 Flash 大模型技术深度解析",
     section 3.2.3: the 288 experts in G groups, one per GPU; L_EP = G sum_g
     f_g p_g): groups are E/G contiguous expert ids; f_g is the fraction of
     the chosen (token, slot) pairs that fall in group g and p_g the mean over
     tokens of the softmax mass of group g's experts, so both sum to 1 and a
     perfectly balanced routing gives L_EP = 1. One GPU's share receives, per
     source rank r and local expert e, that source's rows for e in token
     order, chunks r-major; its experts run on them in expert-major order;
  R14 FP8 expert weights (page "Step3.5 Flash 大模型技术深度解析", section 8.1,
     deploys the model with FP8/FP16 weights): each expert matrix row (one
     output channel) is stored as OCP FP8 E4M3 codes q with one float32
     scale s = float32(max|w| / 448) (1 for an all-zero row); q = the E4M3
     value nearest to float32(w / s), ties to the even code, magnitudes
     above 448 saturating to 448. The weight the layer uses is
     decode(q) * s; activations stay bfloat16 and the router is not
     quantised.
"""
from __future__ import annotations

import numpy as np

try:  # accept torch tensors (bf16 included) as inputs without requiring torch
    import torch as _torch
except ImportError:  # pragma: no cover
    _torch = None


def as_f64(a) -> np.ndarray:
    """Exact conversion of a host array or CPU torch tensor to float64."""
    if _torch is not None and isinstance(a, _torch.Tensor):
        return a.detach().to("cpu", _torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- routing ---

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """Linear router (3.2.2, step 1): l[t,e] = sum_d x[t,d] W_r[e,d] (+ b[e], R7)."""
    l = as_f64(x) @ as_f64(w_router).T
    if bias is not None:
        l = l + as_f64(bias)[None, :]
    return l


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over all routed experts (3.2.2, step 1; R1), max-subtracted."""
    z = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(z)
    return w / w.sum(axis=1, keepdims=True)


def select_topk(p32: np.ndarray, k: int, k_per_token=None):
    """The k most probable experts per token (3.2.2, step 2; R5).

    Order: float32 probability descending, then expert index ascending.
    Returns (idx int32 [T,k], prob float32 [T,k], gap float64 [T]) where gap
    is p of the k-th choice minus p of the (k+1)-th (inf when k == E).
    With k_per_token (R12), token t keeps its first k_t = clip(k_per_token[t],
    0, k) choices; slots j >= k_t hold idx -1 and prob 0, and gap is taken at
    k_t (inf when k_t is 0 or E).
    """
    order = np.argsort(-p32, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    prob = np.take_along_axis(p32, order[:, :k], axis=1).astype(np.float32)
    if k_per_token is not None:
        T, E = p32.shape
        kt = np.clip(np.asarray(k_per_token, dtype=np.int64).reshape(-1), 0, k)
        gap = np.full(T, np.inf)
        for t in range(T):
            n = int(kt[t])
            idx[t, n:] = -1
            prob[t, n:] = 0.0
            if 0 < n < E:
                gap[t] = float(p32[t, order[t, n - 1]]) - float(p32[t, order[t, n]])
        return idx, prob, gap
    if k < p32.shape[1]:
        nxt = np.take_along_axis(p32, order[:, k:k + 1], axis=1)[:, 0]
        gap = prob[:, -1].astype(np.float64) - nxt.astype(np.float64)
    else:
        gap = np.full(p32.shape[0], np.inf)
    return idx, prob, gap


def route(x, w_router, k: int, bias=None, k_per_token=None) -> dict:
    """Router: logits -> softmax (fp64) -> float32 probabilities -> top-k
    (top-k_t per token with k_per_token, R12)."""
    logits = router_logits(x, w_router, bias)
    p64 = softmax(logits)
    p32 = p64.astype(np.float32)
    idx, prob, gap = (select_topk(p32, k) if k_per_token is None else select_topk(p32, k, k_per_token))
    return dict(logits=logits, p64=p64, p32=p32, idx=idx, prob=prob, gap=gap)


# ---------------------------------------------------------------- permute ---

def permute(idx: np.ndarray, n_experts: int) -> dict:
    """Group the (token, choice) pairs by expert (R6: all pairs kept).

    Pairs are taken in token-major order (t, then choice k); a stable sort on
    the expert id lays each expert's pairs out contiguously, in token order.
    Pairs with an expert id outside [0, E) (slot without an expert, R12) get
    no row.
      counts[e]        number of pairs routed to e
      offsets[e]       first row of e's segment (exclusive scan), offsets[E] =
                       number of pairs with an expert (T*k without R12)
      sorted_token[r]  token of permuted row r
      dest[t*k + j]    permuted row of pair (t, j), -1 without an expert
    """
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    pairs = np.nonzero((flat >= 0) & (flat < n_experts))[0]
    order = pairs[np.argsort(flat[pairs], kind="stable")]
    counts = np.bincount(flat[pairs], minlength=n_experts).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_token = (order // k).astype(np.int64)
    dest = np.full(T * k, -1, dtype=np.int64)
    dest[order] = np.arange(len(order))
    return dict(counts=counts, offsets=offsets, sorted_token=sorted_token, dest=dest)


# -------------------------------------------------------------- experts ---

def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ffn(x_rows, w_gate, w_up, w_down) -> np.ndarray:
    """One expert FFN on a block of rows (R4): W_d (silu(W_g x) * (W_u x))."""
    xr = as_f64(x_rows)
    g = xr @ as_f64(w_gate).T
    u = xr @ as_f64(w_up).T
    return (silu(g) * u) @ as_f64(w_down).T


def grouped_ffn(x_rows, offsets, expert_weights) -> np.ndarray:
    """Run expert e's FFN on rows offsets[e]:offsets[e+1] of x_rows.

    expert_weights(e) -> (w_gate [F,D], w_up [F,D], w_down [D,F]).
    """
    xr = as_f64(x_rows)
    y = np.zeros_like(xr)          # experts map d_model back to d_model
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = swiglu_ffn(xr[a:b], *expert_weights(e))
    return y


# -------------------------------------------------------------- combine ---

def combine(ys, y_perm, dest, prob) -> np.ndarray:
    """Weighted sum of the 9 expert outputs (3.2.2, step 3; R2, R3).

    out[t] = ys[t] + sum over j ascending of prob[t,j] * y_perm[dest[t*k+j]].
    ys is the shared expert's output (None: no shared expert).
    """
    prob = as_f64(prob)
    T, k = prob.shape
    y_perm = as_f64(y_perm)
    out = np.zeros((T, y_perm.shape[1])) if ys is None else as_f64(ys).copy()
    d = np.asarray(dest).reshape(T, k)
    for j in range(k):
        ok = d[:, j] >= 0                 # pairs without an expert add nothing (R12)
        out[ok] += prob[ok, j:j + 1] * y_perm[d[ok, j]]
    return out


# ---------------------------------------------------------------- layer ---

class LayerWeights:
    """Weights of one layer as callables, so large layers can be paged in per expert.

    router: [E, D]; bias: [E] or None; expert(e) -> (gate [F,D], up [F,D],
    down [D,F]); shared() -> the same triple or None.
    """

    def __init__(self, router, expert, shared=None, bias=None):
        self.router = router
        self.expert = expert
        self.shared = shared if shared is not None else (lambda: None)
        self.bias = bias

    @classmethod
    def from_dict(cls, L: dict) -> "LayerWeights":
        def expert(e):
            return L["w_gate"][e], L["w_up"][e], L["w_down"][e]

        def shared():
            if L.get("s_gate") is None:
                return None
            return L["s_gate"], L["s_up"], L["s_down"]

        return cls(L["w_router"], expert, shared, L.get("bias"))


def layer_forward(x, W: LayerWeights, k: int, k_per_token=None) -> dict:
    """The whole layer on all tokens: route, permute, experts, combine
    (per-token expert counts with k_per_token, R12)."""
    xr = as_f64(x)
    r = route(xr, W.router, k, W.bias) if k_per_token is None else route(xr, W.router, k, W.bias, k_per_token)
    E = r["p32"].shape[1]
    p = permute(r["idx"], E)
    x_perm = xr[p["sorted_token"]]
    y_perm = grouped_ffn(x_perm, p["offsets"], W.expert)
    sh = W.shared()
    ys = None if sh is None else swiglu_ffn(xr, *sh)
    out = combine(ys, y_perm, p["dest"], r["prob"])
    return dict(**r, **p, y_perm=y_perm, ys=ys, out=out)


def rows_output(x, W: LayerWeights, rows, idx_rows, prob_rows) -> np.ndarray:
    """The layer's output (3.2.2, step 3) for tokens `rows` given their routing.

    idx_rows [R, k]: each selected token's experts (-1: slot without an
    expert, R12); prob_rows [R, k]: their weights. out_rows[i] = shared FFN of
    token rows[i] (R3) + sum over j ascending of prob_rows[i, j] times expert
    idx_rows[i, j]'s FFN of that token. The expert FFNs run grouped by expert,
    so each expert's weights are read once.
    """
    xr = as_f64(x)
    rows = np.asarray(rows, dtype=np.int64)
    idx = np.asarray(idx_rows, dtype=np.int64).reshape(len(rows), -1)
    k = idx.shape[1]
    y_sel = np.zeros((len(rows), k, xr.shape[1]))
    for e in np.unique(idx[idx >= 0]):      # slots without an expert stay zero (R12)
        ri, kj = np.nonzero(idx == e)
        y_sel[ri, kj] = swiglu_ffn(xr[rows[ri]], *W.expert(int(e)))
    sh = W.shared()
    out = np.zeros((len(rows), xr.shape[1])) if sh is None else swiglu_ffn(xr[rows], *sh)
    prob = as_f64(prob_rows).reshape(len(rows), k)
    for j in range(k):
        ok = idx[:, j] >= 0
        out[ok] += prob[ok, j:j + 1] * y_sel[ok, j]
    return out


def layer_rows(x, W: LayerWeights, k: int, rows, k_per_token=None) -> dict:
    """The layer's output for selected tokens only, with routing for all tokens.

    Routing and the permutation are computed for every token (they are
    cheap); the expert FFNs run only for the (token, choice) pairs of the
    selected tokens (rows_output). out_rows[i] is the output of token rows[i].
    """
    xr = as_f64(x)
    r = route(xr, W.router, k, W.bias) if k_per_token is None else route(xr, W.router, k, W.bias, k_per_token)
    E = r["p32"].shape[1]
    p = permute(r["idx"], E)
    rows = np.asarray(rows, dtype=np.int64)
    out = rows_output(xr, W, rows, r["idx"][rows], r["prob"][rows])
    return dict(**r, **p, rows=rows, out_rows=out)


# -------------------------------------------------------------- helpers ---

def expert_load(counts: np.ndarray) -> dict:
    """Expert Activation Skew (the untitled page at tqpw.cn, section 4.4, table
    of serving metrics): the largest activation count of an expert divided by the mean
    activation count, the mean taken over all E routed experts (experts that
    no token chose count as 0). counts[e] is the number of (token, choice)
    pairs routed to expert e. Also returns the max, the mean and the number
    of experts with at least one pair. Skew is 0 when no pair was routed."""
    c = np.asarray(counts, dtype=np.float64)
    mean = c.mean() if c.size else 0.0
    return dict(max=float(c.max()) if c.size else 0.0, mean=float(mean),
                skew=float(c.max() / mean) if mean > 0 else 0.0,
                touched=int((c > 0).sum()))


def group_counts(counts: np.ndarray, groups: int) -> np.ndarray:
    """Activation counts of the G expert groups of page "Step3.5 Flash
    大模型技术深度解析", section 3.2.3 (the routed experts split evenly into G
    groups, one per GPU; R13: group g holds the contiguous ids g*E/G ..
    (g+1)*E/G - 1): entry g is the sum of counts[e] over the experts of
    group g. E must be a multiple of G."""
    c = np.asarray(counts)
    if groups <= 0 or c.size % groups:
        raise ValueError(f"{c.size} experts do not split into {groups} equal groups")
    return c.reshape(groups, -1).sum(axis=1)


# --------------------------------------------------- expert parallelism ---

def group_stats(p64, idx, n_groups: int) -> dict:
    """Balance statistics of G contiguous expert groups (R13).

    mass[g]  = sum over tokens of sum_{e in g} p[t,e]     (p: the softmax, fp64)
    pairs[g] = number of chosen (t, slot) pairs with an expert in g
    f = pairs / sum(pairs), p = mass / T, l_ep = G * sum_g f_g p_g.
    """
    p64 = as_f64(p64)
    T, E = p64.shape
    gs = E // n_groups
    mass = np.array([p64[:, g * gs:(g + 1) * gs].sum() for g in range(n_groups)])
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    flat = flat[(flat >= 0) & (flat < E)]
    pairs = np.bincount(flat // gs, minlength=n_groups).astype(np.int64)
    f = pairs / pairs.sum() if pairs.sum() else np.zeros(n_groups)
    p = mass / T if T else np.zeros(n_groups)
    return dict(mass=mass, pairs=pairs, f=f, p=p, l_ep=float(n_groups * np.sum(f * p)))


def ep_receive_plan(counts) -> dict:
    """Expert-major order of one GPU's receive buffer (R13).

    counts[r, e]: rows of source r for local expert e; the buffer holds the
    chunks (r, e) r-major, each chunk's rows in order. Expert-major order
    takes experts in turn, sources in turn inside an expert, a chunk's rows
    in turn. gather[q] = receive row of expert-major row q; scatter is its
    inverse; offsets[e] = first expert-major row of e.
    """
    c = np.maximum(np.asarray(counts, dtype=np.int64), 0)
    R, El = c.shape
    start = np.concatenate([[0], np.cumsum(c.reshape(-1))])[:-1].reshape(R, El)   # r-major chunk starts
    gather = []
    offsets = [0]
    for e in range(El):
        for r in range(R):
            gather.extend(range(int(start[r, e]), int(start[r, e] + c[r, e])))
        offsets.append(len(gather))
    gather = np.array(gather, dtype=np.int64)
    scatter = np.empty_like(gather)
    scatter[gather] = np.arange(len(gather))
    return dict(offsets=np.array(offsets, dtype=np.int64), gather=gather, scatter=scatter)


# ------------------------------------------------------------ FP8 weights ---

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 code -> value (float64): 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 is subnormal (m * 2^-9); S.1111.111
    is NaN; there are no infinities (R14)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.where((e == 15) & (m == 7), np.nan, sign * v)


def e4m3_encode(v) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8): the nearest finite E4M3 value,
    ties to the even code, magnitudes above 448 saturating to 448 (R14).

    Within the binade [2^e, 2^(e+1)) of |v| (e >= -6; below 2^-6 the
    subnormal spacing) E4M3 values are the multiples of 2^(e-3); |v| is
    rounded to the nearest multiple, ties to the even multiple, which is the
    even code. Every step is an exact power-of-two scaling (float32 suffices).
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v), np.float32(E4M3_MAX))
    _, ex = np.frexp(a)                             # a = f 2^ex, f in [0.5, 1): binade ex - 1
    step = np.ldexp(np.float32(1.0), np.maximum(ex - 1, -6) - 3)
    r = np.minimum(np.rint(a / step) * step, np.float32(E4M3_MAX))
    _, ex2 = np.frexp(r)
    normal = r >= np.float32(2.0 ** -6)
    m = np.where(normal, np.rint(np.ldexp(r, 4 - ex2)) - 8, np.rint(np.ldexp(r, 9))).astype(np.int32)
    code = np.where(normal, ((ex2 - 1 + 7) << 3) + m, m)     # 3-bit mantissa, or m 2^-9 below 2^-6
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows_fp8(w) -> tuple:
    """Per-row FP8 quantisation of w [..., rows, cols] (R14): (codes uint8, scales float32 [..., rows])."""
    if _torch is not None and isinstance(w, _torch.Tensor):
        w32 = w.detach().cpu().float().numpy()    # bf16 / fp32 values are exact in float32
    else:
        w32 = np.asarray(w, dtype=np.float32)
    amax = np.abs(w32).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((w32 / scale[..., None]).astype(np.float32))
    return q, scale


_E4M3_ALL = e4m3_decode(np.arange(256))


def dequantize_fp8(codes, scales) -> np.ndarray:
    """decode(q) * s in float64 (exact; decode through the table of all 256 codes)."""
    return _E4M3_ALL[np.asarray(codes, dtype=np.int64)] * np.asarray(scales, dtype=np.float64)[..., None]
