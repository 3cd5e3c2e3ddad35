/*
 * moe.h - C ABI of a sparse Mixture-of-Experts FFN layer on AMD Instinct
 * MI355X (gfx950).
 *
 * The layer is the one the page "Step3.5 Flash 大模型技术深度解析：稀疏 MoE、
 * 混合注意力与 MTP 的高效推理革命" states in section 3.2.1 (per MoE layer: 288
 * routed experts, each an independent FFN, and 1 always-active shared
 * expert; model width d_model = 4096) and section 3.2.2 (Top-8 routing: a
 * linear layer plus softmax gives every routed expert a probability, the 8
 * most probable routed experts and the shared expert run, and their outputs
 * are summed with weights). For token x:
 *
 *   p      = softmax(W_r x + b)                 over all E routed experts
 *   S      = the K most probable experts        (ties: lower index first)
 *   out(x) = FFN_s(x) + sum_{e in S} p_e FFN_e(x)
 *   FFN(x) = W_d (silu(W_g x) * (W_u x))        (SwiGLU, no biases)
 *
 * The selected probabilities are used as they are (no renormalisation over
 * S); the shared expert has weight 1; no token is dropped (no capacity).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller, dense
 *    row-major (weights: or packed, below), 16-byte aligned. The library never allocates, frees or keeps
 *    a pointer past the call. The one piece of device memory it owns is the
 *    static scratch of moe_layer_forward_noalloc (below); every other entry
 *    point works only in the caller's buffers and workspace.
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *    null stream) and returns; results are valid once the stream is
 *    synchronised. No call copies device data to the host or synchronises.
 *  - Arguments are checked on the host before anything is enqueued; a
 *    failed check returns a non-zero moe_status and enqueues nothing.
 *    moe_last_error() then describes the failure (per thread).
 *  - T == 0 (no tokens / rows) is a valid no-op returning MOE_OK.
 *  - Device-side index inputs (expert ids, offsets, row maps) supplied by
 *    the caller are clamped to their valid ranges inside the kernels, so a
 *    malformed index never causes an out-of-bounds access; the results for
 *    such entries are unspecified.
 *  - Routing and permutation results are bit-deterministic. Floating-point
 *    outputs are deterministic for a fixed configuration (no atomics).
 *
 * dtype: MOE_BF16 -> x and all weights bfloat16, products accumulated in
 * fp32 on the matrix cores; MOE_F32 -> everything fp32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                    */
  MOE_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or inconsistent */
  MOE_ERR_UNSUPPORTED = 3, /* dtype or size outside what the kernels implement */
  MOE_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than *_workspace_bytes */
  MOE_ERR_MISALIGNED = 5,  /* a pointer is not 16-byte aligned             */
  MOE_ERR_HIP = 6          /* the HIP runtime reported an error (launch)   */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Storage layout of the weight matrices (see "Packed weights" below). */
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_PACKED = 1, MOE_LAYOUT_FP8 = 2 } moe_weight_layout;

/* Shape of one layer (section 3.2.1 / 3.2.2 of the page above). */
typedef struct {
  int32_t d_model;   /* D: token width (4096 on the page)                    */
  int32_t n_experts; /* E: routed experts (288); 1 <= E <= 1024              */
  int32_t top_k;     /* K: routed experts per token (8); 1 <= K <= min(E,64) */
  int32_t d_expert;  /* F: SwiGLU width of a routed expert                   */
  int32_t d_shared;  /* Fs: SwiGLU width of the shared expert; 0 = none      */
  int32_t dtype;     /* moe_dtype of x and of every weight                   */
  int32_t out_dtype; /* moe_dtype of the layer output                        */
  int32_t weight_layout; /* moe_weight_layout of every weight matrix argument  */
} moe_config;

/* The layer's weights (device pointers, row-major).
 *   w_router    [E, D]      router linear layer
 *   router_bias [E] fp32 or NULL, added to the logits before the softmax
 *   w_gate      [E, F, D]   routed experts, gate projection
 *   w_up        [E, F, D]   routed experts, up projection
 *   w_down      [E, D, F]   routed experts, down projection
 *   s_gate      [Fs, D], s_up [Fs, D], s_down [D, Fs]: the shared expert
 *               (ignored when d_shared == 0).
 *   *_scale     per-row fp32 scales of the expert matrices, used only with
 *               MOE_LAYOUT_FP8 (below): w_gate_scale, w_up_scale [E, F],
 *               w_down_scale [E, D], s_gate_scale, s_up_scale [Fs],
 *               s_down_scale [D]; NULL otherwise.                           */
typedef struct {
  const void* w_router;
  const float* router_bias;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* s_gate;
  const void* s_up;
  const void* s_down;
  const float* w_gate_scale;
  const float* w_up_scale;
  const float* w_down_scale;
  const float* s_gate_scale;
  const float* s_up_scale;
  const float* s_down_scale;
} moe_weights;

/* Packed weights
 * --------------
 * With cfg->weight_layout == MOE_LAYOUT_PACKED every weight matrix argument
 * (w_router, w_gate, w_up, w_down, s_gate, s_up, s_down) points to the
 * output of moe_pack_weights for that array instead of the row-major array.
 * This is a storage layout only, made once when weights are loaded: the
 * results are bit-identical to those with row-major weights. It exists so
 * that every weight load of the matrix-core kernels reads 1 KB contiguous.
 * It requires dtype MOE_BF16 and d_model, d_expert, d_shared (and d_ff of the
 * grouped entry points) multiples of 64 (else MOE_ERR_UNSUPPORTED).
 *
 * Layout of one matrix W [rows, cols] (cols % 32 == 0): 16-row x 32-column
 * fragments, fragment (ct, kb) = rows 16ct.., columns 32kb.., stored in the
 * order ct-major, kb-minor; a fragment is 64 lanes x 8 values where lane
 * l = c + 16q holds W[16ct + c][32kb + 8q + 0..7]. Rows past `rows` (when
 * rows % 16 != 0) are zero. A stack of n_mats matrices is packed matrix
 * after matrix.
 *
 * moe_packed_weights_bytes: bytes of the packed form of n_mats [rows, cols]
 *   bf16 matrices: n_mats * ceil(rows/16)*16 * cols * 2; SIZE_MAX when a
 *   size is negative or cols % 32 != 0.
 * moe_pack_weights: src [n_mats, rows, cols] bf16 row-major -> dst (device,
 *   >= dst_bytes = moe_packed_weights_bytes(...) bytes, not overlapping src). */
size_t moe_packed_weights_bytes(int64_t n_mats, int64_t rows, int64_t cols);
moe_status moe_pack_weights(int64_t n_mats, int64_t rows, int64_t cols, const void* src, void* dst,
                            size_t dst_bytes, void* stream);

/* FP8 expert weights
 * ------------------
 * With cfg->weight_layout == MOE_LAYOUT_FP8 the expert matrices (w_gate,
 * w_up, w_down, s_gate, s_up, s_down) are OCP FP8 E4M3 codes written by
 * moe_quantize_fp8, with one fp32 scale per matrix row (output channel) in
 * the *_scale fields of moe_weights; the weight the layer uses is
 * decode(code) * scale. Activations stay bf16 (dtype MOE_BF16), the router
 * stays bf16 in the packed layout (moe_pack_weights), and the widths must be
 * multiples of 64. Page "Step3.5 Flash 大模型技术深度解析", section 8.1,
 * deploys the model with FP8/FP16 weights. The expert GEMMs read half the
 * weight bytes and convert to bf16 in registers, with the same row tiles
 * as bf16 weights. Only
 * moe_layer_forward and moe_layer_forward_dynamic take fp8 weights (the
 * grouped expert entry points have no scale arguments: MOE_ERR_UNSUPPORTED).
 *
 * Layout of the codes of W [rows, cols] (cols % 64 == 0): fragments of 16
 * rows x 64 columns (1 KB), ct-major then kb; lane l = c + 16q (c < 16,
 * q < 4) of fragment (ct, kb) holds, at byte 16l, the codes of row 16ct + c
 * at columns 64kb + 8q .. +7, then at 64kb + 32 + 8q .. +7. Rows past
 * `rows` (when rows % 16 != 0) hold zero codes.
 *
 * moe_fp8_weights_bytes: n_mats * ceil(rows/16)*16 * cols; SIZE_MAX when a
 *   size is negative or cols % 64 != 0.
 * moe_quantize_fp8: src [n_mats, rows, cols] bf16 row-major -> dst codes
 *   (>= moe_fp8_weights_bytes bytes) and scales [n_mats, rows] fp32. Per row:
 *   scale = max|w| / 448 in fp32 (1 for an all-zero row); code = the E4M3
 *   value nearest to fp32(w / scale), ties to the even code, magnitudes
 *   above 448 saturating. */
size_t moe_fp8_weights_bytes(int64_t n_mats, int64_t rows, int64_t cols);
moe_status moe_quantize_fp8(int64_t n_mats, int64_t rows, int64_t cols, const void* src, void* dst,
                            size_t dst_bytes, float* scales, void* stream);

/* Workspace queries. They return the bytes the matching entry point needs
 * in its `ws` argument, or SIZE_MAX when the configuration is invalid. */
size_t moe_route_workspace_bytes(const moe_config* cfg, int64_t T);
size_t moe_permute_workspace_bytes(const moe_config* cfg, int64_t T);
size_t moe_grouped_ffn_workspace_bytes(const moe_config* cfg, int32_t n_groups, int64_t n_rows,
                                       int32_t d_ff);
size_t moe_layer_workspace_bytes(const moe_config* cfg, int64_t T);

/* Router (section 3.2.2, steps 1-2): logits = x W_r^T + b, softmax over all
 * E experts in fp32, then the K most probable experts per token.
 *   x          [T, D] dtype
 *   w_router   [E, D] dtype;  bias [E] fp32 or NULL
 *   topk_idx   [T, K] int32 out: expert ids, probability descending,
 *              equal probabilities ordered by lower expert id
 *   topk_prob  [T, K] fp32 out: their softmax probabilities (not renormalised)
 *   gap        [T] fp32 out or NULL: p of the K-th choice minus p of the
 *              (K+1)-th (+inf when K == E); small gaps flag near-ties
 *   ws         >= moe_route_workspace_bytes(cfg, T) bytes                   */
moe_status moe_route(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_prob, float* gap,
                     void* ws, size_t ws_bytes, void* stream);

/* Router with a per-token number of experts (dynamic top-k: page "Step3.5
 * Flash 大模型技术深度解析", section 8.2, picks 4 experts for simple inputs
 * and 8 for complex ones; page "Step 3.5 Flash动态稀疏MoE架构解析与优化实践",
 * section 2.1, 2-3 for short texts and up to 8 for long ones).
 *   k_per_token [T] int32 (device) or NULL (= moe_route): token t keeps its
 *              k_t = k_per_token[t] most probable experts, clamped to
 *              [0, K]; its slots j >= k_t get topk_idx -1 and topk_prob 0
 *   gap        as moe_route, at the token's own cut: p of its k_t-th choice
 *              minus p of the next (+inf when k_t == 0 or k_t == E)
 * Every other argument as moe_route. moe_permute, moe_combine and the
 * grouped expert entry points take pairs with expert -1 as "no expert":
 * no row, dest -1, nothing added. */
moe_status moe_route_dynamic(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                             const float* bias, const int32_t* k_per_token, int32_t* topk_idx,
                             float* topk_prob, float* gap, void* ws, size_t ws_bytes, void* stream);

/* Permutation of the T*K (token, choice) pairs into per-expert segments
 * (the grouping that lets every expert run its FFN as one dense block;
 * section 3.2.2 step 2). Pairs are taken in token-major order and kept in
 * that order inside a segment (stable), so the result is unique.
 *   topk_idx     [T, K] int32 in (ids outside [0,E) are not placed: their
 *                dest is -1 and they are not counted)
 *   offsets      [E+1] int32 out: segment e is rows offsets[e]..offsets[e+1]-1
 *   sorted_token [T*K] int32 out: token of each permuted row
 *   dest         [T*K] int32 out: permuted row of pair (t, j) at t*K+j
 *   x, x_perm    optional pair (both NULL or both set): x [T, D] dtype is
 *                gathered into x_perm [T*K, D] in permuted row order
 *   ws           >= moe_permute_workspace_bytes(cfg, T) bytes               */
moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx,
                       int32_t* offsets, int32_t* sorted_token, int32_t* dest,
                       const void* x, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU expert FFN over row segments (section 3.2.1: every expert
 * is an independent FFN). Group g (0 <= g < n_groups) owns rows
 * offsets[g]..offsets[g+1]-1 and uses weights
 *   w_gate + g*d_ff*D, w_up + g*d_ff*D  ([d_ff, D] each, dtype)
 *   w_down + g*D*d_ff                   ([D, d_ff], dtype)
 * Row r reads input row gather[r] of x (gather NULL: row r of x) and writes
 *   y[r] = W_d (silu(W_g x) * (W_u x))       y: [n_rows, D] fp32
 * The SwiGLU activation is rounded once to dtype before the down projection.
 * Rows outside every segment are left unwritten.
 *   offsets   [n_groups+1] int32, non-decreasing, offsets[n_groups] <= n_rows
 *   x         [n_x_rows, D] dtype;  gather [n_rows] int32 or NULL
 *   ws        >= moe_grouped_ffn_workspace_bytes(cfg, n_groups, n_rows, d_ff) bytes
 * The shared expert is the case n_groups = 1, offsets = {0, T}, gather NULL. */
moe_status moe_grouped_ffn(const moe_config* cfg, int32_t n_groups, int64_t n_rows,
                           const int32_t* offsets, const void* x, int64_t n_x_rows,
                           const int32_t* gather, const void* w_gate, const void* w_up,
                           const void* w_down, int32_t d_ff, float* y, void* ws,
                           size_t ws_bytes, void* stream);

/* The two halves of moe_grouped_ffn, for callers that keep the SwiGLU
 * activation or run the halves apart. Groups 0..n_groups-1 use the stacked
 * weights as in moe_grouped_ffn; when s_gate/s_up (s_down) is non-NULL one
 * more group, n_groups, owns rows offsets[n_groups]..offsets[n_groups+1]-1
 * and uses that single expert's weights ([d_ff, D] / [D, d_ff]), so
 * `offsets` then has n_groups+2 entries (the layer runs its shared expert
 * this way, in the same launch as the routed experts).
 *
 * moe_expert_gate_up: h[r] = dtype(silu(W_g x_r) * (W_u x_r)), h [n_rows, d_ff]
 *   where x_r = x[gather[r]] for r < n_gather and x[r - n_gather] otherwise
 *   (gather may be NULL only with n_gather == 0).
 * moe_expert_down: y[r] = W_d h[r] (fp32), y [n_rows, D].
 *   ws >= moe_expert_workspace_bytes(cfg, n_groups (+1 with the extra group), n_rows, d_ff) */
size_t moe_expert_workspace_bytes(const moe_config* cfg, int32_t n_groups, int64_t n_rows, int32_t d_ff);

moe_status moe_expert_gate_up(const moe_config* cfg, int32_t n_groups, int64_t n_rows,
                              const int32_t* offsets, const void* x, int64_t n_x_rows,
                              const int32_t* gather, int64_t n_gather, const void* w_gate,
                              const void* w_up, const void* s_gate, const void* s_up, int32_t d_ff,
                              void* h, void* ws, size_t ws_bytes, void* stream);

moe_status moe_expert_down(const moe_config* cfg, int32_t n_groups, int64_t n_rows,
                           const int32_t* offsets, const void* h, const void* w_down,
                           const void* s_down, int32_t d_ff, float* y, void* ws, size_t ws_bytes,
                           void* stream);

/* Weighted combine (section 3.2.2, step 3):
 *   out[t] = y_shared[t] + sum_{j=0..K-1} topk_prob[t,j] * y_perm[dest[t*K+j]]
 * summed in fp32 in that order, rounded once to out_dtype.
 *   y_perm [T*K, D] fp32; dest [T*K] int32 (-1: pair skipped);
 *   topk_prob [T, K] fp32; y_shared [T, D] fp32 or NULL; out [T, D] out_dtype */
moe_status moe_combine(const moe_config* cfg, int64_t T, const float* y_perm, const int32_t* dest,
                       const float* topk_prob, const float* y_shared, void* out, void* stream);

/* The whole layer: route, permute, routed + shared expert FFNs, combine.
 *   x     [T, D] dtype;   out [T, D] out_dtype
 *   topk_idx_out [T, K], topk_prob_out [T, K], offsets_out [E+1]: optional
 *   copies of the routing decision (NULL to skip)
 *   ws    >= moe_layer_workspace_bytes(cfg, T) bytes                        */
moe_status moe_layer_forward(const moe_config* cfg, int64_t T, const void* x,
                             const moe_weights* w, void* out, int32_t* topk_idx_out,
                             float* topk_prob_out, int32_t* offsets_out, void* ws,
                             size_t ws_bytes, void* stream);

/* The whole layer with a per-token number of experts (see
 * moe_route_dynamic): k_per_token [T] int32 (device) or NULL (= fixed K).
 * Token t's output is the shared expert plus its k_t routed experts;
 * offsets_out[E] is the number of routed pairs. Same workspace as
 * moe_layer_forward. */
moe_status moe_layer_forward_dynamic(const moe_config* cfg, int64_t T, const void* x,
                                     const moe_weights* w, const int32_t* k_per_token, void* out,
                                     int32_t* topk_idx_out, float* topk_prob_out,
                                     int32_t* offsets_out, void* ws, size_t ws_bytes,
                                     void* stream);

/* The whole layer without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments and results as
 * moe_layer_forward without ws/ws_bytes: the workspace is a static device
 * array of moe_noalloc_scratch_bytes() bytes (64 MiB) inside the library,
 * one copy per GPU, held from the first call on that GPU until the process
 * ends. Nothing is allocated or freed by the call.
 *   - Layers whose moe_layer_workspace_bytes(cfg, T) exceeds that size are
 *     rejected with MOE_ERR_WORKSPACE before anything is enqueued (at
 *     d_model 4096 and expert width 1280: up to 354 tokens).
 *   - The scratch of the current device is used (hipGetDevice); `stream`
 *     must belong to that device.
 *   - Every call on a GPU shares that GPU's scratch and leaves its contents
 *     behind (nothing in it needs to start at zero). Calls that overlap on
 *     one GPU (concurrent streams or threads) race on the scratch: the
 *     caller must order them, e.g. by issuing them on one stream.
 *   - MOE_ERR_HIP if the scratch's device address cannot be obtained. */
size_t moe_noalloc_scratch_bytes(void);
moe_status moe_layer_forward_noalloc(const moe_config* cfg, int64_t T, const void* x,
                                     const moe_weights* w, void* out, int32_t* topk_idx_out,
                                     float* topk_prob_out, int32_t* offsets_out, void* stream);

/* Expert-parallel balance statistics (page "Step3.5 Flash 大模型技术深度解析",
 * section 3.2.3: the 288 routed experts split into G equal groups, one group
 * per GPU, with the balance loss L_EP = G * sum_g f_g p_g, f_g the activation
 * frequency of group g's experts and p_g their routing probability). The
 * router as moe_route_dynamic (k_per_token may be NULL), plus
 *   n_groups   G in [1, 16], dividing E; group g = experts g*E/G .. (g+1)*E/G - 1
 *   stats      [2G] fp64 out: stats[g] = sum over tokens of the softmax mass of
 *              group g's experts (p_g = stats[g] / T); stats[G + g] = number
 *              of chosen (token, slot) pairs in group g (f_g = stats[G + g] /
 *              sum of stats[G..2G-1]). Sums over tokens run in a fixed order:
 *              the result does not depend on scheduling.
 *   ws         >= moe_route_group_stats_workspace_bytes(cfg, T, G) bytes  */
size_t moe_route_group_stats_workspace_bytes(const moe_config* cfg, int64_t T, int32_t n_groups);
moe_status moe_route_group_stats(const moe_config* cfg, int64_t T, const void* x,
                                 const void* w_router, const float* bias,
                                 const int32_t* k_per_token, int32_t n_groups, int32_t* topk_idx,
                                 float* topk_prob, double* stats, void* ws, size_t ws_bytes,
                                 void* stream);

/* Receive plan of one GPU's share under expert parallelism (section 3.2.3:
 * each GPU holds one group of experts). The dispatch exchange delivers one
 * chunk per (source rank r, local expert e), r-major, each chunk holding that
 * source's rows for e in its own (token) order: exactly the source's
 * moe_permute rows of the group's experts, so a source's send buffer is one
 * contiguous slice of its permuted rows per destination.
 *   counts   [n_src * n_local] int32 (device): rows of chunk (r, e) at
 *            r * n_local + e; negative counts count as 0; the total must be
 *            below 2^31. n_src >= 1, n_local >= 1, n_src * n_local <= 1024.
 *   offsets  [n_local + 1] int32 out: expert e's rows in expert-major order
 *            are offsets[e] .. offsets[e+1]-1 (experts in turn, sources in
 *            turn inside an expert, a chunk's rows in turn)
 *   gather   [max_rows] int32 out: expert-major row q is receive row gather[q]
 *   scatter  [max_rows] int32 out: receive row i is expert-major row scatter[i]
 * Rows at or past max_rows are not written. With `gather` as the row map of
 * moe_expert_gate_up (x = the receive buffer) the local experts run on the
 * received rows in place; moe_gather_rows with `scatter` puts their outputs
 * back in receive order, the layout the return exchange sends. */
moe_status moe_ep_receive_plan(int32_t n_src, int32_t n_local, const int32_t* counts,
                               int64_t max_rows, int32_t* offsets, int32_t* gather,
                               int32_t* scatter, void* stream);

/* Row gather: dst[i] = src[index[i]] for i < n_rows, rows of row_bytes bytes
 * (index clamped to [0, n_src_rows)). row_bytes in [1, 2^30]. */
moe_status moe_gather_rows(const void* src, int64_t n_src_rows, int64_t row_bytes,
                           const int32_t* index, int64_t n_rows, void* dst, void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* Text of the last failed check or HIP error in the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
