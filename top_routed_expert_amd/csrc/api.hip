// C ABI of libmoe (declared and documented in include/moe.h): argument
// checks on the host, workspace carving, and the launch sequence of the MoE
// layer of page "Step3.5 Flash 大模型技术深度解析", section 3.2.2:
//   route (linear + softmax + top-K) -> permute -> expert FFNs -> combine.
// Nothing here allocates, synchronises or copies device data to the host.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local char g_last_error[512];

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

moe_status ok() {
  g_last_error[0] = 0;
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY_HIP(expr, what)                          \
  do {                                                   \
    const moe_status _s = hip_status((expr), (what));    \
    if (_s != MOE_OK) return _s;                         \
  } while (0)

#define MOE_TRY(expr)                \
  do {                               \
    const moe_status _s = (expr);    \
    if (_s != MOE_OK) return _s;     \
  } while (0)

constexpr size_t kAlign = 256;
constexpr int64_t kMaxRows = (int64_t)1 << 31;

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

size_t elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Carves aligned sub-buffers out of the caller's workspace; with a NULL
// base it only measures.
struct Arena {
  char* base;
  size_t off = 0;
  explicit Arena(void* b) : base((char*)b) {}
  template <typename T>
  T* take(int64_t n) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? (T*)(base + off) : nullptr;
    off += (size_t)(n > 0 ? n : 0) * sizeof(T);
    return p;
  }
  void* take_bytes(int64_t n) { return take<char>(n); }
};

moe_status check_cfg(const moe_config* c) {
  if (!c) return fail(MOE_ERR_NULL, "cfg is NULL");
  if (c->d_model <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->d_expert <= 0 || c->d_shared < 0)
    return fail(MOE_ERR_SHAPE, "d_model, n_experts, top_k, d_expert must be > 0 and d_shared >= 0");
  if (c->top_k > c->n_experts) return fail(MOE_ERR_SHAPE, "top_k %d > n_experts %d", c->top_k, c->n_experts);
  if (c->n_experts > 1024) return fail(MOE_ERR_UNSUPPORTED, "n_experts %d > 1024", c->n_experts);
  if (c->top_k > 64) return fail(MOE_ERR_UNSUPPORTED, "top_k %d > 64", c->top_k);
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "dtype %d", c->dtype);
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "out_dtype %d", c->out_dtype);
  if (c->weight_layout != MOE_LAYOUT_ROWS && c->weight_layout != MOE_LAYOUT_PACKED &&
      c->weight_layout != MOE_LAYOUT_FP8)
    return fail(MOE_ERR_UNSUPPORTED, "weight_layout %d", c->weight_layout);
  if (c->weight_layout != MOE_LAYOUT_ROWS &&
      (c->dtype != MOE_BF16 || c->d_model % 64 || c->d_expert % 64 || c->d_shared % 64))
    return fail(MOE_ERR_UNSUPPORTED,
                "packed and fp8 weights need bf16 and d_model, d_expert, d_shared multiples of 64");
  return MOE_OK;
}

// bf16 weights in the packed layout: every weight with MOE_LAYOUT_PACKED, the
// router with MOE_LAYOUT_FP8 (only expert matrices are fp8)
bool packed(const moe_config* c) { return c->weight_layout != MOE_LAYOUT_ROWS; }
bool fp8(const moe_config* c) { return c->weight_layout == MOE_LAYOUT_FP8; }

moe_status check_tokens(const moe_config* c, int64_t T) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T = %lld < 0", (long long)T);
  if ((T + 1) * (int64_t)(c->top_k + 1) >= kMaxRows)
    return fail(MOE_ERR_UNSUPPORTED, "T*(top_k+1) must stay below 2^31 rows");
  return MOE_OK;
}

// bf16 MFMA path: contraction lengths (d_model and the FFN widths) multiple of 64.
bool fast_path(int dtype, int D, int F) { return dtype == MOE_BF16 && D % 64 == 0 && F % 64 == 0; }

// ---- workspace layouts (shared by the size queries and the entry points) ----

struct RouteWs {
  float* logits;
};
int route_ksplit(const moe_config* c, int64_t T) {
  const bool fast = fast_path(c->dtype, c->d_model, 64);
  if (fast && router_topk_fits(T, c->d_model, c->n_experts, c->top_k)) return 1;  // no partial sums
  return router_ksplit(fast, T, c->d_model, c->n_experts);
}
RouteWs carve_route(Arena& a, const moe_config* c, int64_t T) {
  return {a.take<float>(route_ksplit(c, T) * T * c->n_experts)};
}

struct PermuteWs {
  int32_t* rank;
  int32_t* counts;
};
PermuteWs carve_permute(Arena& a, const moe_config* c, int64_t T) {
  PermuteWs w;
  w.rank = a.take<int32_t>(T * c->top_k);
  w.counts = a.take<int32_t>(c->n_experts);
  return w;
}

// Tile schedule of a grouped expert launch (and, for the full FFN, the
// SwiGLU activations between its two halves).
struct SchedWs {
  Tile* tiles;
  int32_t* n_tiles;
  bool fast;  // bf16 matrix-core kernels (else the generic 64 x 64 kernel)
  int block_rows;
  int32_t max_tiles;
};
SchedWs carve_sched(Arena& a, const moe_config* c, int n_groups, int64_t n_rows, int d_ff) {
  SchedWs w;
  w.fast = fast_path(c->dtype, c->d_model, d_ff);
  // 256-row tiles need contractions of at least 128 and A offsets that fit
  // 32 bits in 16-byte units (A has at most n_rows rows of either width)
  const int64_t kmax = c->d_model > d_ff ? c->d_model : d_ff;
  const bool big_ok = c->d_model >= 128 && d_ff >= 128 && (uint64_t)n_rows * (uint64_t)kmax / 8u <= 0xffffffffull;
  w.block_rows = gemm_block_rows(w.fast, n_rows, n_groups, big_ok);
  w.max_tiles = (int32_t)gemm_max_tiles(n_rows, n_groups, w.block_rows);
  w.tiles = a.take<Tile>(w.max_tiles);
  w.n_tiles = a.take<int32_t>(1);
  return w;
}

struct FfnWs {
  SchedWs sched;
  void* h;
};
FfnWs carve_ffn(Arena& a, const moe_config* c, int n_groups, int64_t n_rows, int d_ff) {
  FfnWs w;
  w.sched = carve_sched(a, c, n_groups, n_rows, d_ff);
  w.h = a.take_bytes(n_rows * (int64_t)d_ff * (int64_t)elem_bytes(c->dtype));
  return w;
}

struct LayerWs {
  RouteWs route;
  PermuteWs perm;
  int32_t* idx;
  float* prob;
  int32_t* offsets_ext;  // [E+2]: routed segments, then the shared expert's rows
  int32_t* sorted_token;
  int32_t* dest;
  FfnWs ffn;             // routed (+ fused shared) expert rows
  FfnWs ffn_shared;      // shared expert on its own when its width differs
  float* y;              // [T*K (+T), D] fp32 (NULL with y16)
  float* y_shared;       // [T, D] fp32: the shared expert's rows
  bool fused_shared;
  // routed expert outputs in the 16-bit format (moe_internal.h) when the down
  // projection runs on 256-row tiles: half the bytes written by the down GEMM
  // and read by the combine
  bool y16;
  uint16_t* y16v;        // [T*K, D]
  uint8_t* y16e;         // [T*K, D/64]
};
LayerWs carve_layer(Arena& a, const moe_config* c, int64_t T) {
  LayerWs w{};
  const int64_t P = T * c->top_k;
  const bool shared = c->d_shared > 0;
  w.fused_shared = shared && c->d_shared == c->d_expert;
  w.route = carve_route(a, c, T);
  w.perm = carve_permute(a, c, T);
  w.idx = a.take<int32_t>(P);
  w.prob = a.take<float>(P);
  w.offsets_ext = a.take<int32_t>(c->n_experts + 3);
  w.sorted_token = a.take<int32_t>(P);
  w.dest = a.take<int32_t>(P);
  const int64_t rows = P + (w.fused_shared ? T : 0);
  w.ffn = carve_ffn(a, c, c->n_experts + (w.fused_shared ? 2 : 0), rows, c->d_expert);
  if (shared && !w.fused_shared) w.ffn_shared = carve_ffn(a, c, 1, T, c->d_shared);
  w.y16 = w.ffn.sched.block_rows == 256 && c->d_model % 64 == 0;
  if (w.y16) {
    w.y16v = a.take<uint16_t>(P * c->d_model);
    w.y16e = a.take<uint8_t>(P * (c->d_model / 64));
    w.y_shared = shared ? a.take<float>(T * c->d_model) : nullptr;
  } else {
    w.y = a.take<float>((P + (shared ? T : 0)) * c->d_model);
    w.y_shared = shared ? w.y + P * c->d_model : nullptr;
  }
  return w;
}

// ---- launch sequences ----

moe_status run_route(const moe_config* c, int64_t T, const void* x, const void* w_router, const float* bias,
                     const int32_t* k_tok, int32_t* idx, float* prob, float* gap, const RouteWs& ws, hipStream_t s,
                     float* gmass = nullptr, int G = 0) {
  const bool fast = fast_path(c->dtype, c->d_model, 64);
  // many tokens: linear layer, softmax and top-K in one kernel
  if (fast && router_topk_fits(T, c->d_model, c->n_experts, c->top_k)) {
    MOE_TRY_HIP(launch_router_topk((const bf16_t*)x, T, c->d_model, (const bf16_t*)w_router, packed(c), bias,
                                   c->n_experts, c->top_k, k_tok, idx, prob, gap, gmass, G, s),
                "router");
    return MOE_OK;
  }
  GemmArgs g{};
  g.a = x;
  g.n_a_rows = T;
  g.b0 = w_router;
  g.n_main = 1;
  g.N = c->n_experts;
  g.Kdim = c->d_model;
  g.dense_rows = T;
  // the router is one group read by every row tile: up to 32 tokens take
  // one 32-row tile, more follow the expert GEMMs' rule
  const int BM = fast && T <= 32 ? 32 : gemm_block_rows(fast, T, 1, false);
  g.max_tiles = (int32_t)((T + BM - 1) / BM);
  g.out = ws.logits;
  g.ldo = c->n_experts;
  g.bias = bias;
  g.b_packed = packed(c);
  g.b_reuse = 1;
  g.ksplit = route_ksplit(c, T);
  g.slice_stride = T * c->n_experts;
  MOE_TRY_HIP(launch_grouped_gemm(c->dtype, fast, EPI_F32, BM, g, s), "router linear layer");
  MOE_TRY_HIP(launch_topk(ws.logits, g.ksplit, T, c->n_experts, c->top_k, k_tok, idx, prob, gap, gmass, G, s),
              "router top-k");
  return MOE_OK;
}

// Row tiles of a grouped launch: from `offsets` (built on the device when
// `build` is set), or dense rows of a single group when offsets is NULL.
moe_status fill_tiles(GemmArgs& g, const SchedWs& ws, const int32_t* offsets, int n_groups, int64_t n_rows,
                      bool build, int skip_group, hipStream_t s) {
  g.ksplit = 1;
  if (offsets && build)
    MOE_TRY_HIP(launch_build_tiles(offsets, n_groups, n_rows, ws.block_rows, ws.tiles, ws.n_tiles, ws.max_tiles,
                                   skip_group, s),
                "tile schedule");
  g.tiles = offsets ? ws.tiles : nullptr;
  g.n_tiles = offsets ? ws.n_tiles : nullptr;
  g.dense_rows = n_rows;
  g.max_tiles = offsets ? ws.max_tiles : (int32_t)((n_rows + ws.block_rows - 1) / ws.block_rows);
  return MOE_OK;
}

// Gate/up half. Groups g < n_main use the stacked weights (+ g*stride);
// group n_main (present when n_groups > n_main) uses s_gate/s_up.
moe_status run_gate_up(const moe_config* c, const SchedWs& ws, bool build, int n_groups, int n_main, int64_t n_rows,
                       const int32_t* offsets, const void* x, int64_t n_x_rows, const int32_t* gather,
                       int64_t n_gather, const void* w_gate, const void* w_up, const void* s_gate, const void* s_up,
                       int d_ff, void* h, hipStream_t s, int skip_group = -1, const float* const* scales = nullptr) {
  GemmArgs g{};
  MOE_TRY(fill_tiles(g, ws, offsets, n_groups, n_rows, build, skip_group, s));
  if (fp8(c)) {  // scales: gate, up, shared gate, shared up
    g.b_fp8 = 1;
    g.s0 = scales[0];
    g.s1 = scales[1];
    g.s0_extra = scales[2];
    g.s1_extra = scales[3];
    g.s_stride = d_ff;
  }
  g.a = x;
  g.n_a_rows = n_x_rows;
  g.gather = gather;
  g.n_gather = n_gather;
  g.b0 = w_gate;
  g.b1 = w_up;
  g.b0_extra = s_gate;
  g.b1_extra = s_up;
  g.b_stride = (int64_t)d_ff * c->d_model;
  g.n_main = n_main;
  g.N = d_ff;
  g.Kdim = c->d_model;
  g.out = h;
  g.ldo = d_ff;
  g.b_packed = packed(c);
  MOE_TRY_HIP(launch_grouped_gemm(c->dtype, ws.fast, EPI_SWIGLU, ws.block_rows, g, s), "expert gate/up projection");
  return MOE_OK;
}

// y16 (optional): rows below y16_rows in the 16-bit format (y16, y16_exp); the
// rest go to y at row r - y16_rows.
moe_status run_down(const moe_config* c, const SchedWs& ws, bool build, int n_groups, int n_main, int64_t n_rows,
                    const int32_t* offsets, const void* h, const void* w_down, const void* s_down, int d_ff, float* y,
                    hipStream_t s, const float* const* scales = nullptr, uint16_t* y16 = nullptr,
                    uint8_t* y16_exp = nullptr, int64_t y16_rows = 0) {
  GemmArgs g{};
  g.out16 = y16;
  g.out16_exp = y16_exp;
  g.out16_rows = y16_rows;
  MOE_TRY(fill_tiles(g, ws, offsets, n_groups, n_rows, build, -1, s));
  if (fp8(c)) {  // scales: down, shared down
    g.b_fp8 = 1;
    g.s0 = scales[0];
    g.s0_extra = scales[1];
    g.s_stride = c->d_model;
  }
  g.a = h;
  g.n_a_rows = n_rows;
  g.b0 = w_down;
  g.b0_extra = s_down;
  g.b_stride = (int64_t)c->d_model * d_ff;
  g.n_main = n_main;
  g.N = c->d_model;
  g.Kdim = d_ff;
  g.out = y;
  g.ldo = c->d_model;
  g.b_packed = packed(c);
  MOE_TRY_HIP(launch_grouped_gemm(c->dtype, ws.fast, EPI_F32, ws.block_rows, g, s), "expert down projection");
  return MOE_OK;
}

// Both halves on one schedule.
moe_status run_ffn(const moe_config* c, int n_groups, int n_main, int64_t n_rows, const int32_t* offsets,
                   const void* x, int64_t n_x_rows, const int32_t* gather, int64_t n_gather, const void* w_gate,
                   const void* w_up, const void* w_down, const void* s_gate, const void* s_up, const void* s_down,
                   int d_ff, float* y, const FfnWs& ws, hipStream_t s, bool tiles_ready = false,
                   int skip_group = -1, const float* const* scales = nullptr, uint16_t* y16 = nullptr,
                   uint8_t* y16_exp = nullptr, int64_t y16_rows = 0) {
  // scales (fp8 weights): gate, up, down of the main group, then of the extra group
  const float* gu[4] = {nullptr, nullptr, nullptr, nullptr};
  const float* dn[2] = {nullptr, nullptr};
  if (scales) {
    gu[0] = scales[0], gu[1] = scales[1], gu[2] = scales[3], gu[3] = scales[4];
    dn[0] = scales[2], dn[1] = scales[5];
  }
  MOE_TRY(run_gate_up(c, ws.sched, !tiles_ready, n_groups, n_main, n_rows, offsets, x, n_x_rows, gather, n_gather,
                      w_gate, w_up, s_gate, s_up, d_ff, ws.h, s, skip_group, gu));
  MOE_TRY(run_down(c, ws.sched, false, n_groups, n_main, n_rows, offsets, ws.h, w_down, s_down, d_ff, y, s, dn, y16,
                   y16_exp, y16_rows));
  return MOE_OK;
}

// Shared checks of the grouped expert entry points.
moe_status check_grouped(const moe_config* cfg, int32_t n_groups, int64_t n_rows, int32_t d_ff) {
  MOE_TRY(check_cfg(cfg));
  if (n_groups <= 0 || n_groups > 1025) return fail(MOE_ERR_SHAPE, "n_groups %d outside [1, 1025]", n_groups);
  if (n_rows < 0 || n_rows >= kMaxRows || d_ff <= 0)
    return fail(MOE_ERR_SHAPE, "n_rows must be in [0, 2^31) and d_ff > 0");
  if (cfg->dtype == MOE_BF16 && (cfg->d_model % 8 || d_ff % 8))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 rows need d_model and d_ff multiples of 8");
  if (packed(cfg) && d_ff % 64) return fail(MOE_ERR_UNSUPPORTED, "packed weights need d_ff %% 64 == 0");
  if (fp8(cfg))
    return fail(MOE_ERR_UNSUPPORTED, "fp8 weights need their scales: only moe_layer_forward[_dynamic] takes them");
  return MOE_OK;
}

// Pointer and shape checks of the whole-layer entry points (cfg and T checked before).
moe_status check_layer_args(const moe_config* cfg, const void* x, const moe_weights* w, const int32_t* k_per_token,
                            const void* out, const int32_t* topk_idx_out, const float* topk_prob_out,
                            const int32_t* offsets_out) {
  if (!x || !w || !out) return fail(MOE_ERR_NULL, "x, w and out are required");
  if (!w->w_router || !w->w_gate || !w->w_up || !w->w_down)
    return fail(MOE_ERR_NULL, "router and routed expert weights are required");
  const bool shared = cfg->d_shared > 0;
  if (shared && (!w->s_gate || !w->s_up || !w->s_down))
    return fail(MOE_ERR_NULL, "d_shared > 0 needs s_gate, s_up and s_down");
  if (fp8(cfg) && (!w->w_gate_scale || !w->w_up_scale || !w->w_down_scale ||
                   (shared && (!w->s_gate_scale || !w->s_up_scale || !w->s_down_scale))))
    return fail(MOE_ERR_NULL, "fp8 weights need the scales of every expert matrix");
  if (fp8(cfg) && (misaligned(w->w_gate_scale) || misaligned(w->w_up_scale) || misaligned(w->w_down_scale) ||
                   misaligned(w->s_gate_scale) || misaligned(w->s_up_scale) || misaligned(w->s_down_scale)))
    return fail(MOE_ERR_MISALIGNED, "moe_layer_forward: a scale pointer is not 16-byte aligned");
  if (misaligned(x) || misaligned(out) || misaligned(w->w_router) || misaligned(w->router_bias) ||
      misaligned(w->w_gate) || misaligned(w->w_up) || misaligned(w->w_down) ||
      (shared && (misaligned(w->s_gate) || misaligned(w->s_up) || misaligned(w->s_down))) ||
      misaligned(topk_idx_out) || misaligned(topk_prob_out) || misaligned(offsets_out) ||
      misaligned(k_per_token))
    return fail(MOE_ERR_MISALIGNED, "moe_layer_forward: a pointer is not 16-byte aligned");
  if (cfg->dtype == MOE_BF16 && (cfg->d_model % 8 || cfg->d_expert % 8 || (shared && cfg->d_shared % 8)))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 rows need d_model, d_expert, d_shared multiples of 8");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "invalid shape";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error; }

size_t moe_packed_weights_bytes(int64_t n_mats, int64_t rows, int64_t cols) {
  if (n_mats < 0 || rows < 0 || cols < 0 || cols % 32) return SIZE_MAX;
  return (size_t)n_mats * (size_t)((rows + 15) / 16 * 16) * (size_t)cols * 2u;
}

moe_status moe_pack_weights(int64_t n_mats, int64_t rows, int64_t cols, const void* src, void* dst,
                            size_t dst_bytes, void* stream) {
  const size_t need = moe_packed_weights_bytes(n_mats, rows, cols);
  if (need == SIZE_MAX) return fail(MOE_ERR_SHAPE, "pack: sizes must be >= 0 and cols a multiple of 32");
  if (need == 0) return ok();
  if (!src || !dst) return fail(MOE_ERR_NULL, "pack: src and dst are required");
  if (misaligned(src) || misaligned(dst)) return fail(MOE_ERR_MISALIGNED, "pack: src and dst must be 16-byte aligned");
  if (dst_bytes < need) return fail(MOE_ERR_WORKSPACE, "pack: dst has %zu bytes, %zu needed", dst_bytes, need);
  MOE_TRY_HIP(launch_pack((const bf16_t*)src, n_mats, rows, cols, (bf16_t*)dst, (hipStream_t)stream), "pack weights");
  return ok();
}

size_t moe_route_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK) return SIZE_MAX;
  Arena a(nullptr);
  carve_route(a, cfg, T);
  return a.off;
}

size_t moe_permute_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK) return SIZE_MAX;
  Arena a(nullptr);
  carve_permute(a, cfg, T);
  return a.off;
}

size_t moe_grouped_ffn_workspace_bytes(const moe_config* cfg, int32_t n_groups, int64_t n_rows, int32_t d_ff) {
  if (check_cfg(cfg) != MOE_OK || n_groups <= 0 || n_groups > 1025 || n_rows < 0 || n_rows >= kMaxRows || d_ff <= 0)
    return SIZE_MAX;
  Arena a(nullptr);
  carve_ffn(a, cfg, n_groups, n_rows, d_ff);
  return a.off;
}

size_t moe_layer_workspace_bytes(const moe_config* cfg, int64_t T) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK) return SIZE_MAX;
  Arena a(nullptr);
  carve_layer(a, cfg, T);
  return a.off;
}

moe_status moe_route_dynamic(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                             const float* bias, const int32_t* k_per_token, int32_t* topk_idx, float* topk_prob,
                             float* gap, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(cfg, T));
  if (T == 0) return ok();
  if (!x || !w_router || !topk_idx || !topk_prob || !ws)
    return fail(MOE_ERR_NULL, "x, w_router, topk_idx, topk_prob and ws are required");
  if (misaligned(x) || misaligned(w_router) || misaligned(bias) || misaligned(topk_idx) || misaligned(topk_prob) ||
      misaligned(gap) || misaligned(ws))
    return fail(MOE_ERR_MISALIGNED, "moe_route: a pointer is not 16-byte aligned");
  if (misaligned(k_per_token)) return fail(MOE_ERR_MISALIGNED, "moe_route: k_per_token is not 16-byte aligned");
  if (cfg->dtype == MOE_BF16 && cfg->d_model % 8)
    return fail(MOE_ERR_UNSUPPORTED, "bf16 rows need d_model % 8 == 0");
  const size_t need = moe_route_workspace_bytes(cfg, T);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_route needs %zu workspace bytes, got %zu", need, ws_bytes);
  Arena a(ws);
  const RouteWs w = carve_route(a, cfg, T);
  MOE_TRY(run_route(cfg, T, x, w_router, bias, k_per_token, topk_idx, topk_prob, gap, w, (hipStream_t)stream));
  return ok();
}

moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx, int32_t* offsets,
                       int32_t* sorted_token, int32_t* dest, const void* x, void* x_perm, void* ws, size_t ws_bytes,
                       void* stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(cfg, T));
  if (T == 0) {
    // empty input: every segment is empty
    return ok();
  }
  if (!topk_idx || !offsets || !sorted_token || !dest || !ws)
    return fail(MOE_ERR_NULL, "topk_idx, offsets, sorted_token, dest and ws are required");
  if ((x == nullptr) != (x_perm == nullptr)) return fail(MOE_ERR_NULL, "x and x_perm must be both set or both NULL");
  if (misaligned(topk_idx) || misaligned(offsets) || misaligned(sorted_token) || misaligned(dest) || misaligned(x) ||
      misaligned(x_perm) || misaligned(ws))
    return fail(MOE_ERR_MISALIGNED, "moe_permute: a pointer is not 16-byte aligned");
  const size_t need = moe_permute_workspace_bytes(cfg, T);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_permute needs %zu workspace bytes, got %zu", need, ws_bytes);
  Arena a(ws);
  const PermuteWs w = carve_permute(a, cfg, T);
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY_HIP(launch_permute(topk_idx, T, cfg->top_k, cfg->n_experts, w.rank, w.counts, offsets, sorted_token, dest,
                             nullptr, 0, nullptr, nullptr, 0, 0, s),
              "permute");
  if (x_perm)
    MOE_TRY_HIP(launch_gather_rows(x, T, cfg->d_model, (int)elem_bytes(cfg->dtype), sorted_token, T * cfg->top_k,
                                   x_perm, s),
                "row gather");
  return ok();
}

size_t moe_expert_workspace_bytes(const moe_config* cfg, int32_t n_groups, int64_t n_rows, int32_t d_ff) {
  if (check_cfg(cfg) != MOE_OK || n_groups <= 0 || n_groups > 1025 || n_rows < 0 || n_rows >= kMaxRows || d_ff <= 0)
    return SIZE_MAX;
  Arena a(nullptr);
  carve_sched(a, cfg, n_groups, n_rows, d_ff);
  return a.off;
}

moe_status moe_expert_gate_up(const moe_config* cfg, int32_t n_groups, int64_t n_rows, const int32_t* offsets,
                              const void* x, int64_t n_x_rows, const int32_t* gather, int64_t n_gather,
                              const void* w_gate, const void* w_up, const void* s_gate, const void* s_up,
                              int32_t d_ff, void* h, void* ws, size_t ws_bytes, void* stream) {
  const int total = n_groups + ((s_gate || s_up) ? 1 : 0);
  MOE_TRY(check_grouped(cfg, total, n_rows, d_ff));
  if (n_x_rows < 0 || n_gather < 0 || n_gather > n_rows)
    return fail(MOE_ERR_SHAPE, "need n_x_rows >= 0 and 0 <= n_gather <= n_rows");
  if (n_rows == 0) return ok();
  if (n_x_rows == 0) return fail(MOE_ERR_SHAPE, "n_rows > 0 needs n_x_rows > 0");
  if (!offsets || !x || !w_gate || !w_up || !h || !ws || (n_gather > 0 && !gather))
    return fail(MOE_ERR_NULL, "offsets, x, w_gate, w_up, h, ws (and gather when n_gather > 0) are required");
  if ((s_gate == nullptr) != (s_up == nullptr)) return fail(MOE_ERR_NULL, "s_gate and s_up go together");
  if (misaligned(offsets) || misaligned(x) || misaligned(gather) || misaligned(w_gate) || misaligned(w_up) ||
      misaligned(s_gate) || misaligned(s_up) || misaligned(h) || misaligned(ws))
    return fail(MOE_ERR_MISALIGNED, "moe_expert_gate_up: a pointer is not 16-byte aligned");
  const size_t need = moe_expert_workspace_bytes(cfg, total, n_rows, d_ff);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_gate_up needs %zu workspace bytes, got %zu", need, ws_bytes);
  Arena a(ws);
  const SchedWs w = carve_sched(a, cfg, total, n_rows, d_ff);
  MOE_TRY(run_gate_up(cfg, w, true, total, n_groups, n_rows, offsets, x, n_x_rows, gather, n_gather, w_gate, w_up,
                      s_gate, s_up, d_ff, h, (hipStream_t)stream));
  return ok();
}

moe_status moe_expert_down(const moe_config* cfg, int32_t n_groups, int64_t n_rows, const int32_t* offsets,
                           const void* h, const void* w_down, const void* s_down, int32_t d_ff, float* y, void* ws,
                           size_t ws_bytes, void* stream) {
  const int total = n_groups + (s_down ? 1 : 0);
  MOE_TRY(check_grouped(cfg, total, n_rows, d_ff));
  if (n_rows == 0) return ok();
  if (!offsets || !h || !w_down || !y || !ws)
    return fail(MOE_ERR_NULL, "offsets, h, w_down, y and ws are required");
  if (misaligned(offsets) || misaligned(h) || misaligned(w_down) || misaligned(s_down) || misaligned(y) ||
      misaligned(ws))
    return fail(MOE_ERR_MISALIGNED, "moe_expert_down: a pointer is not 16-byte aligned");
  const size_t need = moe_expert_workspace_bytes(cfg, total, n_rows, d_ff);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_down needs %zu workspace bytes, got %zu", need, ws_bytes);
  Arena a(ws);
  const SchedWs w = carve_sched(a, cfg, total, n_rows, d_ff);
  MOE_TRY(run_down(cfg, w, true, total, n_groups, n_rows, offsets, h, w_down, s_down, d_ff, y, (hipStream_t)stream));
  return ok();
}

moe_status moe_grouped_ffn(const moe_config* cfg, int32_t n_groups, int64_t n_rows, const int32_t* offsets,
                           const void* x, int64_t n_x_rows, const int32_t* gather, const void* w_gate,
                           const void* w_up, const void* w_down, int32_t d_ff, float* y, void* ws, size_t ws_bytes,
                           void* stream) {
  MOE_TRY(check_grouped(cfg, n_groups, n_rows, d_ff));
  if (n_x_rows < 0) return fail(MOE_ERR_SHAPE, "n_x_rows < 0");
  if (n_rows == 0) return ok();
  if (n_x_rows == 0) return fail(MOE_ERR_SHAPE, "n_rows > 0 needs n_x_rows > 0");
  if (!offsets || !x || !w_gate || !w_up || !w_down || !y || !ws)
    return fail(MOE_ERR_NULL, "offsets, x, w_gate, w_up, w_down, y and ws are required");
  if (misaligned(offsets) || misaligned(x) || misaligned(gather) || misaligned(w_gate) || misaligned(w_up) ||
      misaligned(w_down) || misaligned(y) || misaligned(ws))
    return fail(MOE_ERR_MISALIGNED, "moe_grouped_ffn: a pointer is not 16-byte aligned");
  const size_t need = moe_grouped_ffn_workspace_bytes(cfg, n_groups, n_rows, d_ff);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_ffn needs %zu workspace bytes, got %zu", need, ws_bytes);
  Arena a(ws);
  const FfnWs w = carve_ffn(a, cfg, n_groups, n_rows, d_ff);
  MOE_TRY(run_ffn(cfg, n_groups, n_groups, n_rows, offsets, x, n_x_rows, gather, gather ? n_rows : 0, w_gate, w_up,
                  w_down, nullptr, nullptr, nullptr, d_ff, y, w, (hipStream_t)stream));
  return ok();
}

moe_status moe_combine(const moe_config* cfg, int64_t T, const float* y_perm, const int32_t* dest,
                       const float* topk_prob, const float* y_shared, void* out, void* stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(cfg, T));
  if (T == 0) return ok();
  if (!y_perm || !dest || !topk_prob || !out) return fail(MOE_ERR_NULL, "y_perm, dest, topk_prob and out are required");
  if (misaligned(y_perm) || misaligned(dest) || misaligned(topk_prob) || misaligned(y_shared) || misaligned(out))
    return fail(MOE_ERR_MISALIGNED, "moe_combine: a pointer is not 16-byte aligned");
  MOE_TRY_HIP(launch_combine(cfg->out_dtype, T, cfg->d_model, cfg->top_k, y_perm, T * cfg->top_k, dest, topk_prob,
                             y_shared, out, (hipStream_t)stream),
              "combine");
  return ok();
}

moe_status moe_layer_forward_dynamic(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w,
                                     const int32_t* k_per_token, void* out, int32_t* topk_idx_out,
                                     float* topk_prob_out, int32_t* offsets_out, void* ws, size_t ws_bytes,
                                     void* stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(cfg, T));
  if (T == 0) return ok();
  if (!ws) return fail(MOE_ERR_NULL, "ws is required");
  if (misaligned(ws)) return fail(MOE_ERR_MISALIGNED, "moe_layer_forward: ws is not 16-byte aligned");
  MOE_TRY(check_layer_args(cfg, x, w, k_per_token, out, topk_idx_out, topk_prob_out, offsets_out));
  const size_t need = moe_layer_workspace_bytes(cfg, T);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_layer_forward needs %zu workspace bytes, got %zu", need, ws_bytes);

  Arena a(ws);
  const LayerWs L = carve_layer(a, cfg, T);
  hipStream_t s = (hipStream_t)stream;
  const int E = cfg->n_experts, K = cfg->top_k, D = cfg->d_model;
  const int64_t P = T * K;
  int32_t* idx = topk_idx_out ? topk_idx_out : L.idx;
  float* prob = topk_prob_out ? topk_prob_out : L.prob;

  // 1. router: linear layer + softmax over all E experts + top-K
  MOE_TRY(run_route(cfg, T, x, w->w_router, w->router_bias, k_per_token, idx, prob, nullptr, L.route, s));
  // 2. permute pairs into expert segments; the shared expert's T rows start at
  //    row T*K (pairs without an expert, under dynamic top-k, leave the rows
  //    between the routed segments and T*K unused). Small batches do it, and
  //    the expert-GEMM tile table, in one block.
  const int32_t extra = L.fused_shared ? (int32_t)T : 0;
  const bool small = permute_small_fits(T, K, E);
  if (small) {
    MOE_TRY_HIP(launch_permute_small(idx, T, K, E, offsets_out, L.sorted_token, L.dest, L.offsets_ext, extra,
                                     L.ffn.sched.tiles, L.ffn.sched.n_tiles, L.ffn.sched.max_tiles,
                                     L.ffn.sched.block_rows, s),
                "permute");
  } else {  // the place kernel writes the tile table too
    MOE_TRY_HIP(launch_permute(idx, T, K, E, L.perm.rank, L.perm.counts, offsets_out, L.sorted_token, L.dest,
                               L.offsets_ext, extra, L.ffn.sched.tiles, L.ffn.sched.n_tiles, L.ffn.sched.max_tiles,
                               L.ffn.sched.block_rows, s),
                "permute");
  }
  // 3. expert FFNs: routed segments (rows gathered through sorted_token) and,
  //    when widths match, the shared expert as one more group over x itself
  //    (group E+1; group E, the unused rows, gets no tiles)
  const int n_groups = E + (L.fused_shared ? 2 : 0);
  const float* sc[6] = {w->w_gate_scale, w->w_up_scale, w->w_down_scale, w->s_gate_scale, w->s_up_scale,
                        w->s_down_scale};
  //    (with y16, routed rows below T*K in the 16-bit format, shared rows to y_shared)
  MOE_TRY(run_ffn(cfg, n_groups, E, P + extra, L.offsets_ext, x, T, L.sorted_token, P, w->w_gate, w->w_up,
                  w->w_down, w->s_gate, w->s_up, w->s_down, cfg->d_expert, L.y16 ? L.y_shared : L.y, L.ffn, s,
                  true, L.fused_shared ? E : -1, sc, L.y16v, L.y16e, L.y16 ? P : 0));
  if (cfg->d_shared > 0 && !L.fused_shared) {
    const float* sc_shared[6] = {w->s_gate_scale, w->s_up_scale, w->s_down_scale, nullptr, nullptr, nullptr};
    MOE_TRY(run_ffn(cfg, 1, 1, T, nullptr, x, T, nullptr, 0, w->s_gate, w->s_up, w->s_down, nullptr, nullptr,
                    nullptr, cfg->d_shared, L.y_shared, L.ffn_shared, s, false, -1, sc_shared));
  }
  // 4. weighted combine: shared + sum_k prob * routed, one rounding to out_dtype
  if (L.y16)
    MOE_TRY_HIP(launch_combine16(cfg->out_dtype, T, D, K, L.y16v, L.y16e, P, L.dest, prob, L.y_shared, out, s),
                "combine");
  else
    MOE_TRY_HIP(launch_combine(cfg->out_dtype, T, D, K, L.y, P, L.dest, prob, L.y_shared, out, s), "combine");
  return ok();
}

size_t moe_route_group_stats_workspace_bytes(const moe_config* cfg, int64_t T, int32_t n_groups) {
  if (check_cfg(cfg) != MOE_OK || check_tokens(cfg, T) != MOE_OK || n_groups < 1 || n_groups > 16 ||
      cfg->n_experts % n_groups)
    return SIZE_MAX;
  Arena a(nullptr);
  carve_route(a, cfg, T);
  a.take<float>(T * n_groups);
  a.take<double>(group_stats_partials(T, n_groups));
  return a.off;
}

moe_status moe_route_group_stats(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                                 const float* bias, const int32_t* k_per_token, int32_t n_groups,
                                 int32_t* topk_idx, float* topk_prob, double* stats, void* ws, size_t ws_bytes,
                                 void* stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(cfg, T));
  if (n_groups < 1 || n_groups > 16 || cfg->n_experts % n_groups)
    return fail(MOE_ERR_SHAPE, "n_groups must be in [1, 16] and divide n_experts (%d)", cfg->n_experts);
  if (!x || !w_router || !topk_idx || !topk_prob || !stats || !ws)
    return fail(MOE_ERR_NULL, "x, w_router, topk_idx, topk_prob, stats and ws are required");
  if (misaligned(x) || misaligned(w_router) || misaligned(bias) || misaligned(k_per_token) || misaligned(topk_idx) ||
      misaligned(topk_prob) || misaligned(stats) || misaligned(ws))
    return fail(MOE_ERR_MISALIGNED, "moe_route_group_stats: a pointer is not 16-byte aligned");
  if (cfg->dtype == MOE_BF16 && cfg->d_model % 8)
    return fail(MOE_ERR_UNSUPPORTED, "bf16 rows need d_model % 8 == 0");
  const size_t need = moe_route_group_stats_workspace_bytes(cfg, T, n_groups);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_route_group_stats needs %zu workspace bytes, got %zu", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {  // no tokens: the statistics kernel writes zeros (it reads nothing)
    MOE_TRY_HIP(launch_group_stats(nullptr, nullptr, 0, cfg->top_k, cfg->n_experts, n_groups, nullptr, stats, s),
                "group statistics");
    return ok();
  }
  Arena a(ws);
  const RouteWs w = carve_route(a, cfg, T);
  float* gmass = a.take<float>(T * n_groups);
  double* part = a.take<double>(group_stats_partials(T, n_groups));
  MOE_TRY(run_route(cfg, T, x, w_router, bias, k_per_token, topk_idx, topk_prob, nullptr, w, s, gmass, n_groups));
  MOE_TRY_HIP(launch_group_stats(gmass, topk_idx, T, cfg->top_k, cfg->n_experts, n_groups, part, stats, s),
              "group statistics");
  return ok();
}

size_t moe_fp8_weights_bytes(int64_t n_mats, int64_t rows, int64_t cols) {
  if (n_mats < 0 || rows < 0 || cols <= 0 || cols % 64) return SIZE_MAX;
  return (size_t)n_mats * (size_t)((rows + 15) / 16 * 16) * (size_t)cols;
}

moe_status moe_quantize_fp8(int64_t n_mats, int64_t rows, int64_t cols, const void* src, void* dst,
                            size_t dst_bytes, float* scales, void* stream) {
  if (n_mats < 0 || rows < 0 || cols <= 0 || cols % 64 || cols > (1 << 20))
    return fail(MOE_ERR_SHAPE, "n_mats, rows >= 0 and cols in (0, 2^20], a multiple of 64, are required");
  if (n_mats == 0 || rows == 0) return ok();
  if (n_mats * ((rows + 15) / 16 * 16) >= kMaxRows) return fail(MOE_ERR_SHAPE, "too many rows");
  if (!src || !dst || !scales) return fail(MOE_ERR_NULL, "src, dst and scales are required");
  if (misaligned(src) || misaligned(dst) || misaligned(scales))
    return fail(MOE_ERR_MISALIGNED, "moe_quantize_fp8: a pointer is not 16-byte aligned");
  const size_t need = moe_fp8_weights_bytes(n_mats, rows, cols);
  if (dst_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_quantize_fp8 needs %zu dst bytes, got %zu", need, dst_bytes);
  MOE_TRY_HIP(launch_quant_fp8((const bf16_t*)src, n_mats, rows, cols, (uint8_t*)dst, scales, (hipStream_t)stream),
              "fp8 quantisation");
  return ok();
}

moe_status moe_ep_receive_plan(int32_t n_src, int32_t n_local, const int32_t* counts, int64_t max_rows,
                               int32_t* offsets, int32_t* gather, int32_t* scatter, void* stream) {
  if (n_src < 1 || n_local < 1 || (int64_t)n_src * n_local > 1024)
    return fail(MOE_ERR_SHAPE, "n_src and n_local must be >= 1 with n_src * n_local <= 1024");
  if (max_rows < 0 || max_rows >= kMaxRows) return fail(MOE_ERR_SHAPE, "max_rows must be in [0, 2^31)");
  if (!counts || !offsets || (max_rows > 0 && (!gather || !scatter)))
    return fail(MOE_ERR_NULL, "counts, offsets, gather and scatter are required");
  if (misaligned(counts) || misaligned(offsets) || misaligned(gather) || misaligned(scatter))
    return fail(MOE_ERR_MISALIGNED, "moe_ep_receive_plan: a pointer is not 16-byte aligned");
  MOE_TRY_HIP(launch_ep_plan(counts, n_src, n_local, max_rows, offsets, gather, scatter, (hipStream_t)stream),
              "receive plan");
  return ok();
}

moe_status moe_gather_rows(const void* src, int64_t n_src_rows, int64_t row_bytes, const int32_t* index,
                           int64_t n_rows, void* dst, void* stream) {
  if (n_rows < 0 || n_rows >= kMaxRows || row_bytes <= 0 || row_bytes > (1 << 30) || n_src_rows < 0)
    return fail(MOE_ERR_SHAPE, "n_rows in [0, 2^31), row_bytes in [1, 2^30] and n_src_rows >= 0 are required");
  if (n_rows == 0) return ok();
  if (n_src_rows == 0) return fail(MOE_ERR_SHAPE, "n_rows > 0 needs n_src_rows > 0");
  if (!src || !index || !dst) return fail(MOE_ERR_NULL, "src, index and dst are required");
  if (misaligned(src) || misaligned(index) || misaligned(dst))
    return fail(MOE_ERR_MISALIGNED, "moe_gather_rows: a pointer is not 16-byte aligned");
  MOE_TRY_HIP(launch_gather_rows(src, n_src_rows, (int)row_bytes, 1, index, n_rows, dst, (hipStream_t)stream),
              "row gather");
  return ok();
}

moe_status moe_layer_forward(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w, void* out,
                             int32_t* topk_idx_out, float* topk_prob_out, int32_t* offsets_out, void* ws,
                             size_t ws_bytes, void* stream) {
  return moe_layer_forward_dynamic(cfg, T, x, w, nullptr, out, topk_idx_out, topk_prob_out, offsets_out, ws, ws_bytes,
                                   stream);
}

moe_status moe_route(const moe_config* cfg, int64_t T, const void* x, const void* w_router, const float* bias,
                     int32_t* topk_idx, float* topk_prob, float* gap, void* ws, size_t ws_bytes, void* stream) {
  return moe_route_dynamic(cfg, T, x, w_router, bias, nullptr, topk_idx, topk_prob, gap, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- the layer without a caller workspace ----
//
// moe_layer_forward_noalloc runs moe_layer_forward with its workspace in the
// static device array below (one copy per GPU, held until the process ends).
// In host code `scratch` names a host-side stand-in, not device memory: the
// array's device address on each GPU comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is passed
// to kernels.
namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure, with the HIP error in *err).
void* scratch_on_current_device(hipError_t* err, int* dev_out) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  *dev_out = dev;
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_layer_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const moe_weights* w, void* out,
                                     int32_t* topk_idx_out, float* topk_prob_out, int32_t* offsets_out,
                                     void* stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(cfg, T));
  if (T == 0) return ok();
  MOE_TRY(check_layer_args(cfg, x, w, nullptr, out, topk_idx_out, topk_prob_out, offsets_out));
  const size_t need = moe_layer_workspace_bytes(cfg, T);
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_layer_forward_noalloc: this layer needs %zu workspace bytes for %lld tokens; the static "
                "scratch holds %zu (use moe_layer_forward with a caller workspace)",
                need, (long long)T, kScratchBytes);
  hipError_t e = hipSuccess;
  int dev = 0;
  void* ws = scratch_on_current_device(&e, &dev);
  if (!ws) return fail(MOE_ERR_HIP, "moe_layer_forward_noalloc: address of the static scratch on device %d: %s", dev,
                       hipGetErrorString(e));
  return moe_layer_forward_dynamic(cfg, T, x, w, nullptr, out, topk_idx_out, topk_prob_out, offsets_out, ws,
                                   kScratchBytes, stream);
}

}  // extern "C"
