// Bounds check of the library's own host path (tests/test_host_path_bounds.py).
//
// The C ABI (csrc/api.hip) is compiled for the host unchanged apart from its
// include, together with the kernels it launches on this path (permutation,
// tile builder, both expert-GEMM families), each turned into host C++; a launch
// runs every lane of every block (tests/emul/runner.h). The caller's buffers
// are exact-size host allocations, so AddressSanitizer reports any access
// outside one of them, from the host code or from any lane.
//
// Scenario (the argument pattern of the standalone expert halves at the
// layer's sizes): random top-K routing -> moe_permute (indices and the row
// gather) -> moe_expert_gate_up with the E routed groups plus one extra group
// (the shared expert: offsets of E+2 entries, gather of T*K rows, n_rows =
// T*K + T) -> moe_expert_down on the same offsets -> moe_grouped_ffn over the
// routed rows and over the shared expert's T rows alone. Every call must
// return MOE_OK.
//
// The permutation kernels synchronise through LDS barriers and wave
// shuffles, which the emulation runs with one OS thread per lane: too slow at
// the layer's full token counts, so with `host_perm` = 1 the offsets and the
// row map are made here on the host (a stable counting sort) and moe_permute
// is not called; the expert launches then see exactly the arguments the
// permutation gives them.
//
// Scenario "layer": the whole layer through moe_layer_forward,
// moe_layer_forward_dynamic (per-token expert counts) and
// moe_layer_forward_noalloc, on the caller's x and weights (row-major,
// packed, or fp8 codes written by moe_quantize_fp8 and bf16 weights packed by
// moe_pack_weights), every kernel on the way emulated: router GEMM, top-k
// (its DPP reductions through emulated lane moves), permutation (the
// single-block form that also writes the tile table, or the rank/place form),
// expert GEMMs, combine. The bf16 matrix-core results are not computed (the
// logits come out zero, so every token picks experts 0..K-1 and a router bias
// spreads them); with fp32 layers the generic GEMM computes real values and
// the routing is the real one.
//
// usage: host_path halves T E K D F seed skew packed [host_perm]
//        host_path layer T E K D F seed layout(0 rows, 1 packed, 2 fp8) fp32
#include <algorithm>
#include <random>
#include <vector>

#include "emul_internal.h"
#include "runner.h"

template <class K, class A> void emul_launch(K kernel, unsigned blocks, unsigned threads, const A& args) {
  emul_run(false, kernel, dim3(blocks), threads, args);
}

#include "emul_api.cpp"
#include "emul_big.cpp"
#include "emul_combine.cpp"
#include "emul_gemm.cpp"
#include "emul_pack.cpp"
#include "emul_permute.cpp"
#include "emul_route.cpp"
#include "emul_router.cpp"

template <class T> T* buffer(size_t n) {  // exact size: ASan sees any access past its end
  T* p = (T*)malloc(n ? n * sizeof(T) : 1);
  if (!p) { fprintf(stderr, "out of host memory (%zu elements)\n", n); exit(4); }
  memset(p, 0, n * sizeof(T));
  return p;
}

static int check(moe_status s, const char* what) {
  printf("  %-44s %s\n", what, s == MOE_OK ? "ok" : moe_last_error());
  fflush(stdout);
  return s == MOE_OK ? 0 : 1;
}

static int run_layer(int argc, char** argv);

static int run_halves(int argc, char** argv) {
  if (argc < 9) { fprintf(stderr, "usage: halves T E K D F seed skew packed [host_perm]\n"); return 2; }
  const int T = atoi(argv[1]), E = atoi(argv[2]), K = atoi(argv[3]), D = atoi(argv[4]), F = atoi(argv[5]),
            seed = atoi(argv[6]);
  const bool skew = atoi(argv[7]) != 0, packed = atoi(argv[8]) != 0;
  const bool host_perm = argc > 9 && atoi(argv[9]) != 0;
  moe_config cfg{D, E, K, F, F, MOE_BF16, MOE_BF16, packed ? MOE_LAYOUT_PACKED : MOE_LAYOUT_ROWS};
  const int64_t P = (int64_t)T * K, n_rows = P + T;
  printf("T=%d E=%d K=%d D=%d F=%d skew=%d %s\n", T, E, K, D, F, (int)skew, packed ? "packed" : "rows");

  // routing: K distinct experts per token (skew: three in four picks among the first dozen)
  std::mt19937 rng(seed);
  int32_t* idx = buffer<int32_t>(P);
  std::vector<int> ids(E);
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) ids[e] = e;
    for (int k = 0; k < K; ++k) {
      const int span = skew && rng() % 4 ? std::max(1, std::min(E - k, 12)) : E - k;
      std::swap(ids[k], ids[k + rng() % span]);
      idx[(int64_t)t * K + k] = ids[k];
    }
  }
  int fails = 0;
  bf16_t* x = buffer<bf16_t>((size_t)T * D);
  // permutation, with and without the row gather
  int32_t* offsets = buffer<int32_t>(E + 1);
  int32_t* sorted_token = buffer<int32_t>(P);
  int32_t* dest = buffer<int32_t>(P);
  size_t wsb = 0;
  char* ws = nullptr;
  if (host_perm) {  // stable counting sort of the pairs by expert
    std::vector<int64_t> cnt(E + 1, 0);
    for (int64_t j = 0; j < P; ++j) cnt[idx[j] + 1]++;
    for (int e = 0; e < E; ++e) cnt[e + 1] += cnt[e];
    for (int e = 0; e <= E; ++e) offsets[e] = (int32_t)cnt[e];
    for (int64_t j = 0; j < P; ++j) {
      const int64_t d = cnt[idx[j]]++;
      dest[j] = (int32_t)d;
      sorted_token[d] = (int32_t)(j / K);
    }
    printf("  %-44s %s\n", "permutation (host)", "done");
  } else {
    wsb = moe_permute_workspace_bytes(&cfg, T);
    ws = buffer<char>(wsb);
    fails += check(moe_permute(&cfg, T, idx, offsets, sorted_token, dest, nullptr, nullptr, ws, wsb, nullptr),
                   "moe_permute");
    bf16_t* x_perm = buffer<bf16_t>((size_t)P * D);
    fails += check(moe_permute(&cfg, T, idx, offsets, sorted_token, dest, x, x_perm, ws, wsb, nullptr),
                   "moe_permute with the row gather");
    free(x_perm);
    free(ws);
  }
  // the permutation itself: offsets scan the counts, rows of a segment in token order, dest inverse
  {
    std::vector<int64_t> cnt(E, 0);
    for (int64_t j = 0; j < P; ++j) cnt[idx[j]]++;
    int64_t run = 0;
    for (int e = 0; e < E; ++e) {
      if (offsets[e] != run) { printf("  offsets[%d] = %d, expected %lld\n", e, offsets[e], (long long)run); ++fails; break; }
      run += cnt[e];
    }
    for (int64_t j = 0; j < P && fails == 0; ++j)
      if (sorted_token[dest[j]] != j / K) { printf("  dest/sorted_token mismatch at pair %lld\n", (long long)j); ++fails; }
  }
  // the layer's expert launch arguments: E routed groups, then the shared expert's T rows
  int32_t* offs_ext = buffer<int32_t>(E + 2);
  memcpy(offs_ext, offsets, (E + 1) * sizeof(int32_t));
  offs_ext[E + 1] = (int32_t)n_rows;
  auto wsize = [&](int64_t mats, int64_t rows, int64_t cols) {
    return packed ? moe_packed_weights_bytes(mats, rows, cols) / 2 : (size_t)(mats * rows * cols);
  };
  bf16_t* w_gate = buffer<bf16_t>(wsize(E, F, D));
  bf16_t* w_up = buffer<bf16_t>(wsize(E, F, D));
  bf16_t* s_gate = buffer<bf16_t>(wsize(1, F, D));
  bf16_t* s_up = buffer<bf16_t>(wsize(1, F, D));
  bf16_t* h = buffer<bf16_t>((size_t)n_rows * F);
  wsb = moe_expert_workspace_bytes(&cfg, E + 1, n_rows, F);
  ws = buffer<char>(wsb);
  fails += check(moe_expert_gate_up(&cfg, E, n_rows, offs_ext, x, T, sorted_token, P, w_gate, w_up, s_gate, s_up, F,
                                    h, ws, wsb, nullptr),
                 "moe_expert_gate_up (routed + shared group)");
  {  // the tile table the emulated tile builder left at the start of the workspace
    const int BM = moe::gemm_block_rows(true, n_rows, E + 1, true);
    const int32_t max_tiles = (int32_t)moe::gemm_max_tiles(n_rows, E + 1, BM);
    const moe::Tile* tiles = (const moe::Tile*)ws;
    const int32_t n = *(const int32_t*)(ws + ((size_t)max_tiles * sizeof(moe::Tile) + 255) / 256 * 256);
    int32_t want = 0;
    for (int g = 0; g <= E; ++g) {
      const int first = want, count = (offs_ext[g + 1] - offs_ext[g] + BM - 1) / BM;
      for (int r = offs_ext[g]; r < offs_ext[g + 1]; r += BM, ++want) {
        const moe::Tile& t = tiles[want];
        if (want >= n || t.group != g || t.row0 != r || t.row1 != std::min(r + BM, offs_ext[g + 1]) ||
            t.first != first || t.count != count) {
          printf("  tile %d differs from the segmentation of the offsets\n", want);
          ++fails;
          g = E + 1;
          break;
        }
      }
    }
    printf("  tile table: %d tiles of %d rows, %lld direct loads into LDS\n", n, BM, emul_loads);
    if (n != want) ++fails;
  }
  free(w_gate);
  free(w_up);
  bf16_t* w_down = buffer<bf16_t>(wsize(E, D, F));
  bf16_t* s_down = buffer<bf16_t>(wsize(1, D, F));
  float* y = buffer<float>((size_t)n_rows * D);
  fails += check(moe_expert_down(&cfg, E, n_rows, offs_ext, h, w_down, s_down, F, y, ws, wsb, nullptr),
                 "moe_expert_down (routed + shared group)");
  free(ws);
  free(h);
  free(y);
  // the grouped FFN: routed rows through the gather, then the shared expert alone
  w_gate = buffer<bf16_t>(wsize(E, F, D));
  w_up = buffer<bf16_t>(wsize(E, F, D));
  float* yr = buffer<float>((size_t)P * D);
  wsb = moe_grouped_ffn_workspace_bytes(&cfg, E, P, F);
  ws = buffer<char>(wsb);
  fails += check(moe_grouped_ffn(&cfg, E, P, offsets, x, T, sorted_token, w_gate, w_up, w_down, F, yr, ws, wsb,
                                 nullptr),
                 "moe_grouped_ffn (routed rows, gathered)");
  free(ws);
  free(yr);
  int32_t* one = buffer<int32_t>(2);
  one[1] = T;
  float* ys = buffer<float>((size_t)T * D);
  wsb = moe_grouped_ffn_workspace_bytes(&cfg, 1, T, F);
  ws = buffer<char>(wsb);
  fails += check(moe_grouped_ffn(&cfg, 1, T, one, x, T, nullptr, s_gate, s_up, s_down, F, ys, ws, wsb, nullptr),
                 "moe_grouped_ffn (shared expert alone)");
  free(ws);
  printf("%s\n", fails ? "FAILED" : "all calls ok");
  return fails ? 1 : 0;
}

static int run_layer(int argc, char** argv) {
  if (argc < 9) { fprintf(stderr, "usage: layer T E K D F seed layout fp32\n"); return 2; }
  const int T = atoi(argv[1]), E = atoi(argv[2]), K = atoi(argv[3]), D = atoi(argv[4]), F = atoi(argv[5]),
            seed = atoi(argv[6]), layout = atoi(argv[7]);
  const bool f32 = atoi(argv[8]) != 0;
  const int dt = f32 ? MOE_F32 : MOE_BF16;
  moe_config cfg{D, E, K, F, F, dt, dt, layout};
  printf("layer T=%d E=%d K=%d D=%d F=%d layout=%d %s\n", T, E, K, D, F, layout, f32 ? "fp32" : "bf16");
  std::mt19937 rng(seed);
  const size_t es = f32 ? 4 : 2;
  auto rnd = [&](size_t n, float scale) {  // bf16 or fp32 values of a seeded draw
    char* p = buffer<char>(n * es);
    std::normal_distribution<float> nd(0.f, scale);
    for (size_t i = 0; i < n; ++i) {
      const float v = nd(rng);
      if (f32) ((float*)p)[i] = v;
      else { uint32_t u; memcpy(&u, &v, 4); ((uint16_t*)p)[i] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16); }
    }
    return (void*)p;
  };
  int fails = 0;
  // weights: row-major draws; the packed and fp8 layouts are made by the library's own converters
  void* wr = rnd((size_t)E * D, 0.02f);
  void* wg = rnd((size_t)E * F * D, 0.03f);
  void* wu = rnd((size_t)E * F * D, 0.03f);
  void* wd = rnd((size_t)E * D * F, 0.03f);
  void* sg = rnd((size_t)F * D, 0.03f);
  void* su = rnd((size_t)F * D, 0.03f);
  void* sd = rnd((size_t)D * F, 0.03f);
  float* bias = buffer<float>(E);
  for (int e = 0; e < E; ++e) bias[e] = (float)(rng() % 1000) * 1e-3f;  // spreads the zero logits of bf16 runs
  moe_weights w{};
  float* scales[6] = {};
  void* conv[7] = {};
  if (layout == MOE_LAYOUT_ROWS) {
    w = moe_weights{wr, bias, wg, wu, wd, sg, su, sd};
  } else {
    auto pack = [&](void* src, int64_t n, int64_t r, int64_t c, int slot) {
      const size_t nb = moe_packed_weights_bytes(n, r, c);
      conv[slot] = buffer<char>(nb);
      fails += check(moe_pack_weights(n, r, c, src, conv[slot], nb, nullptr), "moe_pack_weights");
      return conv[slot];
    };
    auto quant = [&](void* src, int64_t n, int64_t r, int64_t c, int slot) {
      const size_t nb = moe_fp8_weights_bytes(n, r, c);
      conv[slot] = buffer<char>(nb);
      scales[slot - 1] = buffer<float>((size_t)n * r);
      fails += check(moe_quantize_fp8(n, r, c, src, conv[slot], nb, scales[slot - 1], nullptr), "moe_quantize_fp8");
      return conv[slot];
    };
    auto cv = [&](void* src, int64_t n, int64_t r, int64_t c, int slot) {
      return layout == MOE_LAYOUT_FP8 ? quant(src, n, r, c, slot) : pack(src, n, r, c, slot);
    };
    w.w_router = pack(wr, 1, E, D, 0);
    w.router_bias = bias;
    w.w_gate = cv(wg, E, F, D, 1);
    w.w_up = cv(wu, E, F, D, 2);
    w.w_down = cv(wd, E, D, F, 3);
    w.s_gate = cv(sg, 1, F, D, 4);
    w.s_up = cv(su, 1, F, D, 5);
    w.s_down = cv(sd, 1, D, F, 6);
    if (layout == MOE_LAYOUT_FP8) {
      w.w_gate_scale = scales[0], w.w_up_scale = scales[1], w.w_down_scale = scales[2];
      w.s_gate_scale = scales[3], w.s_up_scale = scales[4], w.s_down_scale = scales[5];
    }
  }
  void* x = rnd((size_t)T * D, 1.0f);
  char* out = buffer<char>((size_t)T * D * es);
  int32_t* idx = buffer<int32_t>((size_t)T * K);
  float* prob = buffer<float>((size_t)T * K);
  int32_t* offs = buffer<int32_t>(E + 1);
  const size_t wsb = moe_layer_workspace_bytes(&cfg, T);
  char* ws = buffer<char>(wsb);
  fails += check(moe_layer_forward(&cfg, T, x, &w, out, idx, prob, offs, ws, wsb, nullptr), "moe_layer_forward");
  // the routing must be a valid top-K set per token and the segments must count the pairs
  for (int64_t t = 0; t < T && !fails; ++t)
    for (int k = 0; k < K; ++k)
      if (idx[t * K + k] < 0 || idx[t * K + k] >= E) { printf("  token %lld: expert id %d\n", (long long)t, idx[t * K + k]); ++fails; break; }
  if (offs[E] != T * K) { printf("  offsets[E] = %d, expected %d\n", offs[E], T * K); ++fails; }
  int32_t* kt = buffer<int32_t>(T);
  for (int t = 0; t < T; ++t) kt[t] = (int32_t)(rng() % (K + 2)) - 1;  // includes -1 and K+1 (clamped)
  fails += check(moe_layer_forward_dynamic(&cfg, T, x, &w, kt, out, idx, prob, offs, ws, wsb, nullptr),
                 "moe_layer_forward_dynamic");
  if (wsb <= moe_noalloc_scratch_bytes())
    fails += check(moe_layer_forward_noalloc(&cfg, T, x, &w, out, idx, prob, offs, nullptr),
                   "moe_layer_forward_noalloc");
  // balance statistics over G groups: the chosen pairs of all groups add up to T*K
  const int G = E % 8 == 0 ? 8 : (E % 4 == 0 ? 4 : 1);
  const size_t gsb = moe_route_group_stats_workspace_bytes(&cfg, T, G);
  char* gws = buffer<char>(gsb);
  double* stats = buffer<double>(2 * G);
  fails += check(moe_route_group_stats(&cfg, T, x, w.w_router, bias, nullptr, G, idx, prob, stats, gws, gsb,
                                       nullptr), "moe_route_group_stats");
  double pairs = 0.0;
  for (int g = 0; g < G; ++g) pairs += stats[G + g];
  if (pairs != (double)T * K) { printf("  group pair counts add up to %.0f, expected %d\n", pairs, T * K); ++fails; }
  printf("  experts of token 0:");
  for (int k = 0; k < K; ++k) printf(" %d", idx[k]);
  printf("\n%s\n", fails ? "FAILED" : "all calls ok");
  return fails ? 1 : 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && !strcmp(argv[1], "layer")) return run_layer(argc - 1, argv + 1);
  if (argc >= 2 && !strcmp(argv[1], "halves")) return run_halves(argc - 1, argv + 1);
  fprintf(stderr, "usage: host_path halves|layer ...\n");
  return 2;
}
