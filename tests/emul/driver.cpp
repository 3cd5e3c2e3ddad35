// Bounds-checking driver for the 256x256 expert GEMM (grouped_gemm_big8.hip
// turned into host C++ by
// tests/test_gemm_big_bounds.py). It builds the launch arguments of one
// workload the way the library does (random top-k routing, the tile table,
// exact-size buffers for activations, weights, outputs and tables) and runs
// every lane of every block of both projections, packed and row-major (fp8
// weights: packed only), under
// AddressSanitizer.
//
// usage: driver T E K D F Fs seed [skew] [fp8]
#include <algorithm>
#include <mutex>
#include <random>
#include <thread>
#include <vector>
#include "emul_internal.h"
#include "runner.h"
template <class K, class A> void emul_launch(K kernel, unsigned blocks, unsigned threads, const A& args) {
  emul_run(false, kernel, dim3(blocks), threads, args);
}
#include "emul_big.cpp"

using namespace moe;
// The tile table as the library's tile builder writes it.
static std::vector<Tile> build_tiles(const std::vector<int32_t>& off, int64_t n_rows, int BM) {
  std::vector<Tile> t;
  for (size_t g = 0; g + 1 < off.size(); ++g) {
    int64_t a = std::clamp<int64_t>(off[g], 0, n_rows), b = std::clamp<int64_t>(off[g + 1], a, n_rows);
    const int first = (int)t.size(), count = (int)((b - a + BM - 1) / BM);
    for (int64_t r = a; r < b; r += BM)
      t.push_back(Tile{(int)g, (int)r, (int)std::min<int64_t>(r + BM, b), first, count, 0, 0, 0});
  }
  return t;
}
template <class T> T* buffer(size_t n) {  // exact size, so ASan sees any access past its end
  T* p = (T*)malloc(n ? n * sizeof(T) : 1);
  memset(p, 0, n * sizeof(T));
  return p;
}

int main(int argc, char** argv) {
  if (argc < 8) { fprintf(stderr, "usage: T E K D F Fs seed [skew]\n"); return 2; }
  const int T = atoi(argv[1]), E = atoi(argv[2]), K = atoi(argv[3]), D = atoi(argv[4]), F = atoi(argv[5]),
            Fs = atoi(argv[6]), seed = atoi(argv[7]);
  const bool skew = argc > 8 && atoi(argv[8]);
  const bool fp8 = argc > 9 && atoi(argv[9]);  // fp8 weights (codes + per-row scales) instead of bf16
  if (Fs && Fs != F) { fprintf(stderr, "a fused shared expert needs Fs == F\n"); return 2; }
  std::mt19937 rng(seed);
  std::vector<std::vector<int>> by_e(E);
  std::vector<int> ids(E);
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) ids[e] = e;
    for (int k = 0; k < K; ++k) {  // skew: three in four picks among the first dozen experts
      const int span = skew && rng() % 4 ? std::max(1, std::min(E - k, 12)) : E - k;
      std::swap(ids[k], ids[k + rng() % span]);
    }
    for (int k = 0; k < K; ++k) by_e[ids[k]].push_back(t);
  }
  const int64_t P = (int64_t)T * K, n_rows = P + (Fs ? T : 0);
  const int n_groups = E + (Fs ? 1 : 0);
  std::vector<int32_t> off(1, 0);
  int32_t* gather = buffer<int32_t>(P);
  int64_t pos = 0;
  for (int e = 0; e < E; ++e) {
    for (int t : by_e[e]) gather[pos++] = t;
    off.push_back((int32_t)pos);
  }
  if (Fs) off.push_back((int32_t)(P + T));
  const int BM = 256;
  const std::vector<Tile> tv = build_tiles(off, n_rows, BM);
  const int32_t max_tiles = (int32_t)(n_rows / BM + n_groups);
  Tile* tiles = buffer<Tile>(max_tiles);
  std::copy(tv.begin(), tv.end(), tiles);
  int32_t* n_tiles = buffer<int32_t>(1);
  *n_tiles = (int32_t)tv.size();
  printf("T=%d E=%d K=%d D=%d F=%d Fs=%d skew=%d: %zu tiles\n", T, E, K, D, F, Fs, (int)skew, tv.size());
  auto pad16 = [](int n) { return (n + 15) / 16 * 16; };
  for (int epi : {EPI_SWIGLU, EPI_F32})
    for (int pk = 1; pk >= (fp8 ? 1 : 0); --pk) {
      GemmArgs g{};
      g.tiles = tiles;
      g.n_tiles = n_tiles;
      g.dense_rows = n_rows;
      g.max_tiles = max_tiles;
      g.n_main = E;
      g.b_packed = pk;
      g.b_fp8 = fp8;
      bf16_t *a, *b0, *b1 = nullptr, *b0x = nullptr, *b1x = nullptr;
      float *s0 = nullptr, *s1 = nullptr, *s0x = nullptr, *s1x = nullptr;
      void* out;
      // weight buffers in bf16 elements: fp8 codes take half as many bytes
      auto wbuf = [&](size_t elems) { return fp8 ? (bf16_t*)buffer<uint8_t>(elems) : buffer<bf16_t>(elems); };
      if (epi == EPI_SWIGLU) {  // A: the token rows, gathered
        a = buffer<bf16_t>((size_t)T * D);
        g.n_a_rows = T;
        g.gather = gather;
        g.n_gather = P;
        const size_t wn = (size_t)(pk ? pad16(F) : F) * D;
        b0 = wbuf(wn * E);
        b1 = wbuf(wn * E);
        if (Fs) { b0x = wbuf(wn); b1x = wbuf(wn); }
        if (fp8) {
          s0 = buffer<float>((size_t)E * F);
          s1 = buffer<float>((size_t)E * F);
          if (Fs) { s0x = buffer<float>(F); s1x = buffer<float>(F); }
          g.s_stride = F;
        }
        g.b_stride = (int64_t)F * D;
        g.N = F;
        g.Kdim = D;
        out = buffer<bf16_t>((size_t)n_rows * F);
        g.ldo = F;
      } else {  // A: the SwiGLU rows in expert order
        a = buffer<bf16_t>((size_t)n_rows * F);
        g.n_a_rows = n_rows;
        const size_t wn = (size_t)(pk ? pad16(D) : D) * F;
        b0 = wbuf(wn * E);
        if (Fs) b0x = wbuf(wn);
        if (fp8) {
          s0 = buffer<float>((size_t)E * D);
          if (Fs) s0x = buffer<float>(D);
          g.s_stride = D;
        }
        g.b_stride = (int64_t)D * F;
        g.N = D;
        g.Kdim = F;
        out = buffer<float>((size_t)n_rows * D);
        g.ldo = D;
      }
      g.a = a;
      g.b0 = b0;
      g.b1 = b1;
      g.b0_extra = b0x;
      g.b1_extra = b1x;
      g.out = out;
      g.s0 = s0;
      g.s1 = s1;
      g.s0_extra = s0x;
      g.s1_extra = s1x;
      emul_loads = 0;
      const int rc = launch_grouped_gemm_big8(epi, g, nullptr);
      printf("  %s %s: rc=%d direct loads %lld ok\n", epi == EPI_SWIGLU ? "gate/up" : "down",
             fp8 ? "fp8" : (pk ? "packed" : "rows"), rc, emul_loads);
      fflush(stdout);
      if (rc != 0) return 3;
      free(a); free(b0); free(b1); free(b0x); free(b1x); free(out);
      free(s0); free(s1); free(s0x); free(s1x);
    }
  return 0;
}
