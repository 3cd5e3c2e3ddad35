// Expert GEMMs for many rows per expert, bf16 weights: 256 x 256 block
// tiles with eight waves, two per SIMD.
//
// Every expert is an independent FFN (page "Step3.5 Flash 大模型技术深度解析",
// section 3.2.1). The work item, the persistent walk over items, the two
// rings (gathered activation rows in 64-element stages, 128 bytes of a row;
// weights in 32-element steps) and the explicit waits are those of the
// four-wave kernel in grouped_gemm_big.hip. The difference is the wave
// layout: eight waves in a 2 x 4 arrangement, each wave 128 rows x 64 weight
// rows = 8 x 4 MFMA 16x16x32 tiles (128 fp32 accumulators), so two waves
// share each SIMD: while one waits at a barrier, for LDS reads or for its
// loads to be issued, the other keeps the matrix core busy, and two waves
// interleaving their MFMAs reach a higher issue rate than one (about 86% of
// peak against 72% back to back). The price is 50% more LDS operand reads
// per step (96 KB for the block against 64 KB); gfx950's LDS serves about
// 220 bytes per clock per CU, about twice what a step of multiplies needs.
//
// For gate/up the 256 weight rows of an item are 4 x [gate c0+32j ..
// c0+32j+31, up c0+32j .. c0+32j+31] (j = 0..3), so wave (wm, j) holds the
// gate and up sums of the same 32 output columns and applies the SwiGLU in
// registers.
//
// Loads per wave: an A stage is 4 direct loads (8 rows x 128 bytes each),
// a weight step 2 (one 16-row fragment or 16 rows x 64 bytes each).
#include "moe_internal.h"

// The operand-read lambdas capture their asm operands explicitly (clang's
// device pass does not capture names used only as asm operands); the host
// pass, which does not see the asm's use, would warn about those captures.
#pragma clang diagnostic ignored "-Wunused-lambda-capture"

namespace moe {

namespace {

constexpr int B8_NS = 4;      // weight ring steps
constexpr int B8_KS = 32;     // contraction elements per weight step (one MFMA step)
constexpr int B8_AKS = 64;    // contraction elements per A stage (two MFMA steps)
constexpr int B8_ROWS = 256;  // A rows and weight rows per item
constexpr int B8_CHUNK = 16;  // row tiles of one group that share weight columns in flight
constexpr int B8_CPOL_NT = 2; // weight loads: non-temporal

typedef __attribute__((address_space(3))) void lds8_void_t;
typedef uint32_t u32x4_8 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8_8(u32x4_8 v) { return __builtin_bit_cast(bf16x8, v); }
constexpr int waitcnt_vm8(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 3; }   // 64-byte weight rows
__device__ __forceinline__ int swzA8(int row) { return (row >> 1) & 7; }  // 128-byte A rows

template <int EPI, bool PK>
__global__ void __launch_bounds__(512) gemm_bf16_big8(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t ldsA[2][B8_ROWS * B8_AKS];
  __shared__ __attribute__((aligned(16))) bf16_t ldsB[B8_NS][B8_ROWS * B8_KS];
  __shared__ __attribute__((aligned(16))) float stg[8][1024];  // epilogue staging, 4 KB per wave

  const int BN = EPI == EPI_SWIGLU ? B8_ROWS / 2 : B8_ROWS;  // output columns per item
  const int n_nb = (p.N + BN - 1) / BN;
  const int n_tiles = p.tiles ? *p.n_tiles : (int)((p.dense_rows + B8_ROWS - 1) / B8_ROWS);
  const int active = n_tiles * n_nb;
  // block b runs on XCD b % 8; the items are split into 8 contiguous runs
  const int per_xcd = (active + 7) >> 3;
  const int L_begin = (blockIdx.x & 7) * per_xcd;
  const int L_end = L_begin + per_xcd < active ? L_begin + per_xcd : active;
  const int L_step = gridDim.x >> 3;
  int L = L_begin + (blockIdx.x >> 3);
  if (L >= L_end) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kdim = p.Kdim, nk = Kdim / B8_KS;
  const bf16_t* A = (const bf16_t*)p.a;

  // item -> (row tile, column block); multi-tile groups in chunks of row tiles
  auto map_item = [&](int L, Tile& t, int& nb) {
    int ti = L / n_nb;
    nb = L - ti * n_nb;
    if (p.tiles) {
      const Tile g = p.tiles[ti];
      const int first = g.first;
      int count = g.count;
      count = first + count <= n_tiles ? count : n_tiles - first;
      if (count > 1 && first >= 0 && first <= ti && ti < first + count) {
        const int local = L - first * n_nb;
        const int c = local / (B8_CHUNK * n_nb);
        const int wc = count - c * B8_CHUNK < B8_CHUNK ? count - c * B8_CHUNK : B8_CHUNK;
        const int local2 = local - c * B8_CHUNK * n_nb;
        nb = local2 / wc;
        ti = first + c * B8_CHUNK + local2 % wc;
      }
      t = p.tiles[ti];
    } else {
      t.group = 0;
      t.row0 = ti * B8_ROWS;
      t.row1 = (int32_t)((int64_t)t.row0 + B8_ROWS < p.dense_rows ? t.row0 + B8_ROWS : p.dense_rows);
    }
  };

  // A load instruction i (0..3) of this wave fills rows wave*32 + i*8 .. +7
  // of a stage: lane l writes row +l/8, physical chunk l%8 = logical chunk
  // (l%8) ^ swzA8(row). Rows outside the tile read row 0 (never stored).
  auto load_rows = [&](const Tile& t, int32_t(&rows)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = (int64_t)t.row0 + wave * 32 + i * 8 + (lane >> 3);
      int64_t src = -1;
      if (r < t.row1) {
        src = r < p.n_gather ? (int64_t)p.gather[r] : r - p.n_gather;
        if (src >= p.n_a_rows) src = -1;
      }
      rows[i] = (int32_t)(src >= 0 ? src : 0);
    }
  };
  uint32_t aoff[4];  // 16-byte-unit offsets from A (the launcher checks the 32-bit range)
  const bf16_t* bsrc[2];
  auto set_a_sources = [&](const int32_t(&rows)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wave * 32 + i * 8 + (lane >> 3);
      aoff[i] = (uint32_t)rows[i] * (uint32_t)(Kdim >> 3) + (uint32_t)((lane & 7) ^ swzA8(row));
    }
  };
  // weight load instruction i (0..1) of this wave fills weight rows
  // wave*32 + i*16 .. +15: the fragment of those rows (packed) or row
  // +l/4, chunk (l%4) ^ swz8(row) (row-major)
  auto set_b_sources = [&](const Tile& t, int nb) {
    const bf16_t* Bg = t.group < p.n_main ? (const bf16_t*)p.b0 + (int64_t)t.group * p.b_stride
                                          : (const bf16_t*)p.b0_extra;
    const bf16_t* Bu = EPI == EPI_SWIGLU ? (t.group < p.n_main ? (const bf16_t*)p.b1 + (int64_t)t.group * p.b_stride
                                                               : (const bf16_t*)p.b1_extra)
                                         : Bg;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wave * 32 + i * 16 + (lane >> 2);
      int col;
      const bf16_t* base;
      if constexpr (EPI == EPI_SWIGLU) {
        const int seg = row >> 5;  // gate, up, gate, up, ... in 32-row segments
        col = nb * BN + (seg >> 1) * 32 + (row & 31);
        base = (seg & 1) ? Bu : Bg;
      } else {
        col = nb * BN + row;
        base = Bg;
      }
      if constexpr (PK) {
        int ct = (col - (row & 15)) >> 4;
        const int ct_last = (p.N + 15) / 16 - 1;
        ct = ct < ct_last ? ct : ct_last;
        bsrc[i] = base + packed_offset(ct, 0, lane, Kdim);
      } else {
        col = col < p.N ? col : p.N - 1;
        bsrc[i] = base + (int64_t)col * Kdim + (((lane & 3) ^ swz8(row)) * 8);
      }
    }
  };
  auto issue_a = [&](int slot, int ja) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(A + (uint64_t)aoff[i] * 8u + ja * B8_AKS),
                                       (lds8_void_t*)&ldsA[slot][(wave * 32 + i * 8) * B8_AKS], 16, 0, 0);
  };
  auto issue_b = [&](int slot, int ks) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + (PK ? ks * PACKED_FRAG : ks * B8_KS)),
                                       (lds8_void_t*)&ldsB[slot][(wave * 32 + i * 16) * B8_KS], 16, 0, B8_CPOL_NT);
  };

  // wave (wm, wn): rows wm*128 .., weight rows wn*64 ..
  const int wm = wave >> 2, wn = wave & 3;
  f32x4 acc[8][4];

  // operand reads: lane (r = lane & 15, q = lane >> 4) of a 16-row tile; A
  // row tile m at +2048 m, weight row tile n at +1024 n (immediates)
  const int rq = lane >> 4, rr = lane & 15;
  const uint32_t aoffA0 = (uint32_t)((wm * 128 + rr) * B8_AKS + ((rq ^ swzA8(rr)) << 3)) * 2u;
  const uint32_t aoffA1 = (uint32_t)((wm * 128 + rr) * B8_AKS + (((rq + 4) ^ swzA8(rr)) << 3)) * 2u;
  const uint32_t boff0 = PK ? (uint32_t)(wn * 64 * B8_KS) * 2u + (uint32_t)lane * 16u
                            : (uint32_t)((wn * 64 + rr) * B8_KS + ((rq ^ swz8(rr)) << 3)) * 2u;
  const uint32_t ldsA_base = (uint32_t)(uintptr_t)(lds8_void_t*)&ldsA[0][0];
  const uint32_t ldsB_base = (uint32_t)(uintptr_t)(lds8_void_t*)&ldsB[0][0];
  constexpr uint32_t SLOT_A = B8_ROWS * B8_AKS * 2u, SLOT_B = B8_ROWS * B8_KS * 2u;
  auto read_b = [&](int slot, u32x4_8(&b)[4]) {
    const uint32_t addr = ldsB_base + (uint32_t)slot * SLOT_B + boff0;
    static_for<0, 4>([&b, addr](auto N) {
      constexpr int n = decltype(N)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(b[n]) : "v"(addr), "n"(n * 1024));
    });
  };
  auto read_a = [&](int slot, int sub, u32x4_8(&a)[8]) {
    const uint32_t addr = ldsA_base + (uint32_t)slot * SLOT_A + (sub ? aoffA1 : aoffA0);
    static_for<0, 8>([&a, addr](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[m]) : "v"(addr), "n"(m * 2048));
    });
  };
  // A chunk m lands at lgkmcnt(11 - m): the 8 A reads are followed by the 4
  // weight reads of the next step
  auto multiply = [&](u32x4_8(&a)[8], const u32x4_8(&b)[4]) {
    static_for<0, 8>([&](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a[m]) : "n"(11 - m));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_8(a[m]), as_bf16x8_8(b[n]), acc[m][n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Epilogue through this wave's 4 KB staging area, one 16-row tile at a
  // time (accumulator layout: lane holds column lane & 15 of each 16-column
  // tile, rows 4*(lane >> 4) + v); whole rows are stored 16 bytes per lane.
  auto epilogue = [&](const Tile& t, int nb) {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int LDW = 40;  // 16 rows x 32 bf16 columns, rows padded to 40
      bf16_t* wbuf = (bf16_t*)&stg[wave][0];
      const int col0 = nb * BN + wn * 32;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            wbuf[(4 * (lane >> 4) + v) * LDW + n * 16 + (lane & 15)] = f32_to_bf16(silu(acc[m][n][v]) * acc[m][n + 2][v]);
        // 4 lanes per row (8 bf16 each), 16 rows: one pass
        const int rr16 = lane >> 2, c8 = (lane & 3) * 8;
        const uint4 v = *(const uint4*)&wbuf[rr16 * LDW + c8];
        const int64_t r = (int64_t)t.row0 + wm * 128 + m * 16 + rr16;
        const int col = col0 + c8;
        if (r < t.row1 && col < p.N) *(uint4*)&((bf16_t*)p.out)[r * p.ldo + col] = v;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // 16 rows x 64 fp32 columns; 16-column groups XOR-swizzled by (row >> 2) & 3
      float* wbuf = &stg[wave][0];
      const int col0 = nb * BN + wn * 64;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 4 * (lane >> 4) + v;
            wbuf[row * 64 + ((n ^ ((row >> 2) & 3)) << 4) + (lane & 15)] = acc[m][n][v];
          }
        // 16 lanes per row (4 floats each), 4 rows per pass, 4 passes
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
          const int rr16 = pass * 4 + (lane >> 4), c4 = (lane & 15) * 4;
          float4 v = *(const float4*)&wbuf[rr16 * 64 + (c4 ^ (((rr16 >> 2) & 3) << 4))];
          const int64_t r = (int64_t)t.row0 + wm * 128 + m * 16 + rr16;
          const int col = col0 + c4;
          if (r < t.row1 && col < p.N) {
            if (p.bias) {
              v.x += p.bias[col];
              v.y += p.bias[col + 1];
              v.z += p.bias[col + 2];
              v.w += p.bias[col + 3];
            }
            *(float4*)&((float*)p.out)[r * p.ldo + col] = v;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Rings and steps as in the four-wave kernel, with this wave's loads:
  // even step k issues A(k/2+1) (4 loads) and weight step k+3 (2); odd step
  // k weight step k+3 (2). At even k the loads younger than those waited for
  // are weight step k+2 (2); at odd k, A(k/2+1) and weight step k+2 (6).
  const int nh = nk >> 1;
  Tile t_cur, t_next;
  int nb_cur, nb_next;
  int32_t rows[4];
  map_item(L, t_cur, nb_cur);
  load_rows(t_cur, rows);
  set_a_sources(rows);
  set_b_sources(t_cur, nb_cur);
  int L_next = L + L_step;
  bool has_next = L_next < L_end;
  if (has_next) {
    map_item(L_next, t_next, nb_next);
    load_rows(t_next, rows);
  }
  int baseA = 0, baseB = 0;
  const int lastA = nh - 1, lastB = nk - 1;
  u32x4_8 a[8], b0[4], b1[4];
  issue_a(0, 0);
#pragma unroll
  for (int s = 0; s < B8_NS - 1; ++s) issue_b(s, s);  // nk >= 4
  __builtin_amdgcn_s_waitcnt(waitcnt_vm8(4));          // A stage 0, weight step 0
  asm volatile("s_barrier" ::: "memory");
  read_b(0, b0);
  auto step = [&](int k, auto ODD, const u32x4_8(&b_cur)[4], u32x4_8(&b_next)[4]) {
    constexpr bool odd = decltype(ODD)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm8(odd ? 6 : 2));
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const int h = k >> 1;
    if constexpr (!odd) {
      const int ha = h + 1;
      if (ha == nh && has_next) set_a_sources(rows);
      issue_a((baseA + ha) & 1, ha < nh ? ha : (has_next ? ha - nh : lastA));
    }
    const int ks = k + B8_NS - 1;
    if (ks == nk && has_next) set_b_sources(t_next, nb_next);
    issue_b((baseB + ks) % B8_NS, ks < nk ? ks : (has_next ? ks - nk : lastB));
    read_a((baseA + h) & 1, odd ? 1 : 0, a);
    read_b((baseB + k + 1) % B8_NS, b_next);
    multiply(a, b_cur);
  };
  for (;;) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int k = 0; k < nk; k += 2) {
      step(k, std::false_type{}, b0, b1);
      step(k + 1, std::true_type{}, b1, b0);
    }
    epilogue(t_cur, nb_cur);
    if (!has_next) break;
    baseA = (baseA + nh) & 1;
    baseB = (baseB + nk) % B8_NS;
    t_cur = t_next;
    nb_cur = nb_next;
    L_next += L_step;
    has_next = L_next < L_end;
    if (has_next) {
      map_item(L_next, t_next, nb_next);
      load_rows(t_next, rows);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm8(0));
}

int g_cus8 = 0;  // compute units of the device (queried once)

}  // namespace

hipError_t launch_grouped_gemm_big8(int epi, const GemmArgs& g, hipStream_t s) {
  if (g.max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.b_fp8) return hipErrorInvalidValue;  // fp8 weights take the four-wave kernel
  if (g.Kdim % B8_AKS || g.Kdim < 2 * B8_AKS) return hipErrorInvalidValue;
  if ((uint64_t)g.n_a_rows * (uint64_t)g.Kdim / 8u > 0xffffffffull) return hipErrorInvalidValue;
  if (g.N % 8 || g.ldo % 8) return hipErrorInvalidValue;
  if (g_cus8 == 0) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus8 = cus > 8 ? cus : 8;
  }
  const int BN = epi == EPI_SWIGLU ? B8_ROWS / 2 : B8_ROWS;
  const int n_nb = (g.N + BN - 1) / BN;
  int64_t blocks = ((int64_t)g.max_tiles * n_nb + 7) / 8 * 8;
  const int64_t cap = (int64_t)g_cus8 / 8 * 8;
  blocks = blocks < cap ? blocks : cap;
  if (g.b_packed) {
    if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, true><<<(unsigned)blocks, 512, 0, s>>>(g);
    else gemm_bf16_big8<EPI_F32, true><<<(unsigned)blocks, 512, 0, s>>>(g);
  } else {
    if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, false><<<(unsigned)blocks, 512, 0, s>>>(g);
    else gemm_bf16_big8<EPI_F32, false><<<(unsigned)blocks, 512, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
