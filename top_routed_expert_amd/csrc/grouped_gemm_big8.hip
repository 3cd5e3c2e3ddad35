// Expert GEMMs for many rows per expert (prefill): 256 x 256 block tiles,
// eight waves, bf16 or fp8 weights.
//
// Every expert is an independent FFN (page "Step3.5 Flash 大模型技术深度解析",
// section 3.2.1). With a few hundred rows per expert, the weights of one
// column block should leave HBM once and be multiplied by all of the
// expert's rows; a 256-row tile covers a whole expert in most cases.
//
// Work item: one (row tile, column block) pair, 256 rows x 256 weight rows.
// Block: eight waves in a 2 x 4 layout, each wave 128 rows x 64 weight rows
// = 8 x 4 MFMA 16x16x32 tiles (128 fp32 accumulators per lane), so two waves
// share each SIMD: while one waits at a barrier, for LDS reads or for its
// loads to be issued, the other keeps the matrix core busy, and two waves
// interleaving their MFMAs issue faster than one back to back. For gate/up
// the 256 weight rows of an item are 4 x [gate c0+32j .. c0+32j+31, up
// c0+32j .. c0+32j+31] (j = 0..3), so wave (wm, j) holds the gate and up
// sums of the same 32 output columns and applies the SwiGLU in registers.
//
// Persistent blocks: one block per CU walks its share of the items (split
// evenly over the 8 XCDs, column blocks fastest; the row tiles of a group
// with several run in chunks, row tile fastest, so blocks running together
// read the same weight columns). The load stream runs on across items: the
// last stages of an item issue the first stages of the next one, so items
// meet with no pipeline drain and an item's epilogue (results through LDS
// to HBM) runs while the next item's operands are already in flight.
//
// Both operands go HBM/L2 -> LDS through direct loads (global_load_lds, 16
// bytes per lane, no VGPR staging). The weights stream from HBM through a
// ring of 4 slots of 16 KB (bf16: one 32-element MFMA step per slot),
// non-temporal since each weight byte is used by one block. The gathered
// activation rows come mostly from L2 and move in stages of two MFMA steps,
// 128 bytes of each row (32 KB per stage, two slots): a 64-byte piece of a
// row uses half of a 128-byte cache line, and fetching whole lines raises
// the per-CU fetch rate of the gathered rows by about 40%. With a 32 KB
// epilogue staging area that fills the 160 KB of LDS. The weight operand of
// a step is read from LDS into registers one step ahead (two register sets)
// and the activation operand row tile by row tile in the step itself. Waits
// are explicit: a wave waits for its own loads with s_waitcnt vmcnt (loads
// complete in issue order), then one s_barrier per step makes every wave's
// loads visible and ends every wave's reads of the slots about to be
// refilled. The barrier is inline asm with a memory clobber, so the
// compiler moves no memory access across it and adds no drain of its own.
//
// Activation rows in LDS are 128 bytes (eight 16-byte chunks); chunk q of
// row r is stored at q ^ ((r >> 1) & 7), so the 16-byte operand reads of 16
// consecutive rows cover all banks once. Weight rows without packing are 64
// bytes with chunk q at q ^ ((r >> 1) & 3); with packed weights each 16-row
// group is one 1 KB fragment copied as it is (lane order).
//
// Loads per wave: an activation stage is 4 direct loads (8 rows x 128 bytes
// each), a weight step 2 (one 16-row fragment or 16 rows x 64 bytes each).
//
// FP8 weights (F8, packed): a weight stage holds 64 contraction elements of
// E4M3 codes (one 1 KB fragment per 16 weight rows, the same 16 KB slot), so
// both operands move in 64-element stages and a trip of two MFMA steps
// needs one wait and one barrier. Each wave reads its 4 fragments once per
// trip, converts the first halves of the codes to bf16 operands for the
// first step and the second halves for the second (the conversion is exact),
// and the epilogue multiplies by the per-column scales. The other wave of
// the SIMD multiplies while one waits for its codes or converts them.
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

template <int EPI, bool PK, bool F8, bool SKIP>
__global__ void __launch_bounds__(512) gemm_bf16_big8(GemmArgs p) {
  static_assert(!F8 || PK, "fp8 weights are packed");
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
  // (fp8: byte pointers into the codes, kept in the same bf16_t* slots)
  constexpr int64_t EB = F8 ? 1 : 2;  // bytes per weight element
  auto set_b_sources = [&](const Tile& t, int nb) {
    const bf16_t* Bg = (const bf16_t*)(t.group < p.n_main ? (const char*)p.b0 + (int64_t)t.group * p.b_stride * EB
                                                          : (const char*)p.b0_extra);
    const bf16_t* Bu =
        EPI == EPI_SWIGLU
            ? (const bf16_t*)(t.group < p.n_main ? (const char*)p.b1 + (int64_t)t.group * p.b_stride * EB
                                                 : (const char*)p.b1_extra)
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
      if constexpr (F8) {
        int ct = (col - (row & 15)) >> 4;
        const int ct_last = (p.N + 15) / 16 - 1;
        ct = ct < ct_last ? ct : ct_last;
        bsrc[i] = (const bf16_t*)((const char*)base + fp8_offset(ct, 0, lane, Kdim));
      } else if constexpr (PK) {
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
  auto issue_b = [&](int slot, int ks) {  // ks: a 32-element step (bf16) or a 64-element stage (fp8)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(
          F8 ? (const void*)((const char*)bsrc[i] + (int64_t)ks * FP8_FRAG)
             : (const void*)(bsrc[i] + (PK ? ks * PACKED_FRAG : ks * B8_KS)),
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
  // Even steps: right after row tile m's multiplies, a[m] is refilled with
  // row tile m's chunk of the following odd step (the second half of the
  // same activation stage, visible since this step's barrier), so odd steps
  // multiply at once. Chunk m of this step has landed once at most 11
  // younger reads are pending: the later chunks, the 4 weight reads and the
  // m refills issued so far add up to 11 for every m.
  // (The refill is an inline-asm read like the others: a plain LDS load would
  // make the compiler drain the direct loads in flight, which it cannot prove
  // do not alias it.)
  auto multiply_refill = [&](u32x4_8(&a)[8], const u32x4_8(&b)[4], int slot) {
    const uint32_t next = ldsA_base + (uint32_t)slot * SLOT_A + aoffA1;
    static_for<0, 8>([&a, &b, next, this_acc = &acc](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a[m]) : "n"(11));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        (*this_acc)[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_8(a[m]), as_bf16x8_8(b[n]), (*this_acc)[m][n], 0, 0, 0);
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[m]) : "v"(next), "n"(m * 2048));
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // odd steps: the activation operand is in registers (refilled in the even step)
  auto multiply_ready = [&](const u32x4_8(&a)[8], const u32x4_8(&b)[4]) {
    static_for<0, 8>([&](auto M) {
      constexpr int m = decltype(M)::value;
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_8(a[m]), as_bf16x8_8(b[n]), acc[m][n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // fp8: this wave's 4 weight fragments of a stage, 16 bytes per lane (both
  // MFMA steps' codes); raw[n] lands at lgkmcnt(11 - n) when the 8 A reads
  // follow them.
  auto read_b8 = [&](int slot, u32x4_8(&raw)[4]) {
    const uint32_t addr = ldsB_base + (uint32_t)slot * SLOT_B + (uint32_t)(wn * 4) * 1024u + (uint32_t)lane * 16u;
    static_for<0, 4>([&raw, addr](auto N) {
      constexpr int n = decltype(N)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(raw[n]) : "v"(addr), "n"(n * 1024));
    });
  };
  // operands of MFMA step `hi` (0, 1) of a stage from the raw codes
  auto convert_b = [&](const u32x4_8(&raw)[4], int hi, u32x4_8(&b)[4]) {
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint4 v = hi ? fp8x8_bf16x8(raw[n].z, raw[n].w) : fp8x8_bf16x8(raw[n].x, raw[n].y);
      b[n] = u32x4_8{v.x, v.y, v.z, v.w};
    }
  };
  // multiply with the A chunks as the only LDS reads in flight behind them
  auto multiply_a_only = [&](u32x4_8(&a)[8], const u32x4_8(&b)[4]) {
    static_for<0, 8>([&](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a[m]) : "n"(7 - m));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_8(a[m]), as_bf16x8_8(b[n]), acc[m][n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // SKIP: a wave whose 128 rows of the item hold no row of its tile (an
  // item of at most 128 rows: cold experts, the last tile of a group) reads
  // no activation chunks and multiplies nothing for the whole item; it still
  // issues its share of the block's loads, reads the weight operand the ring
  // hands to the next item, and takes part in every barrier. Its results
  // are never stored. The test costs about 1.5% when every item is full, so
  // the launcher picks this form only when items of at most 128 rows are
  // common.
  int busy = 1;
  auto set_active = [&](const Tile& t) {
    if constexpr (SKIP) busy = __builtin_amdgcn_readfirstlane(t.row1 - t.row0 > wm * 128 ? 1 : 0);
  };

  // Epilogue through this wave's 4 KB staging area, one 16-row tile at a
  // time (accumulator layout: lane holds column lane & 15 of each 16-column
  // tile, rows 4*(lane >> 4) + v); whole rows are stored 16 bytes per lane.
  auto epilogue = [&](const Tile& t, int nb) {
    if constexpr (EPI == EPI_SWIGLU) {
      constexpr int LDW = 40;  // 16 rows x 32 bf16 columns, rows padded to 40
      bf16_t* wbuf = (bf16_t*)&stg[wave][0];
      const int col0 = nb * BN + wn * 32;
      // fp8: the scales of this lane's columns (clamped: columns past N are never stored)
      float fg[2] = {1.f, 1.f}, fu[2] = {1.f, 1.f};
      if constexpr (F8) {
        const float* sg = group_scale(p, p.s0, p.s0_extra, t.group);
        const float* su = group_scale(p, p.s1, p.s1_extra, t.group);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int sc = col0 + n * 16 + (lane & 15) < p.N ? col0 + n * 16 + (lane & 15) : p.N - 1;
          fg[n] = sg[sc];
          fu[n] = su[sc];
        }
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            wbuf[(4 * (lane >> 4) + v) * LDW + n * 16 + (lane & 15)] =
                F8 ? f32_to_bf16(silu(acc[m][n][v] * fg[n]) * (acc[m][n + 2][v] * fu[n]))
                   : f32_to_bf16(silu(acc[m][n][v]) * acc[m][n + 2][v]);
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
      float fd[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (F8) {
        const float* sd = group_scale(p, p.s0, p.s0_extra, t.group);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int sc = col0 + n * 16 + (lane & 15) < p.N ? col0 + n * 16 + (lane & 15) : p.N - 1;
          fd[n] = sd[sc];
        }
      }
      // routed rows in the 16-bit format (the item's rows are all on one side of out16_rows)
      const bool half = p.out16 != nullptr && t.row0 < p.out16_rows;
      const int64_t row_shift = p.out16 != nullptr ? p.out16_rows : 0;
      // 16-bit form: this lane's row of pass 0 of row tile 0 (rows advance by 4 per pass), its
      // 4 columns and its row chunk's exponent byte; rows left before the item's end
      const int64_t rb = (int64_t)t.row0 + wm * 128 + (lane >> 4);
      const int rows_left = (int)((int64_t)t.row1 - rb);
      const bool col_ok = col0 + (lane & 15) * 4 < p.N;
      uint16_t* q16 = half ? p.out16 + rb * p.ldo + col0 + (lane & 15) * 4 : nullptr;
      uint8_t* qe = half ? p.out16_exp + rb * (p.ldo >> 6) + (col0 >> 6) : nullptr;
      const int64_t step16 = 4 * p.ldo, stepe = 4 * (p.ldo >> 6);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 4 * (lane >> 4) + v;
            wbuf[row * 64 + ((n ^ ((row >> 2) & 3)) << 4) + (lane & 15)] = F8 ? acc[m][n][v] * fd[n] : acc[m][n][v];
          }
        // 16 lanes per row (4 floats each), 4 rows per pass, 4 passes
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
          const int rr16 = pass * 4 + (lane >> 4), c4 = (lane & 15) * 4;
          float4 v = *(const float4*)&wbuf[rr16 * 64 + (c4 ^ (((rr16 >> 2) & 3) << 4))];
          const int64_t r = (int64_t)t.row0 + wm * 128 + m * 16 + rr16;
          const int col = col0 + c4;
          if (half) {
            // the row's 64-column maximum of |y| over its 16 lanes (one DPP row), taken on the
            // bit patterns (non-negative floats order like unsigned integers), then its exponent
            const uint32_t ax = __float_as_uint(v.x) & 0x7fffffffu, ay = __float_as_uint(v.y) & 0x7fffffffu;
            const uint32_t az = __float_as_uint(v.z) & 0x7fffffffu, aw = __float_as_uint(v.w) & 0x7fffffffu;
            uint32_t a = max(max(ax, ay), max(az, aw));
            a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xb1, 0xf, 0xf, true));
            a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4e, 0xf, 0xf, true));
            a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x141, 0xf, 0xf, true));
            a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x140, 0xf, 0xf, true));
            int e = (int)(a >> 23);
            e = e < EXP16_MIN ? EXP16_MIN : e;
            const float sc = ldexpf(1.f, EXP16_BIAS - e);  // exact power of two
            const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.x * sc)) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.y * sc)) << 16);
            const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.z * sc)) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v.w * sc)) << 16);
            if (m * 16 + pass * 4 < rows_left && col_ok) {
              // read once, by the combine: non-temporal
              typedef uint32_t u32x2_st __attribute__((ext_vector_type(2)));
              __builtin_nontemporal_store(u32x2_st{lo, hi}, (u32x2_st*)(q16 + (m * 4 + pass) * step16));
              if ((lane & 15) == 0) qe[(m * 4 + pass) * stepe] = (uint8_t)e;
            }
          } else if (r < t.row1 && col < p.N) {
            if (p.bias) {
              v.x += p.bias[col];
              v.y += p.bias[col + 1];
              v.z += p.bias[col + 2];
              v.w += p.bias[col + 3];
            }
            // read once, by the combine: non-temporal, so it does not displace operands in L2
            typedef float f32x4_st __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(f32x4_st{v.x, v.y, v.z, v.w},
                                        (f32x4_st*)&((float*)p.out)[(r - row_shift) * p.ldo + col]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Each ring holds stages in one sequence running across this block's
  // items. Weights: global step s (item j, step k: s = j*nk + k) lives in
  // slot s % 4; while step k is multiplied the ring holds steps k .. k+3
  // (landed or in flight). Activations: global stage (item j, stage h:
  // j*nk/2 + h, covering steps 2h and 2h+1) lives in slot stage % 2; while
  // stage h is multiplied stage h+1 is in flight. After the last item,
  // stages past its end re-load its last stage (never multiplied), so every
  // trip issues the same loads and fixed wait counts hold.
  //
  // Step k: (1) wait until this wave's loads of weight step k+1 (and, for
  // even k, of activation stage k/2) have landed; (2) lgkmcnt(0) + barrier:
  // every wave's loads are visible and every wave has finished reading
  // weight step k-1 (and, for even k, stage k/2-1), so (3) those slots are
  // refilled: even k issues stage k/2+1 (4 loads per lane) and weight step
  // k+3 (2), odd k weight step k+3 (2), of this item or else of the next
  // one; (4) the activation chunks of step k and the weight chunks of step
  // k+1 are read from LDS while (5) the matrix cores multiply step k. At
  // even k the loads younger than those waited for are weight step k+2 (2);
  // at odd k, stage k/2+1 and weight step k+2 (6).
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
  if constexpr (!F8) {
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
      if constexpr (!odd) {
        if (!SKIP || busy) read_a((baseA + h) & 1, 0, a);
        read_b((baseB + k + 1) % B8_NS, b_next);
        if (!SKIP || busy) multiply_refill(a, b_cur, (baseA + h) & 1);
      } else {
        read_b((baseB + k + 1) % B8_NS, b_next);
        if (!SKIP || busy) multiply_ready(a, b_cur);
      }
    };
    for (;;) {
  #pragma unroll
      for (int m = 0; m < 8; ++m)
  #pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      set_active(t_cur);
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
  } else {
    // fp8 weights: trips of one A stage and one weight stage (64 contraction
    // elements, two MFMA steps), one wait and one barrier per trip. Per wave,
    // trip h issues A(h+1) (4 loads) and then weight stage h+2 (2 loads); at
    // the start of trip h, A(h) and weight stage h must have landed, so only
    // weight stage h+1 (issued after A(h)) may still be in flight. A slot
    // (h+1) % 2 was last read in trip h-1 and weight slot (h+2) % 4 in trip
    // h-2, both before this trip's barrier.
    int baseA = 0, baseB = 0;  // slots of the current item's first stages
    const int last = nh - 1;
    u32x4_8 a[8], b[4], raw[4];
    issue_a(0, 0);
    issue_b(0, 0);
    issue_b(1, 1);  // nh >= 2: the contraction is at least 128
    for (;;) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      set_active(t_cur);
#pragma unroll 1
      for (int h = 0; h < nh; ++h) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm8(2));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int ha = h + 1;  // A stage to issue, counted from this item's start
        if (ha == nh && has_next) set_a_sources(rows);
        issue_a((baseA + ha) & 1, ha < nh ? ha : (has_next ? ha - nh : last));
        const int hb = h + 2;  // weight stage to issue
        if (hb == nh && has_next) set_b_sources(t_next, nb_next);
        issue_b((baseB + hb) % B8_NS, hb < nh ? hb : (has_next ? hb - nh : last));
        if (!SKIP || busy) {
          read_b8((baseB + h) % B8_NS, raw);
          read_a((baseA + h) & 1, 0, a);
          asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");  // the 4 weight reads have landed
          __builtin_amdgcn_sched_barrier(0);
          convert_b(raw, 0, b);
          multiply_a_only(a, b);
          read_a((baseA + h) & 1, 1, a);
          convert_b(raw, 1, b);
          multiply_a_only(a, b);
        }
      }
      epilogue(t_cur, nb_cur);
      if (!has_next) break;
      baseA = (baseA + nh) & 1;
      baseB = (baseB + nh) % B8_NS;
      t_cur = t_next;
      nb_cur = nb_next;
      L_next += L_step;
      has_next = L_next < L_end;
      if (has_next) {
        map_item(L_next, t_next, nb_next);
        load_rows(t_next, rows);
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm8(0));
}

// Compute units of the device `s` runs on (the runtime caches the attribute,
// so asking on every launch is cheap and holds no state here).
hipError_t stream_cus(hipStream_t s, int* cus) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, (int)dev);
  return e;
}

}  // namespace

hipError_t launch_grouped_gemm_big8(int epi, const GemmArgs& g, hipStream_t s) {
  if (g.max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.b_fp8 && !g.b_packed) return hipErrorInvalidValue;  // fp8 codes come in the packed layout only
  if (g.Kdim % B8_AKS || g.Kdim < 2 * B8_AKS) return hipErrorInvalidValue;
  if ((uint64_t)g.n_a_rows * (uint64_t)g.Kdim / 8u > 0xffffffffull) return hipErrorInvalidValue;
  if (g.N % 8 || g.ldo % 8) return hipErrorInvalidValue;
  if (g.out16 && (epi != EPI_F32 || g.N % 64 || g.ldo != g.N || !g.out16_exp)) return hipErrorInvalidValue;
  int cus = 0;
  const hipError_t ce = stream_cus(s, &cus);
  if (ce != hipSuccess) return ce;
  cus = cus > 8 ? cus : 8;
  const int BN = epi == EPI_SWIGLU ? B8_ROWS / 2 : B8_ROWS;
  const int n_nb = (g.N + BN - 1) / BN;
  int64_t blocks = ((int64_t)g.max_tiles * n_nb + 7) / 8 * 8;
  const int64_t cap = (int64_t)cus / 8 * 8;
  blocks = blocks < cap ? blocks : cap;
  // mean rows per group below 160: many items of at most 128 rows (half of
  // the tiles at 4096 tokens over 289 groups), where the SKIP form gains
  // about 8%; above, nearly every item is full and the plain form is faster
  const bool skip = g.b_packed && g.dense_rows < 160 * (int64_t)(g.n_main + (g.b0_extra ? 1 : 0));
  if (g.b_fp8) {
    if (skip) {
      if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, true, true, true><<<(unsigned)blocks, 512, 0, s>>>(g);
      else gemm_bf16_big8<EPI_F32, true, true, true><<<(unsigned)blocks, 512, 0, s>>>(g);
    } else {
      if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, true, true, false><<<(unsigned)blocks, 512, 0, s>>>(g);
      else gemm_bf16_big8<EPI_F32, true, true, false><<<(unsigned)blocks, 512, 0, s>>>(g);
    }
  } else if (g.b_packed) {
    if (skip) {
      if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, true, false, true><<<(unsigned)blocks, 512, 0, s>>>(g);
      else gemm_bf16_big8<EPI_F32, true, false, true><<<(unsigned)blocks, 512, 0, s>>>(g);
    } else {
      if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, true, false, false><<<(unsigned)blocks, 512, 0, s>>>(g);
      else gemm_bf16_big8<EPI_F32, true, false, false><<<(unsigned)blocks, 512, 0, s>>>(g);
    }
  } else {
    if (epi == EPI_SWIGLU) gemm_bf16_big8<EPI_SWIGLU, false, false, false><<<(unsigned)blocks, 512, 0, s>>>(g);
    else gemm_bf16_big8<EPI_F32, false, false, false><<<(unsigned)blocks, 512, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
