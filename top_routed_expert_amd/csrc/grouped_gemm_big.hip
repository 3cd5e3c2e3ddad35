// Expert GEMMs for many rows per expert (prefill): 256 x 256 block tiles.
//
// Every expert is an independent FFN (page "Step3.5 Flash 大模型技术深度解析",
// section 3.2.1). With a few hundred rows per expert, the weights of one
// column block should leave HBM once and be multiplied by all of the
// expert's rows; a 256-row tile covers a whole expert in most cases, and a
// 256-weight-row tile halves the operand bytes per flop pulled from L2
// relative to 128 x 256 tiles.
//
// Work item: one (row tile, column block) pair. Block: 4 waves in a 2 x 2
// layout, each wave 128 rows x 128 weight rows = 8 x 8 MFMA 16x16x32 tiles
// (256 fp32 accumulators per lane). For gate/up the 256 weight rows of an
// item are [gate c0..c0+63, up c0..c0+63, gate c0+64..c0+127, up
// c0+64..c0+127], so each wave holds the gate and up sums of the same 64
// columns and applies the SwiGLU in registers.
//
// Persistent blocks: one block per CU walks its share of the items. The
// load stream runs on across items: the last stages of an item issue the
// first stages of the next one, so items meet with no pipeline drain and
// an item's epilogue (results through LDS to HBM) runs while the next
// item's operands are already in flight.
//
// Both operands go HBM/L2 -> LDS through direct loads (global_load_lds,
// 16 bytes per lane, no VGPR staging). The weights (B) stream from HBM
// through a ring of NS = 4 stages of one 32-element MFMA step (16 KB each).
// The gathered activation rows (A) come mostly from L2 and move in stages
// of two MFMA steps, 128 bytes of each row (32 KB per stage, two slots):
// a 64-byte piece of a row uses half of a 128-byte cache line, and fetching
// whole lines raises the per-CU fetch rate of the gathered rows by about
// 40%. With a 32 KB epilogue staging area that fills the 160 KB of LDS.
// The B operand of a step is read from LDS into registers one step ahead
// (two register sets) and the A operand row tile by row tile in the step
// itself, so the LDS reads overlap the matrix-core work. Waits are
// explicit: a wave waits for its own loads with s_waitcnt vmcnt (loads
// complete in issue order), then one s_barrier per step makes every wave's
// loads visible and ends every wave's reads of the slots about to be
// refilled. The barrier is issued as inline asm with a memory clobber: the
// compiler may not move memory accesses across it and does not add a drain
// of its own.
//
// FP8 weights (F8): the codes of a weight stage cover 64 contraction
// elements (a 1 KB fragment per 16 weight rows, the packed fp8 layout), so
// both operands move in 64-element stages and a trip of two MFMA steps needs
// one wait and one barrier. A wave reads its 8 weight fragments once per
// trip, converts the first halves to bf16 operands for the first step and
// the second halves for the second, and the epilogue applies the per-column
// scales.
//
// A rows in LDS are 128 bytes (eight 16-byte chunks); chunk q of row r is
// stored at position q ^ ((r >> 1) & 7), so the 16-byte MFMA operand reads
// of 16 consecutive rows cover all banks once. B rows without packing are
// 64 bytes with chunk q at q ^ ((r >> 1) & 3). With packed weights (PK)
// each 16-row group of B is one 1 KB fragment copied as it is (lane order),
// which the operand reads take at 16 bytes per lane, conflict-free.
#include "moe_internal.h"

// The operand-read lambdas capture their asm operands explicitly (clang's
// device pass does not capture names used only as asm operands); the host
// pass, which does not see the asm's use, would warn about those captures.
#pragma clang diagnostic ignored "-Wunused-lambda-capture"

namespace moe {

namespace {

#ifndef MOE_BIG_NS
#define MOE_BIG_NS 4
#endif
constexpr int BIG_NS = MOE_BIG_NS;  // B ring stages
constexpr int BIG_KS = 32;     // contraction elements per B stage (one MFMA step)
constexpr int A_KS = 64;       // contraction elements per A stage (two MFMA steps)
constexpr int BIG_ROWS = 256;  // A rows and B (weight) rows per item
#ifndef MOE_BIG_CHUNK
#define MOE_BIG_CHUNK 16
#endif
constexpr int CHUNK = MOE_BIG_CHUNK;  // row tiles of one group that share weight columns in flight
// Cache policy of the weight loads: non-temporal. Every weight byte is used
// by one item only (per row tile), so it should not push the activation
// rows, which the column blocks of a row tile share, out of L2.
constexpr int CPOL_NT = 2;
static_assert(BIG_NS >= 4 && 2 * 32 + BIG_NS * 16 + 32 <= 160, "rings + staging must fit 160 KB of LDS");

typedef __attribute__((address_space(3))) void lds_void_t;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte operand chunk

__device__ __forceinline__ bf16x8 as_bf16x8_big(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// s_waitcnt immediate (gfx9 encoding) waiting for at most `vm` outstanding
// vector-memory operations and leaving the other counters unconstrained.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }   // 64-byte B rows
__device__ __forceinline__ int swzA(int row) { return (row >> 1) & 7; }  // 128-byte A rows

template <int EPI, bool PK, bool F8 = false>
__global__ void __launch_bounds__(256) gemm_bf16_big(GemmArgs p) {
  static_assert(!F8 || PK, "fp8 weights are packed");
  __shared__ __attribute__((aligned(16))) bf16_t ldsA[2][BIG_ROWS * A_KS];
  __shared__ __attribute__((aligned(16))) bf16_t ldsB[BIG_NS][BIG_ROWS * BIG_KS];
  __shared__ __attribute__((aligned(16))) float stg[4][16 * 128];  // epilogue staging, 8 KB per wave

  const int BN = EPI == EPI_SWIGLU ? BIG_ROWS / 2 : BIG_ROWS;  // output columns per item
  const int n_nb = (p.N + BN - 1) / BN;
  const int n_tiles = p.tiles ? *p.n_tiles : (int)((p.dense_rows + BIG_ROWS - 1) / BIG_ROWS);
  const int active = n_tiles * n_nb;
  // Hardware places block b on XCD b % 8. The active items, counted on the
  // device, are split into 8 contiguous runs, one per XCD (column blocks
  // fastest, so the items of one row tile share an L2); the XCD's blocks
  // take its items in turn.
  const int per_xcd = (active + 7) >> 3;
  const int L_begin = (blockIdx.x & 7) * per_xcd;
  const int L_end = L_begin + per_xcd < active ? L_begin + per_xcd : active;
  const int L_step = gridDim.x >> 3;
  int L = L_begin + (blockIdx.x >> 3);
  if (L >= L_end) return;

  // the wave index as a scalar: branches on it are uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kdim = p.Kdim, nk = Kdim / BIG_KS;
  const bf16_t* A = (const bf16_t*)p.a;

  // Item L -> (row tile, column block). A group (expert) with several row
  // tiles runs in chunks of up to CHUNK row tiles with the row tile
  // fastest, so the items running together on an XCD read the same weight
  // columns (read from HBM once, then from L2) instead of each row tile
  // streaming all of the expert's weights again. Single-tile groups keep
  // column blocks fastest. The group's items are L = first*n_nb ..
  // (first+count)*n_nb - 1 either way.
  auto map_item = [&](int L, Tile& t, int& nb) {
    int ti = L / n_nb;
    nb = L - ti * n_nb;
    if (p.tiles) {
      const Tile g = p.tiles[ti];
      const int first = g.first;
      int count = g.count;
      count = first + count <= n_tiles ? count : n_tiles - first;  // malformed table: stay in range
      if (count > 1 && first >= 0 && first <= ti && ti < first + count) {
        const int local = L - first * n_nb;
        const int c = local / (CHUNK * n_nb);
        const int wc = count - c * CHUNK < CHUNK ? count - c * CHUNK : CHUNK;
        const int local2 = local - c * CHUNK * n_nb;
        nb = local2 / wc;
        ti = first + c * CHUNK + local2 % wc;
      }
      t = p.tiles[ti];
    } else {
      t.group = 0;
      t.row0 = ti * BIG_ROWS;
      t.row1 = (int32_t)((int64_t)t.row0 + BIG_ROWS < p.dense_rows ? t.row0 + BIG_ROWS : p.dense_rows);
    }
  };

  // Direct-load sources of an item. A load instruction i (0..7) of this
  // wave fills rows R = wave*64 + i*8 .. R+7 of an A stage; lane l writes
  // the 16 bytes at LDS position (row R + l/8, physical chunk l%8), i.e.
  // logical chunk (l%8) ^ swzA(row). B load instruction i (0..3) fills
  // weight rows R = wave*64 + i*16 .. R+15 of a B stage: the fragment of
  // those rows (packed) or row R + l/4, chunk (l%4) ^ swz(row) (rows).
  // Rows outside the tile read row 0 (never stored).
  // Source rows of this wave's A loads for an item (gather read early:
  // the loads of the next item's rows are issued at the start of the
  // current item, so setting the sources inside the loop needs no load).
  auto load_rows = [&](const Tile& t, int32_t(&rows)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = (int64_t)t.row0 + wave * 64 + i * 8 + (lane >> 3);
      int64_t src = -1;
      if (r < t.row1) {
        src = r < p.n_gather ? (int64_t)p.gather[r] : r - p.n_gather;
        if (src >= p.n_a_rows) src = -1;
      }
      rows[i] = (int32_t)(src >= 0 ? src : 0);
    }
  };
  // A sources as 16-byte-unit offsets from A (the launcher checks that
  // n_a_rows * Kdim / 8 fits in 32 bits), B sources as pointers.
  uint32_t aoff[8];
  const bf16_t* bsrc[4];
  auto set_a_sources = [&](const int32_t(&rows)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wave * 64 + i * 8 + (lane >> 3);
      aoff[i] = (uint32_t)rows[i] * (uint32_t)(Kdim >> 3) + (uint32_t)((lane & 7) ^ swzA(row));
    }
  };
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
    for (int i = 0; i < 4; ++i) {
      const int row = wave * 64 + i * 16 + (lane >> 2);
      const int q = (lane & 3) ^ swz(row);
      // weight row `row` of the item
      int col;
      const bf16_t* base;
      if constexpr (EPI == EPI_SWIGLU) {
        const int seg = row >> 6;  // gate, up, gate, up
        col = nb * BN + (seg >> 1) * 64 + (row & 63);
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
        // the 16 rows of this instruction are one fragment column tile
        int ct = (col - (row & 15)) >> 4;
        const int ct_last = (p.N + 15) / 16 - 1;
        ct = ct < ct_last ? ct : ct_last;
        bsrc[i] = base + packed_offset(ct, 0, lane, Kdim);
      } else {
        col = col < p.N ? col : p.N - 1;
        bsrc[i] = base + (int64_t)col * Kdim + q * 8;
      }
    }
  };

  auto issue_a = [&](int slot, int ja) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(A + (uint64_t)aoff[i] * 8u + ja * A_KS),
                                       (lds_void_t*)&ldsA[slot][(wave * 64 + i * 8) * A_KS], 16, 0, 0);
  };
  auto issue_b = [&](int slot, int ks) {  // ks: a 32-element step (bf16) or a 64-element stage (fp8)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(
          F8 ? (const void*)((const char*)bsrc[i] + (int64_t)ks * FP8_FRAG)
             : (const void*)(bsrc[i] + (PK ? ks * PACKED_FRAG : ks * BIG_KS)),
          (lds_void_t*)&ldsB[slot][(wave * 64 + i * 16) * BIG_KS], 16, 0, CPOL_NT);
  };

  // wave (wm, wn): rows wm*128 .., weight rows wn*128 ..
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[8][8];

  // operand read of lane (r = lane & 15, q = lane >> 4) from a 16-row tile.
  // LDS byte offsets of this lane's operand chunks inside a slot: the row
  // swizzles depend on the row modulo 16 only, so A row tile m is the first
  // one's offset + 2048 m and B row tile n the first one's + 1024 n, an
  // immediate of the read instruction. The two MFMA steps of an A stage read
  // logical chunks q and q + 4 of a row.
  const int rq = lane >> 4, rr = lane & 15;
  const uint32_t aoffA0 = (uint32_t)((wm * 128 + rr) * A_KS + ((rq ^ swzA(rr)) << 3)) * 2u;
  const uint32_t aoffA1 = (uint32_t)((wm * 128 + rr) * A_KS + (((rq + 4) ^ swzA(rr)) << 3)) * 2u;
  const uint32_t boff0 = PK ? (uint32_t)(wn * 128 * BIG_KS) * 2u + (uint32_t)lane * 16u
                            : (uint32_t)((wn * 128 + rr) * BIG_KS + ((rq ^ swz(wn * 128 + rr)) << 3)) * 2u;
  const uint32_t ldsA_base = (uint32_t)(uintptr_t)(lds_void_t*)&ldsA[0][0];
  const uint32_t ldsB_base = (uint32_t)(uintptr_t)(lds_void_t*)&ldsB[0][0];
  constexpr uint32_t SLOT_A = BIG_ROWS * A_KS * 2u, SLOT_B = BIG_ROWS * BIG_KS * 2u;
  // Operand reads are inline ds_read_b128: the compiler cannot prove they do
  // not alias the direct loads in flight and would otherwise drain every
  // load before each read.
  auto read_b = [&](int slot, u32x4(&b)[8]) {
    const uint32_t addr = ldsB_base + (uint32_t)slot * SLOT_B + boff0;
    // (explicit captures: clang does not capture names used only as asm operands)
    static_for<0, 8>([&b, addr](auto N) {
      constexpr int n = decltype(N)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(b[n]) : "v"(addr), "n"(n * 1024));
    });
  };
  auto read_a = [&](int slot, int sub, u32x4(&a)[8]) {
    const uint32_t addr = ldsA_base + (uint32_t)slot * SLOT_A + (sub ? aoffA1 : aoffA0);
    static_for<0, 8>([&a, addr](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[m]) : "v"(addr), "n"(m * 2048));
    });
  };
  // Row tile m multiplies as soon as its A chunk is in: LDS reads complete in
  // issue order, and the 8 A reads are issued before the 8 B reads of the
  // next stage, so A chunk m has landed at lgkmcnt(15 - m). Each wait names
  // the register it guards and a scheduling barrier closes every row tile,
  // so no multiply moves above the wait that covers its operand.
  auto multiply = [&](u32x4(&a)[8], const u32x4(&b)[8]) {
    static_for<0, 8>([&](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a[m]) : "n"(15 - m));
#pragma unroll
      for (int n = 0; n < 8; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_big(a[m]), as_bf16x8_big(b[n]), acc[m][n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // fp8: this wave's 8 weight fragments of a stage, 16 bytes per lane (both
  // MFMA steps' codes); raw[n] lands at lgkmcnt(15 - n) when the 8 A reads
  // follow them.
  auto read_b8 = [&](int slot, u32x4(&raw)[8]) {
    const uint32_t addr = ldsB_base + (uint32_t)slot * SLOT_B + (uint32_t)(wn * 8) * 1024u + (uint32_t)lane * 16u;
    static_for<0, 8>([&raw, addr](auto N) {
      constexpr int n = decltype(N)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(raw[n]) : "v"(addr), "n"(n * 1024));
    });
  };
  // operands of MFMA step `hi` (0, 1) of a stage from the raw codes
  auto convert_b = [&](const u32x4(&raw)[8], int hi, u32x4(&b)[8]) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint4 v = hi ? fp8x8_bf16x8(raw[n].z, raw[n].w) : fp8x8_bf16x8(raw[n].x, raw[n].y);
      b[n] = u32x4{v.x, v.y, v.z, v.w};
    }
  };
  // multiply with the A chunks as the only LDS reads in flight behind them
  auto multiply_a_only = [&](u32x4(&a)[8], const u32x4(&b)[8]) {
    static_for<0, 8>([&](auto M) {
      constexpr int m = decltype(M)::value;
      asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a[m]) : "n"(7 - m));
#pragma unroll
      for (int n = 0; n < 8; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_big(a[m]), as_bf16x8_big(b[n]), acc[m][n], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Epilogue of an item through this wave's staging area, one 16-row tile
  // at a time: the wave writes its results (accumulator layout: lane holds
  // column lane & 15 of each 16-column tile, rows 4*(lane >> 4) + v), then
  // reads whole rows back 16 bytes per lane and stores them, so every store
  // instruction writes full contiguous row runs. The staging area is the
  // wave's own, outside the ring, so no barrier is needed around it.
  auto epilogue = [&](const Tile& t, int nb) {
    if constexpr (EPI == EPI_SWIGLU) {
      // 16 rows x 64 bf16 columns; rows padded to 72 elements
      constexpr int LDW = 72;
      bf16_t* wbuf = (bf16_t*)&stg[wave][0];
      const int col0 = nb * BN + wn * 64;
      const float* sg = F8 ? group_scale(p, p.s0, p.s0_extra, t.group) : nullptr;
      const float* su = F8 ? group_scale(p, p.s1, p.s1_extra, t.group) : nullptr;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          // fp8: the scales of this lane's column (clamped: columns past N are never stored)
          const int sc = col0 + n * 16 + (lane & 15) < p.N ? col0 + n * 16 + (lane & 15) : p.N - 1;
          const float fg = F8 ? sg[sc] : 1.f, fu = F8 ? su[sc] : 1.f;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            wbuf[(4 * (lane >> 4) + v) * LDW + n * 16 + (lane & 15)] =
                F8 ? f32_to_bf16(silu(acc[m][n][v] * fg) * (acc[m][n + 4][v] * fu))
                   : f32_to_bf16(silu(acc[m][n][v]) * acc[m][n + 4][v]);
        }
        // 8 lanes per row (16 bytes each), 8 rows per pass, 2 passes
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          const int rr16 = pass * 8 + (lane >> 3), c8 = (lane & 7) * 8;
          const uint4 v = *(const uint4*)&wbuf[rr16 * LDW + c8];
          const int64_t r = (int64_t)t.row0 + wm * 128 + m * 16 + rr16;
          const int col = col0 + c8;
          if (r < t.row1 && col < p.N) *(uint4*)&((bf16_t*)p.out)[r * p.ldo + col] = v;
        }
        __builtin_amdgcn_sched_barrier(0);  // one row tile at a time (register pressure)
      }
    } else {
      // 16 rows x 128 fp32 columns; 16-column groups XOR-swizzled by
      // (row >> 2) & 3, so the four rows one write instruction covers land
      // in different banks (no padding: the area is exactly 8 KB)
      float* wbuf = &stg[wave][0];
      const int col0 = nb * BN + wn * 128;
      const float* sd = F8 ? group_scale(p, p.s0, p.s0_extra, t.group) : nullptr;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int sc = col0 + n * 16 + (lane & 15) < p.N ? col0 + n * 16 + (lane & 15) : p.N - 1;
          const float fd = F8 ? sd[sc] : 1.f;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 4 * (lane >> 4) + v;
            wbuf[row * 128 + ((n ^ ((row >> 2) & 3)) << 4) + (lane & 15)] = F8 ? acc[m][n][v] * fd : acc[m][n][v];
          }
        }
        // 32 lanes per row (16 bytes each), 2 rows per pass, 8 passes
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
          const int rr16 = pass * 2 + (lane >> 5), c4 = (lane & 31) * 4;
          float4 v = *(const float4*)&wbuf[rr16 * 128 + (c4 ^ (((rr16 >> 2) & 3) << 4))];
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

  // Each ring holds stages in one sequence running across this block's
  // items. B: global step s (item j, step k: s = j*nk + k) lives in slot
  // s % NS; while step k of the current item is multiplied the B ring holds
  // steps k .. k+NS-1 (landed or in flight). A: global A stage (item j,
  // stage h: j*nk/2 + h, covering steps 2h and 2h+1) lives in slot
  // (stage % 2); while stage h is multiplied stage h+1 is in flight. The B
  // operand is read one step ahead (two register sets), the A operand in the
  // step that uses it. After the last item, stages past its end re-load its
  // last stage (never multiplied), so every trip issues the same loads and
  // fixed wait counts hold.
  //
  // Step k: (1) wait until this wave's loads of B step k+1 (and, for even
  // k, of A stage k/2) have landed; (2) lgkmcnt(0) + barrier: every wave's
  // loads are visible and every wave has finished reading B step k-1 (and,
  // for even k, A stage k/2-1), so (3) those slots are refilled: for even k
  // A stage k/2+1 (8 loads per lane), then B step k+NS-1 (4 loads), of this
  // item or else of the next one; (4) the A chunks of step k and then the
  // B chunks of step k+1 are read from LDS while (5) the matrix cores
  // multiply step k. Loads issued in order per wave: even step k: A(k/2+1),
  // B(k+3); odd step: B(k+3). At even k the loads younger than those waited
  // for are B(k+2) (4); at odd k, A(k/2+1) and B(k+2) of step k-1 (12).
  static_assert(BIG_NS == 4, "the wait counts below assume a four-step B ring");
  const int nh = nk >> 1;  // A stages per item
  Tile t_cur, t_next;
  int nb_cur, nb_next;
  int32_t rows[8];
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
    int baseA = 0, baseB = 0;  // slots of the current item's first A stage and first B step
    const int lastA = nh - 1, lastB = nk - 1;
    u32x4 a[8], b0[8], b1[8];
    issue_a(0, 0);
  #pragma unroll
    for (int s = 0; s < BIG_NS - 1; ++s) issue_b(s, s);  // nk >= 4: steps 0..2 exist
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));             // A stage 0, B step 0
    asm volatile("s_barrier" ::: "memory");
    read_b(0, b0);
    auto step = [&](int k, auto ODD, const u32x4(&b_cur)[8], u32x4(&b_next)[8]) {
      constexpr bool odd = decltype(ODD)::value;
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(odd ? 12 : 4));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const int h = k >> 1;
      if constexpr (!odd) {
        const int ha = h + 1;  // A stage to issue, counted from this item's start
        if (ha == nh && has_next) set_a_sources(rows);  // from here on the next item's A stages
        issue_a((baseA + ha) & 1, ha < nh ? ha : (has_next ? ha - nh : lastA));
      }
      const int ks = k + BIG_NS - 1;  // B step to issue, counted from this item's start
      if (ks == nk && has_next) set_b_sources(t_next, nb_next);
      issue_b((baseB + ks) % BIG_NS, ks < nk ? ks : (has_next ? ks - nk : lastB));
      read_a((baseA + h) & 1, odd ? 1 : 0, a);
      read_b((baseB + k + 1) % BIG_NS, b_next);
      multiply(a, b_cur);
    };
    for (;;) {
  #pragma unroll
      for (int m = 0; m < 8; ++m)
  #pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      // nk is even (the contraction is a multiple of 64): one A stage, two
      // steps per trip, alternating the B register sets; every item starts
      // with b0.
  #pragma unroll 1
      for (int k = 0; k < nk; k += 2) {
        step(k, std::false_type{}, b0, b1);
        step(k + 1, std::true_type{}, b1, b0);
      }
      epilogue(t_cur, nb_cur);
      if (!has_next) break;
      baseA = (baseA + nh) & 1;
      baseB = (baseB + nk) % BIG_NS;
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
    // trip h issues A(h+1) (8 loads) and then weight stage h+2 (4 loads); at
    // the start of trip h, A(h) and weight stage h must have landed, so only
    // weight stage h+1 (issued after A(h)) may still be in flight. A slot
    // (h+1) % 2 was last read in trip h-1 and weight slot (h+2) % 4 in trip
    // h-2, both before this trip's barrier. The weight codes of a stage are
    // read once per trip, before the A chunks, and converted half by half.
    int baseA = 0, baseB = 0;  // slots of the current item's first stages
    const int last = nh - 1;
    u32x4 a[8], b[8], raw[8];
    issue_a(0, 0);
    issue_b(0, 0);
    issue_b(1, 1);  // nh >= 2: the contraction is at least 128
    for (;;) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int h = 0; h < nh; ++h) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        const int ha = h + 1;  // A stage to issue, counted from this item's start
        if (ha == nh && has_next) set_a_sources(rows);
        issue_a((baseA + ha) & 1, ha < nh ? ha : (has_next ? ha - nh : last));
        const int hb = h + 2;  // weight stage to issue
        if (hb == nh && has_next) set_b_sources(t_next, nb_next);
        issue_b((baseB + hb) % BIG_NS, hb < nh ? hb : (has_next ? hb - nh : last));
        read_b8((baseB + h) % BIG_NS, raw);
        read_a((baseA + h) & 1, 0, a);
        asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");  // the 8 weight reads have landed
        __builtin_amdgcn_sched_barrier(0);
        convert_b(raw, 0, b);
        multiply_a_only(a, b);
        read_a((baseA + h) & 1, 1, a);
        convert_b(raw, 1, b);
        multiply_a_only(a, b);
      }
      epilogue(t_cur, nb_cur);
      if (!has_next) break;
      baseA = (baseA + nh) & 1;
      baseB = (baseB + nh) % BIG_NS;
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
  // drain the trailing reads and the loads of the clamped stages before the block ends
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

int g_cus = 0;  // compute units of the device (queried once)

}  // namespace

hipError_t launch_grouped_gemm_big(int epi, const GemmArgs& g, hipStream_t s) {
  if (g.max_tiles <= 0 || g.N <= 0) return hipSuccess;
  // the main loop takes one A stage (two steps) per trip; the B ring's
  // hand-over to the next item needs at least NS - 1 steps per item
  if (g.Kdim % A_KS || g.Kdim < 2 * A_KS) return hipErrorInvalidValue;
  if ((uint64_t)g.n_a_rows * (uint64_t)g.Kdim / 8u > 0xffffffffull) return hipErrorInvalidValue;  // 32-bit A offsets
  if (g.N % 8 || g.ldo % 8) return hipErrorInvalidValue;    // the epilogue stores 8 bf16 / 4 fp32 columns at once
  if (g_cus == 0) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus = cus > 8 ? cus : 8;
  }
  const int BN = epi == EPI_SWIGLU ? BIG_ROWS / 2 : BIG_ROWS;
  const int n_nb = (g.N + BN - 1) / BN;
  // one block per CU (the kernel takes all of a CU's LDS), at most one per
  // possible item, a multiple of 8 so every XCD gets the same number
  int64_t blocks = ((int64_t)g.max_tiles * n_nb + 7) / 8 * 8;
  const int64_t cap = (int64_t)g_cus / 8 * 8;
  blocks = blocks < cap ? blocks : cap;
  if (g.b_fp8) {
    if (epi == EPI_SWIGLU) gemm_bf16_big<EPI_SWIGLU, true, true><<<(unsigned)blocks, 256, 0, s>>>(g);
    else gemm_bf16_big<EPI_F32, true, true><<<(unsigned)blocks, 256, 0, s>>>(g);
  } else if (g.b_packed) {
    if (epi == EPI_SWIGLU) gemm_bf16_big<EPI_SWIGLU, true><<<(unsigned)blocks, 256, 0, s>>>(g);
    else gemm_bf16_big<EPI_F32, true><<<(unsigned)blocks, 256, 0, s>>>(g);
  } else {
    if (epi == EPI_SWIGLU) gemm_bf16_big<EPI_SWIGLU, false><<<(unsigned)blocks, 256, 0, s>>>(g);
    else gemm_bf16_big<EPI_F32, false><<<(unsigned)blocks, 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

}  // namespace moe
