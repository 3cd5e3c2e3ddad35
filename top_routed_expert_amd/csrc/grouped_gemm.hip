// Grouped GEMMs of the MoE layer: the experts' gate/up projections with the
// SwiGLU epilogue, their down projections, and the router's linear layer
// (one group). Every expert is an independent FFN (page "Step3.5 Flash
// 大模型技术深度解析", section 3.2.1), so the permuted rows routed to expert e
// form one dense block multiplied by that expert's weights alone.
//
// Fast path (bf16, contraction length a multiple of 64): bf16 MFMA
// 16x16x32 with fp32 accumulation. A block owns up to BM = 16*MT rows of one
// expert and 4*NW*16 output columns (for gate/up: that many gate columns
// and the same up columns, so the SwiGLU is applied in registers). The A
// rows are gathered through the permutation on the fly (the permuted
// activations are never written to HBM) and staged in LDS, 64 contraction
// elements per stage, double buffered, XOR-swizzled so MFMA operand reads
// are bank-conflict free. The weights are streamed straight from HBM into
// VGPRs in MFMA operand layout, one stage ahead, and read once per row tile.
//
// Generic path (fp32, or shapes the fast path does not cover): 64x64 output
// tiles staged through LDS, plain fp32 FMA.
#include <type_traits>

#include "moe_internal.h"

#ifndef MOE_NS_SMALL
#define MOE_NS_SMALL 4  // pipeline depth of the 32-row tiles (few rows per expert: weight streaming)
#endif
#ifndef MOE_GU_NW_SMALL
#define MOE_GU_NW_SMALL 1  // 16-column tiles per wave (gate and up each), 32-row tiles
#endif
#ifndef MOE_DN_NW_SMALL
#define MOE_DN_NW_SMALL 1  // 16-column tiles per wave, down projection, 32-row tiles
#endif
#ifndef MOE_ROWS_32
#define MOE_ROWS_32 24  // mean rows per group up to which expert GEMMs use 32-row tiles (above ~24, many groups would need two)
#endif
#ifndef MOE_ROWS_64
#define MOE_ROWS_64 48  // ... up to which 64-row tiles (then 128-row tiles)
#endif
#ifndef MOE_ROWS_256
#define MOE_ROWS_256 48  // mean rows per group from which they use the 256 x 256 kernel (its skipping form below 160)
#endif
#ifndef MOE_NS_LARGE
#define MOE_NS_LARGE 4  // pipeline depth of the 128-row tiles
#endif


namespace moe {

namespace {


__device__ __forceinline__ bool fetch_tile(const GemmArgs& p, int ti, int BM, Tile& t) {
  if (p.tiles == nullptr) {
    const int64_t r0 = (int64_t)ti * BM;
    if (r0 >= p.dense_rows) return false;
    t.group = 0;
    t.row0 = (int32_t)r0;
    t.row1 = (int32_t)(r0 + BM < p.dense_rows ? r0 + BM : p.dense_rows);
    return true;
  }
  if (ti >= *p.n_tiles) return false;
  t = p.tiles[ti];
  return true;
}

// Number of row tiles of a launch (device schedule, or dense rows).
__device__ __forceinline__ int tile_count(const GemmArgs& p, int BM) {
  return p.tiles ? *p.n_tiles : (int)((p.dense_rows + BM - 1) / BM);
}

// Source row of problem row r (gathered through the permutation, or direct);
// -1 when it falls outside the A operand.
__device__ __forceinline__ int64_t source_row(const GemmArgs& p, int64_t r) {
  const int64_t src = r < p.n_gather ? (int64_t)p.gather[r] : r - p.n_gather;
  return (src >= 0 && src < p.n_a_rows) ? src : -1;
}

template <typename T>
__device__ __forceinline__ const T* group_b(const GemmArgs& p, const void* main, const void* extra,
                                            int g) {
  return g < p.n_main ? (const T*)main + (int64_t)g * p.b_stride : (const T*)extra;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte load of weights. Non-temporal (NT) for the expert GEMMs: each
// weight byte is used by one block only, so the loads stream past L2
// instead of displacing the shared activation rows. Measured: decode
// gate/up 0.634 -> 0.535 ms for the same bytes.
template <bool NT>
__device__ __forceinline__ uint4 load_b(const bf16_t* p) {
  if constexpr (NT) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *(const uint4*)p;
  }
}

// LDS offset (in bf16 elements) of 16-byte chunk `c` of staged row `r` (row
// length KS): chunks are XOR-swizzled by (r & 7) so the 16-byte operand reads
// of 8 consecutive rows hit distinct banks.
template <int KS>
__device__ __forceinline__ int lds_off(int r, int c) { return r * KS + ((c ^ (r & 7)) << 3); }

// EPI: epilogue; MT: 16-row MFMA tiles per block; NW: 16-column weight tiles
// per wave and operand; KSTEPS: 32-element MFMA steps per pipeline stage;
// NS: pipeline depth; PK: weights in the packed fragment layout (below);
// NT: weights loaded non-temporally (load_stream; not for the router, whose
// weights every row tile reads again); F8: weights are FP8 E4M3 codes in the
// packed fp8 layout (one 16-byte load per lane covers a stage's two MFMA
// steps), converted to bf16 in registers, with per-column scales applied in
// the epilogue. Loads of stage k+NS-1 are issued before stage k is
// multiplied, so NS-1 stages of weights (and A rows) are in flight per wave
// while the matrix cores work; the ring lives in VGPRs and the loop is
// unrolled by NS so every ring slot is a fixed register range.
template <int EPI, int MT, int NW, int KSTEPS, int NS, bool PK, bool NT, bool F8 = false>
__global__ void __launch_bounds__(256) gemm_bf16_mfma(GemmArgs p) {
  static_assert(!F8 || (PK && KSTEPS == 2), "fp8 weights: packed, one fragment (64 columns) per stage");
  constexpr int KS = 32 * KSTEPS;                       // contraction elements per stage
  constexpr int CPR = KS / 8;                           // 16-byte chunks per staged row
  constexpr int RPP = 256 / CPR;                        // rows staged per pass of the block
  constexpr int BM = 16 * MT;
  constexpr int NA = BM / RPP;                          // chunks staged per thread
  constexpr int NBT = EPI == EPI_SWIGLU ? 2 * NW : NW;  // weight tiles (16 columns) per wave
  constexpr int BN = 4 * NW * 16;                       // output columns per block
  static_assert(BM % RPP == 0, "row tile must be a whole number of staging passes");
  static_assert(NS >= 2, "pipeline needs at least two stages");
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * KS];

  // Hardware places block b on XCD b % 8. The grid is sized for the most
  // tiles the schedule can produce; the active (tile, column block) pairs,
  // counted on the device, are split evenly over the 8 XCDs, each XCD taking
  // a contiguous run with column blocks fastest: the column blocks of a row
  // tile (same A rows) and the row tiles of one expert (same weights) then
  // run together on one XCD and share its L2.
  const int n_nb = (p.N + BN - 1) / BN;
  const int active = tile_count(p, BM) * n_nb;
  const int per_xcd = (active + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  const int L = (blockIdx.x & 7) * per_xcd + slot;
  if (slot >= per_xcd || L >= active) return;
  const int ti = L / n_nb, nb = L - ti * n_nb;
  Tile t;
  if (!fetch_tile(p, ti, BM, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Kdim = p.Kdim;
  // contraction slice of this block (router split-K): stages [kbase, kbase + nk)
  const int nk = Kdim / KS / p.ksplit;
  const int kbase = (int)blockIdx.y * nk;
  const bf16_t* A = (const bf16_t*)p.a + (int64_t)kbase * KS;

  // A staging: this thread copies 16-byte chunk (tid % CPR) of local rows
  // tid / CPR + RPP*i. Rows outside the tile (or with an invalid source) read
  // row 0 of A instead: their outputs are never stored, and keeping every
  // load unconditional keeps the pipeline's wait counts exact.
  const bf16_t* arow[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int64_t r = (int64_t)t.row0 + tid / CPR + RPP * i;
    const int64_t src = r < t.row1 ? source_row(p, r) : -1;
    arow[i] = A + (src >= 0 ? src : 0) * Kdim + (tid % CPR) * 8;
  }

  // Weight rows of this wave: tile j covers output columns wcol0 + (j % NW)*16 + 0..15.
  // Lane (c = lane & 15, q = lane >> 4) reads column c, contraction offset q*8 of each
  // 32-element MFMA step. Columns past N are clamped to a valid row; their
  // results are never stored.
  const int wcol0 = nb * BN + wave * NW * 16;
  const bf16_t* bg = F8 ? (const bf16_t*)group_b<uint8_t>(p, p.b0, p.b0_extra, t.group)
                        : group_b<bf16_t>(p, p.b0, p.b0_extra, t.group);
  const bf16_t* bu = EPI == EPI_SWIGLU ? (F8 ? (const bf16_t*)group_b<uint8_t>(p, p.b1, p.b1_extra, t.group)
                                             : group_b<bf16_t>(p, p.b1, p.b1_extra, t.group))
                                       : bg;
  // Packed weights: the operand of a whole wave for one 16-column tile and
  // one MFMA step is one contiguous 1 KB fragment, lane l at l*16 bytes
  // (packed_offset); the tiles past the last one are clamped to it.
  const bf16_t* bptr[NBT];
#pragma unroll
  for (int j = 0; j < NBT; ++j) {
    const bf16_t* base = j < NW ? bg : bu;
    if constexpr (F8) {  // byte offsets into the fp8 codes
      int ct = (wcol0 + (j % NW) * 16) >> 4;
      const int ct_last = (p.N + 15) / 16 - 1;
      ct = ct < ct_last ? ct : ct_last;
      bptr[j] = (const bf16_t*)((const uint8_t*)base + fp8_offset(ct, kbase, lane, Kdim));
    } else if constexpr (PK) {
      int ct = (wcol0 + (j % NW) * 16) >> 4;
      const int ct_last = (p.N + 15) / 16 - 1;
      ct = ct < ct_last ? ct : ct_last;
      bptr[j] = base + packed_offset(ct, kbase * KSTEPS, lane, Kdim);
    } else {
      int col = wcol0 + (j % NW) * 16 + (lane & 15);
      col = col < p.N ? col : p.N - 1;
      bptr[j] = base + (int64_t)col * Kdim + (int64_t)kbase * KS + (lane >> 4) * 8;
    }
  }

  uint4 ra[NS][NA];
  uint4 rb[NS][NBT][KSTEPS];
  f32x4 acc[MT][NBT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NBT; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_stage = [&](uint4(&a)[NA], uint4(&b)[NBT][KSTEPS], int ks) {
#pragma unroll
    for (int j = 0; j < NBT; ++j) {
      if constexpr (F8) {  // one fragment (both MFMA steps) per stage
        b[j][0] = load_b<NT>((const bf16_t*)((const uint8_t*)bptr[j] + (int64_t)ks * FP8_FRAG));
      } else {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          b[j][s] = load_b<NT>(bptr[j] + (PK ? (ks * KSTEPS + s) * PACKED_FRAG : ks * KS + s * 32));
      }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) a[i] = *(const uint4*)(arow[i] + ks * KS);
  };
  auto store_a = [&](const uint4(&a)[NA], int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) *(uint4*)&sA[buf][lds_off<KS>(tid / CPR + RPP * i, tid % CPR)] = a[i];
  };
  auto compute = [&](int buf, const uint4(&b)[NBT][KSTEPS]) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint4 bop[NBT];
#pragma unroll
      for (int j = 0; j < NBT; ++j) {
        if constexpr (F8) bop[j] = s == 0 ? fp8x8_bf16x8(b[j][0].x, b[j][0].y) : fp8x8_bf16x8(b[j][0].z, b[j][0].w);
        else bop[j] = b[j][s];
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8 a =
            as_bf16x8(*(const uint4*)&sA[buf][lds_off<KS>(m * 16 + (lane & 15), s * 4 + (lane >> 4))]);
#pragma unroll
        for (int j = 0; j < NBT; ++j)
          acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(bop[j]), acc[m][j], 0, 0, 0);
      }
    }
  };

  // Software pipeline over nkp = nk rounded up to a multiple of NS stages.
  // Every trip of the loop runs NS stages with no exit and no conditional
  // memory operation, so the compiler's wait counts follow the fixed
  // instruction order: a stage's loads are waited for only when its A tile
  // is stored to LDS, NS-2 stages after they were issued. Stages past the
  // end load the last real stage again (never used) and stage zeros as
  // their A tile, so they add exactly zero to the accumulators.
  const int last = nk - 1;
  const int nkp = (nk + NS - 1) / NS * NS;
  auto store_next = [&](const uint4(&a)[NA], int k_next) {
    // component-wise mask (a select of whole vector structs would keep the
    // ring in memory instead of registers)
    const uint32_t keep = k_next < nk ? 0xffffffffu : 0u;
    uint4 v[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) v[i] = make_uint4(a[i].x & keep, a[i].y & keep, a[i].z & keep, a[i].w & keep);
    store_a(v, k_next & 1);
  };
  static_for<0, NS - 1>([&](auto S) {
    constexpr int s = decltype(S)::value;
    load_stage(ra[s], rb[s], s < nk ? s : last);
  });
  store_a(ra[0], 0);
  __syncthreads();
  for (int k0 = 0; k0 < nkp; k0 += NS) {
    static_for<0, NS>([&](auto U) {
      constexpr int u = decltype(U)::value;
      const int k = k0 + u;
      load_stage(ra[(u + NS - 1) % NS], rb[(u + NS - 1) % NS], k + NS - 1 < nk ? k + NS - 1 : last);
      compute(k & 1, rb[u]);
      store_next(ra[(u + 1) % NS], k + 1);
      __syncthreads();
    });
  }

  // Accumulator layout of a 16x16 MFMA tile: lane holds column (lane & 15),
  // rows 4*(lane >> 4) + v for v = 0..3.
  const int64_t rbase = (int64_t)t.row0 + (lane >> 4) * 4;
  const float* sc0 = F8 ? group_scale(p, p.s0, p.s0_extra, t.group) : nullptr;
  const float* sc1 = F8 && EPI == EPI_SWIGLU ? group_scale(p, p.s1, p.s1_extra, t.group) : nullptr;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int col = wcol0 + j * 16 + (lane & 15);
      if (col >= p.N) continue;
      // fp8 weights: the column's scale (one per weight row)
      const float f0 = F8 ? sc0[col] : 1.f;
      const float f1 = F8 && EPI == EPI_SWIGLU ? sc1[col] : 1.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t r = rbase + m * 16 + v;
        if (r >= t.row1) continue;
        if constexpr (EPI == EPI_SWIGLU) {
          const float gv = F8 ? acc[m][j][v] * f0 : acc[m][j][v];
          const float uv = F8 ? acc[m][j + NW][v] * f1 : acc[m][j + NW][v];
          ((bf16_t*)p.out)[r * p.ldo + col] = f32_to_bf16(silu(gv) * uv);
        } else {
          const float b = (p.bias && blockIdx.y == 0) ? p.bias[col] : 0.f;
          const float a = F8 ? acc[m][j][v] * f0 : acc[m][j][v];
          ((float*)p.out + (int64_t)blockIdx.y * p.slice_stride)[r * p.ldo + col] = a + b;
        }
      }
    }
  }
}

// Generic grouped GEMM: 64x64 output tile, 16x16 threads with 4x4 outputs
// each, contraction in chunks of 32 through LDS. The next chunk's operands
// are loaded into registers before the current chunk is multiplied, so a
// chunk's load latency overlaps the previous chunk's arithmetic (small
// layers are latency-bound here). TI is float or bf16_t.
template <typename TI, int EPI>
__global__ void __launch_bounds__(256) gemm_generic(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 32, PER = BM * BK / 256;
  constexpr int NB = EPI == EPI_SWIGLU ? 2 : 1;
  __shared__ float sA[BK][BM + 1];
  __shared__ float sB[NB][BK][BN + 1];

  const int n_nb = (p.N + BN - 1) / BN;
  const int ti = blockIdx.x / n_nb, nb = blockIdx.x - ti * n_nb;
  Tile t;
  if (!fetch_tile(p, ti, BM, t)) return;

  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const TI* A = (const TI*)p.a;
  const TI* B[NB];
  B[0] = group_b<TI>(p, p.b0, p.b0_extra, t.group);
  if constexpr (NB == 2) B[1] = group_b<TI>(p, p.b1, p.b1_extra, t.group);

  // Staging: element e = tid + 256*i is (row or column e / 32, contraction e % 32).
  const int kk = tid & (BK - 1);
  int64_t asrc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t r = (int64_t)t.row0 + ((tid + 256 * i) >> 5);
    asrc[i] = r < t.row1 ? source_row(p, r) : -1;
  }
  float ra[PER], rb[NB][PER];
  auto load = [&](int k0) {
    const int k = k0 + kk;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int rc = (tid + 256 * i) >> 5, col = nb * BN + rc;
      ra[i] = (asrc[i] >= 0 && k < p.Kdim) ? load_f32(A + asrc[i] * p.Kdim + k) : 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        rb[b][i] = (col < p.N && k < p.Kdim) ? load_f32(B[b] + (int64_t)col * p.Kdim + k) : 0.f;
    }
  };
  float acc[NB][4][4] = {};
  load(0);
  for (int k0 = 0; k0 < p.Kdim; k0 += BK) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int rc = (tid + 256 * i) >> 5;
      sA[kk][rc] = ra[i];
#pragma unroll
      for (int b = 0; b < NB; ++b) sB[b][kk][rc] = rb[b][i];
    }
    __syncthreads();
    if (k0 + BK < p.Kdim) load(k0 + BK);
#pragma unroll 8
    for (int c = 0; c < BK; ++c) {
      float a[4], bv[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[c][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[b][j] = sB[b][c][tx * 4 + j];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a[i], bv[b][j], acc[b][i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = (int64_t)t.row0 + ty * 4 + i;
    if (r >= t.row1) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = nb * BN + tx * 4 + j;
      if (col >= p.N) continue;
      if constexpr (EPI == EPI_SWIGLU) {
        store_out((TI*)p.out + r * p.ldo + col, silu(acc[0][i][j]) * acc[NB - 1][i][j]);
      } else {
        ((float*)p.out)[r * p.ldo + col] = acc[0][i][j] + (p.bias ? p.bias[col] : 0.f);
      }
    }
  }
}

// Device-side schedule: cut every group's row segment into tiles of BM rows,
// in group order. Segment bounds are clamped to [0, n_rows] and made
// non-decreasing, so malformed offsets cannot address rows out of range.
__global__ void __launch_bounds__(1024) build_tiles_kernel(const int32_t* __restrict__ offsets, int n_groups,
                                                           int64_t n_rows, int BM, Tile* __restrict__ tiles,
                                                           int32_t* __restrict__ n_tiles, int32_t max_tiles,
                                                           int skip_group) {
  __shared__ int32_t s_scan[1024];
  const int tid = threadIdx.x;
  const int per = (n_groups + 1023) / 1024;
  const int g0 = tid * per, g1 = min(g0 + per, n_groups);
  auto seg = [&](int g, int64_t& a, int64_t& b) {
    a = offsets[g];
    b = offsets[g + 1];
    a = a < 0 ? 0 : (a > n_rows ? n_rows : a);
    b = b < a ? a : (b > n_rows ? n_rows : b);
    if (g == skip_group) b = a;  // a group with no work (rows of pairs without an expert)
  };
  int mine = 0;
  for (int g = g0; g < g1; ++g) {
    int64_t a, b;
    seg(g, a, b);
    mine += (int)((b - a + BM - 1) / BM);
  }
  s_scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int slot = s_scan[tid] - mine;
  for (int g = g0; g < g1; ++g) {
    int64_t a, b;
    seg(g, a, b);
    const int first = slot, count = (int)((b - a + BM - 1) / BM);
    for (int64_t r = a; r < b; r += BM, ++slot)
      if (slot < max_tiles) tiles[slot] = Tile{g, (int32_t)r, (int32_t)(r + BM < b ? r + BM : b), first, count, 0, 0, 0};
  }
  if (tid == 1023) *n_tiles = min(s_scan[1023], max_tiles);
}

}  // namespace

int gemm_block_rows(bool fast, int64_t rows, int n_groups, bool allow_big) {
  if (!fast) return 64;
  if (rows <= MOE_ROWS_32 * (int64_t)n_groups) return 32;
  if (allow_big && rows >= MOE_ROWS_256 * (int64_t)n_groups) return 256;
  return rows <= MOE_ROWS_64 * (int64_t)n_groups ? 64 : 128;
}

// Up to 64 tokens: 16 slices (fewer when the stage count is not a multiple).
// More tokens: a few row tiles leave most compute units idle while each block
// walks the whole contraction, so the slices double (up to 16, dividing the
// stage count) while the grid stays within 384 blocks, about one and a half
// blocks per compute unit.
int router_ksplit(bool fast, int64_t T, int Kdim, int E) {
  if (!fast) return 1;
  const int nk = Kdim / 64;
  int ks = 16;
  if (T <= 64) {
    while (ks > 1 && nk % ks) ks >>= 1;
    return ks;
  }
  const int64_t BM = gemm_block_rows(fast, T, 1, false);
  const int64_t BN = E <= 512 ? 64 : 256;  // column width of the launch that takes BM-row tiles
  const int64_t blocks = (T + BM - 1) / BM * ((E + BN - 1) / BN);
  ks = 1;
  while (ks < 16 && nk % (2 * ks) == 0 && blocks * 2 * ks <= 384) ks *= 2;
  return ks;
}

int64_t gemm_max_tiles(int64_t n_rows, int n_groups, int block_rows) {
  return n_rows / block_rows + n_groups;  // sum over groups of ceil(len / BM)
}

hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int64_t n_rows, int block_rows, Tile* tiles,
                              int32_t* n_tiles, int32_t max_tiles, int skip_group, hipStream_t s) {
  build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, n_groups, n_rows, block_rows, tiles, n_tiles, max_tiles,
                                        skip_group);
  return hipGetLastError();
}

template <int EPI, int MT, int NW, int NS, int KSTEPS = 2>
static hipError_t launch_fast(const GemmArgs& g, hipStream_t s) {
  const int n_nb = (g.N + 4 * NW * 16 - 1) / (4 * NW * 16);
  const int64_t blocks = ((int64_t)g.max_tiles * n_nb + 7) / 8 * 8;
  const dim3 grid((unsigned)blocks, (unsigned)g.ksplit);
  if (g.b_fp8) {  // expert weights only (streamed, packed)
    if (g.b_reuse || KSTEPS != 2) return hipErrorInvalidValue;
    gemm_bf16_mfma<EPI, MT, NW, KSTEPS, NS, true, true, true><<<grid, 256, 0, s>>>(g);
  } else if (g.b_reuse) {
    if (g.b_packed) gemm_bf16_mfma<EPI, MT, NW, KSTEPS, NS, true, false><<<grid, 256, 0, s>>>(g);
    else gemm_bf16_mfma<EPI, MT, NW, KSTEPS, NS, false, false><<<grid, 256, 0, s>>>(g);
  } else {
    if (g.b_packed) gemm_bf16_mfma<EPI, MT, NW, KSTEPS, NS, true, true><<<grid, 256, 0, s>>>(g);
    else gemm_bf16_mfma<EPI, MT, NW, KSTEPS, NS, false, true><<<grid, 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int dtype, bool fast, int epi, int block_rows, const GemmArgs& g, hipStream_t s) {
  if (g.max_tiles <= 0 || g.N <= 0) return hipSuccess;
  if (g.b_fp8 && !fast) return hipErrorInvalidValue;  // fp8 weights: bf16 MFMA kernels only
  if (g.out16 && !fast) return hipErrorInvalidValue;
  if (!fast) {
    if (g.b_packed) return hipErrorInvalidValue;  // packed weights exist only on the bf16 MFMA path
    const int n_nb = (g.N + 63) / 64;
    const unsigned blocks = (unsigned)((int64_t)g.max_tiles * n_nb);
    if (dtype == MOE_BF16) {
      if (epi == EPI_SWIGLU) gemm_generic<bf16_t, EPI_SWIGLU><<<blocks, 256, 0, s>>>(g);
      else gemm_generic<bf16_t, EPI_F32><<<blocks, 256, 0, s>>>(g);
    } else {
      if (epi == EPI_SWIGLU) gemm_generic<float, EPI_SWIGLU><<<blocks, 256, 0, s>>>(g);
      else gemm_generic<float, EPI_F32><<<blocks, 256, 0, s>>>(g);
    }
    return hipGetLastError();
  }
  if (block_rows == 256) return launch_grouped_gemm_big8(epi, g, s);
  if (g.out16) return hipErrorInvalidValue;  // the 16-bit expert-output format: 256x256 kernel only
  const bool narrow = g.N <= 512;  // router-sized outputs: 64 columns per block
  if (block_rows == 64) {
    if (epi == EPI_SWIGLU) return launch_fast<EPI_SWIGLU, 4, 2, MOE_NS_SMALL>(g, s);
    return narrow ? launch_fast<EPI_F32, 4, 1, MOE_NS_SMALL>(g, s) : launch_fast<EPI_F32, 4, 2, MOE_NS_SMALL>(g, s);
  }
  if (block_rows == 32) {
    if (epi == EPI_SWIGLU) return launch_fast<EPI_SWIGLU, 2, MOE_GU_NW_SMALL, MOE_NS_SMALL>(g, s);
    return narrow ? launch_fast<EPI_F32, 2, 1, MOE_NS_SMALL>(g, s)
                  : launch_fast<EPI_F32, 2, MOE_DN_NW_SMALL, MOE_NS_SMALL>(g, s);
  }
  if (epi == EPI_SWIGLU) return launch_fast<EPI_SWIGLU, 8, 2, MOE_NS_LARGE>(g, s);
  return narrow ? launch_fast<EPI_F32, 8, 1, MOE_NS_LARGE>(g, s) : launch_fast<EPI_F32, 8, 4, MOE_NS_LARGE>(g, s);
}

}  // namespace moe
