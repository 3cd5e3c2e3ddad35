// Internal declarations shared by the HIP translation units of libmoe.
// Nothing here is part of the C ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe.h"

// Size of the static device scratch of moe_layer_forward_noalloc (64 MiB).
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

namespace moe {

typedef uint16_t bf16_t;  // storage type of bfloat16 values
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even; NaN stays NaN (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ float load_f32(const float* p) { return *p; }
__device__ __forceinline__ float load_f32(const bf16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// g * sigmoid(g) with the hardware reciprocal (1 ulp): the result is rounded to
// bf16 (8 significant bits) before anything reads it, or compared at 1e-4 of
// the RMS in fp32 layers, far above that error.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// f(std::integral_constant<int, I>{}) for I = B .. E-1: indices into register
// arrays are constant expressions, so the arrays never need memory.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// One row segment of a grouped GEMM: rows [row0, row1) of group `group`.
// first/count: the group's tiles are first .. first+count-1 (consecutive).
struct Tile {
  int32_t group, row0, row1, first;
  int32_t count, pad0, pad1, pad2;
};

// Packed FP8 layout of W [N, K] (K % 64 == 0), E4M3 codes: fragments of 16
// rows x 64 columns (1 KB), ct-major then kb; lane l = c + 16q of fragment
// (ct, kb) holds, at byte 16l, the codes of row 16ct + c at columns
// 64kb + 8q .. +8 and then 64kb + 32 + 8q .. +8: the two 32-column halves
// are the lane's operands of two consecutive MFMA steps.
constexpr int FP8_FRAG = 1024;  // bytes per fp8 fragment
__host__ __device__ __forceinline__ int64_t fp8_offset(int64_t ct, int64_t kb, int lane, int64_t K) {
  return (ct * (K / 64) + kb) * FP8_FRAG + lane * 16;
}

// Packed fragment layout of a bf16 weight matrix W [N, K] (K % 32 == 0):
// W is cut into 16-row x 32-column fragments, fragment (ct, kb) covering rows
// 16ct.. and columns 32kb.. . Each fragment is 1 KB stored in MFMA operand
// order: lane l = c + 16q (c < 16, q < 4) holds W[16ct + c][32kb + 8q .. +8]
// at byte 16l. Fragments are stored kb-fastest; rows past N are zero.
// Element offset of lane l's 8 values of fragment (ct, kb):
constexpr int PACKED_FRAG = 512;  // bf16 elements per fragment
__host__ __device__ __forceinline__ int64_t packed_offset(int64_t ct, int64_t kb, int lane, int64_t K) {
  return (ct * (K / 32) + kb) * PACKED_FRAG + lane * 8;
}

// FP8 E4M3 -> bf16, exactly (an E4M3 value has at most 4 significant bits
// and its exponent range lies inside bf16's): one gfx950 scaled conversion of
// two codes (OCP E4M3) with scale 1, giving the two bf16 values packed. HI
// selects bytes 2-3 of w instead of 0-1. (Through fp32 with the unscaled
// conversion and keeping the upper halves gives the same bits for all 65536
// code pairs, at three instructions instead of one.)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// 8 codes (lo: the first 4, hi: the next 4) -> one bf16x8 MFMA operand
__device__ __forceinline__ uint4 fp8x8_bf16x8(uint32_t lo, uint32_t hi) {
  return make_uint4(fp8x2_bf16x2<false>(lo), fp8x2_bf16x2<true>(lo), fp8x2_bf16x2<false>(hi),
                    fp8x2_bf16x2<true>(hi));
}

// Epilogues of the grouped GEMM.
enum GemmEpilogue {
  EPI_SWIGLU = 0,  // two B operands (gate, up): out = dtype(silu(A Bg^T) * (A Bu^T))
  EPI_F32 = 1      // one B operand: out = fp32(A B^T + bias)
};

// Arguments of one grouped GEMM launch: out[r, n] for rows r of each tile and
// columns n < N, contracting over Kdim.
struct GemmArgs {
  const void* a;          // A rows: [n_a_rows, Kdim] (row r of the problem reads row map(r))
  int64_t n_a_rows;
  const int32_t* gather;  // map(r) = gather[r] for r < n_gather, else r - n_gather
  int64_t n_gather;
  const void* b0;         // B of group g < n_main: b0 + g*b_stride; group n_main: b0_extra
  const void* b1;         // second B operand (EPI_SWIGLU only), same indexing
  const void* b0_extra;
  const void* b1_extra;
  int64_t b_stride;       // elements between consecutive groups' B matrices ([N, Kdim])
  int32_t n_main;
  int32_t N;
  int32_t Kdim;
  const Tile* tiles;      // schedule built on the device, or NULL: one group (group 0)
  const int32_t* n_tiles; //   of dense_rows rows cut into consecutive row tiles
  int64_t dense_rows;
  int32_t max_tiles;      // host-side upper bound of the tile count (grid size)
  void* out;              // [rows, ldo]
  int64_t ldo;
  int32_t b_packed;       // B operands in the packed fragment layout (bf16 MFMA kernels only)
  int32_t b_fp8;          // B operands are FP8 E4M3 codes in the packed fp8 layout (b_stride in bytes),
  const float* s0;        //   with per-column scales: group g < n_main: s0 + g*s_stride, else s0_extra
  const float* s1;        //   (second B operand: s1 / s1_extra)
  const float* s0_extra;
  const float* s1_extra;
  int64_t s_stride;
  int32_t b_reuse;        // B is read again by many row tiles (router): keep it cacheable
  const float* bias;      // EPI_F32: per-column bias or NULL
  int32_t ksplit;         // EPI_F32 only: the contraction is cut into ksplit slices;
  int64_t slice_stride;   //   slice s writes its partial sums to out + s*slice_stride
  // EPI_F32, 256x256 kernel only (out16 != NULL): rows r < out16_rows are stored as fp16 in
  // out16 [out16_rows, ldo] with one exponent byte per 64 columns in out16_exp
  // [out16_rows, ldo/64] (the 16-bit expert-output format, below); rows r >= out16_rows go to
  // `out` (fp32) at row r - out16_rows. Needs N % 64 == 0 and ldo == N.
  uint16_t* out16;
  uint8_t* out16_exp;
  int64_t out16_rows;
};

// 16-bit expert-output format. A row's 64-column chunk c holds fp16 values
// q = fp16_rne(y * 2^(141 - e)) and one byte e = max(14, biased fp32 exponent of
// max |y| over the chunk), so the chunk's largest magnitude lands in [2^14, 2^15)
// and no value overflows fp16; y = q * 2^(e - 141) up to fp16 rounding (2^-11
// relative). EXP16_BIAS is that 141.
constexpr int EXP16_BIAS = 141;
constexpr int EXP16_MIN = 14;

// Per-column scales of group g (fp8 weights).
__device__ __forceinline__ const float* group_scale(const GemmArgs& p, const float* main, const float* extra, int g) {
  return g < p.n_main ? main + (int64_t)g * p.s_stride : extra;
}

// Launchers (grouped_gemm.hip). `dtype` is MOE_BF16 or MOE_F32 for A/B; the
// SwiGLU output has the same dtype; EPI_F32 output is fp32.
// Row-tile height on the bf16 MFMA path (`fast`): 32, 64, 128 or (expert
// GEMMs with many rows per group, `allow_big`) 256; 64 on the generic path.
int gemm_block_rows(bool fast, int64_t rows, int n_groups, bool allow_big);
// Contraction slices of the router GEMM for T tokens and E experts (1 on the
// generic path and when the row tiles alone fill the chip).
int router_ksplit(bool fast, int64_t T, int Kdim, int E);
int64_t gemm_max_tiles(int64_t n_rows, int n_groups, int block_rows);
// Tiles of groups g = 0 .. n_groups-1 over rows [offsets[g], offsets[g+1]);
// group skip_group (if >= 0) gets none.
hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int64_t n_rows, int block_rows,
                              Tile* tiles, int32_t* n_tiles, int32_t max_tiles, int skip_group, hipStream_t s);
hipError_t launch_grouped_gemm(int dtype, bool fast, int epi, int block_rows, const GemmArgs& g, hipStream_t s);
// 256 x 256 block tiles (block_rows == 256): grouped_gemm_big8.hip (eight
// waves, bf16 or fp8 weights).
hipError_t launch_grouped_gemm_big8(int epi, const GemmArgs& g, hipStream_t s);

// router.hip: linear layer, softmax and top-K in one kernel, 32 tokens per
// block (bf16, router row-major or packed with the same results,
// 6144 < T <= 12288, E <= 320, d_model a multiple of 64 and at least 128); k_tok, gap and gmass
// as launch_topk.
bool router_topk_fits(int64_t T, int D, int E, int K);
hipError_t launch_router_topk(const bf16_t* x, int64_t T, int D, const bf16_t* w_router, bool packed,
                              const float* bias, int E, int K, const int32_t* k_tok, int32_t* idx, float* prob,
                              float* gap, float* gmass, int G, hipStream_t s);

// route.hip
// Logits are the sum of nsplit partial arrays [nsplit][T][E], added in slice order.
// k_tok (optional): token t keeps its first k_tok[t] (clamped to [0, K])
// choices; later slots get idx -1 and prob 0.
// gmass (optional): [T][G] routing probability mass of each of G equal
// contiguous expert groups (E % G == 0, G <= 16).
hipError_t launch_topk(const float* logits, int nsplit, int64_t T, int E, int K, const int32_t* k_tok, int32_t* idx,
                       float* prob, float* gap, float* gmass, int G, hipStream_t s);
// out [2G] fp64: per-group probability mass summed over tokens, then the
// number of chosen pairs per group; part: group_stats_partials(T, G) fp64
// values of scratch (per-chunk partial sums).
int64_t group_stats_partials(int64_t T, int G);
hipError_t launch_group_stats(const float* gmass, const int32_t* idx, int64_t T, int K, int E, int G, double* part,
                              double* out, hipStream_t s);

// permute.hip. Pairs with idx outside [0, E) get dest -1 and no row.
// offsets_ext [E+3] (optional), the row groups of the fused expert launch:
// the E routed segments (ending at the valid pair count V), then [V, T*K)
// (rows of pairs without an expert: no tiles), then the extra_rows rows
// from T*K on (the shared expert).
// tiles (optional): also the expert GEMMs' tile table over the groups of
// offsets_ext, as launch_permute_small writes it (E <= 1023).
hipError_t launch_permute(const int32_t* idx, int64_t T, int K, int E, int32_t* rank, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_token, int32_t* dest,
                          int32_t* offsets_ext, int32_t extra_rows, Tile* tiles, int32_t* n_tiles,
                          int32_t max_tiles, int block_rows, hipStream_t s);
bool permute_small_fits(int64_t T, int K, int E);
// Single-block permutation for small batches; also writes the tile table of
// the expert GEMMs over the groups of offsets_ext (E, or E+2 with
// extra_rows) when tiles != NULL.
hipError_t launch_permute_small(const int32_t* idx, int64_t T, int K, int E, int32_t* offsets, int32_t* sorted_token,
                                int32_t* dest, int32_t* offsets_ext, int32_t extra_rows, Tile* tiles,
                                int32_t* n_tiles, int32_t max_tiles, int block_rows, hipStream_t s);
hipError_t launch_gather_rows(const void* x, int64_t T, int D, int elem_bytes, const int32_t* sorted_token,
                              int64_t rows, void* x_perm, hipStream_t s);
// Expert-parallel receive plan (see moe_ep_receive_plan in include/moe.h).
hipError_t launch_ep_plan(const int32_t* counts, int n_src, int n_local, int64_t max_rows, int32_t* offsets,
                          int32_t* gather, int32_t* scatter, hipStream_t s);

// pack.hip: n_mats row-major [rows, cols] bf16 matrices -> packed fragment
// layout (rows rounded up to a multiple of 16, zero-filled), matrix after
// matrix.
hipError_t launch_pack(const bf16_t* src, int64_t n_mats, int64_t rows, int64_t cols, bf16_t* dst, hipStream_t s);
// pack.hip: per-row FP8 quantisation of n_mats row-major [rows, cols] bf16
// matrices (cols % 64 == 0) into the packed fp8 layout (rows rounded up to
// 16, zero codes) and scales [n_mats, rows].
hipError_t launch_quant_fp8(const bf16_t* src, int64_t n_mats, int64_t rows, int64_t cols, uint8_t* dst,
                            float* scales, hipStream_t s);

// combine.hip
hipError_t launch_combine(int out_dtype, int64_t T, int D, int K, const float* y_perm, int64_t n_perm_rows,
                          const int32_t* dest, const float* prob, const float* y_shared, void* out,
                          hipStream_t s);
// The same combine with the routed rows in the 16-bit expert-output format (D % 64 == 0).
hipError_t launch_combine16(int out_dtype, int64_t T, int D, int K, const uint16_t* y16, const uint8_t* y16_exp,
                            int64_t n_perm_rows, const int32_t* dest, const float* prob, const float* y_shared,
                            void* out, hipStream_t s);

}  // namespace moe
