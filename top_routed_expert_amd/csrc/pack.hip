// Weight packing: row-major bf16 matrices into the packed fragment layout
// read by the MFMA kernels (layout defined in moe_internal.h). A pure data
// movement done once when weights are loaded; the layer's results are the
// same with either layout, since the kernels place the same values in the
// same operand registers.
#include "moe_internal.h"

namespace moe {

namespace {

// One thread per 16-byte lane chunk of the output: chunk i of matrix m is
// lane (i % 64) of fragment i / 64 = ct * (cols / 32) + kb.
__global__ void __launch_bounds__(256) pack_kernel(const bf16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                   int64_t chunks_per_mat, int64_t n_chunks, bf16_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int64_t m = i / chunks_per_mat, j = i - m * chunks_per_mat;
  const int lane = (int)(j & 63);
  const int64_t frag = j >> 6, kbs = cols / 32;
  const int64_t ct = frag / kbs, kb = frag - ct * kbs;
  const int64_t r = ct * 16 + (lane & 15), c = kb * 32 + (lane >> 4) * 8;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r < rows) v = *(const uint4*)(src + (m * rows + r) * cols + c);
  *(uint4*)(dst + i * 8) = v;
}

// float32 -> OCP FP8 E4M3 code: round to nearest, ties to even; magnitudes
// above 448 (and non-finite values) saturate to 448 with their sign.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a < 464.f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);  // subnormal grid m * 2^-9 (m = 8: 2^-6)
  const uint32_t ua = __float_as_uint(a);
  int e = (int)(ua >> 23) - 127;  // -6 .. 8
  uint32_t q = (ua >> 20) & 7u;
  const uint32_t rem = ua & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) {
    if (++q == 8u) {
      q = 0u;
      ++e;
    }
  }
  if (e > 8 || (e == 8 && q > 6u)) return sign | 0x7Eu;
  return sign | ((uint32_t)(e + 7) << 3) | q;
}

// Per-row FP8 quantisation (one block per padded row): scale = max|w| / 448
// (1 for a zero row), code = e4m3_rne(w / scale), written in the packed fp8
// layout (fragments of 16 rows x 64 columns, 1 KB each, ct-major; lane
// l = c + 16q of fragment (ct, kb) holds the 8 codes of row 16ct + c at
// columns 64kb + 8q .. +8, then the 8 at 64kb + 32 + 8q .. +8). Padding rows
// (past `rows` in the last 16-row group) are written as zero codes.
__global__ void __launch_bounds__(256) quant_fp8_kernel(const bf16_t* __restrict__ src, int64_t rows,
                                                        int64_t rows_pad, int cols, uint8_t* __restrict__ dst,
                                                        float* __restrict__ scales) {
  __shared__ float s_max[256];
  const int64_t R = blockIdx.x;
  const int64_t m = R / rows_pad, r = R - m * rows_pad;
  const int tid = threadIdx.x;
  const int nchunk = cols / 8;  // 8 consecutive columns per chunk
  const bool real = r < rows;
  const bf16_t* row = src + (m * rows + (real ? r : 0)) * (int64_t)cols;
  float amax = 0.f;
  if (real)
    for (int c = tid; c < cols; c += 256) amax = fmaxf(amax, fabsf(bf16_to_f32(row[c])));
  s_max[tid] = amax;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) s_max[tid] = fmaxf(s_max[tid], s_max[tid + w]);
    __syncthreads();
  }
  amax = s_max[0];
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  if (real && tid == 0) scales[m * rows + r] = scale;
  uint8_t* mat = dst + m * rows_pad * (int64_t)cols;
  const int64_t ct = r >> 4, c16 = r & 15, kbs = cols / 64;
  for (int ch = tid; ch < nchunk; ch += 256) {
    const int col0 = ch * 8, kb = col0 >> 6, kk = col0 & 63, half = kk >> 5, q4 = (kk & 31) >> 3;
    uint32_t lo = 0u, hi = 0u;
    if (real) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= e4m3_rne(bf16_to_f32(row[col0 + e]) / scale) << (8 * e);
        hi |= e4m3_rne(bf16_to_f32(row[col0 + 4 + e]) / scale) << (8 * e);
      }
    }
    *(uint2*)(mat + (ct * kbs + kb) * 1024 + (c16 + 16 * q4) * 16 + half * 8) = make_uint2(lo, hi);
  }
}

}  // namespace

hipError_t launch_quant_fp8(const bf16_t* src, int64_t n_mats, int64_t rows, int64_t cols, uint8_t* dst,
                            float* scales, hipStream_t s) {
  const int64_t rows_pad = (rows + 15) / 16 * 16;
  const int64_t n = n_mats * rows_pad;
  if (n <= 0) return hipSuccess;
  quant_fp8_kernel<<<(unsigned)n, 256, 0, s>>>(src, rows, rows_pad, (int)cols, dst, scales);
  return hipGetLastError();
}

hipError_t launch_pack(const bf16_t* src, int64_t n_mats, int64_t rows, int64_t cols, bf16_t* dst, hipStream_t s) {
  const int64_t chunks_per_mat = (rows + 15) / 16 * (cols / 32) * 64;
  const int64_t n = n_mats * chunks_per_mat;
  if (n <= 0) return hipSuccess;
  pack_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, rows, cols, chunks_per_mat, n, dst);
  return hipGetLastError();
}

}  // namespace moe
