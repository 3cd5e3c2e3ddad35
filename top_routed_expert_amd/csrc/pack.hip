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

}  // namespace

hipError_t launch_pack(const bf16_t* src, int64_t n_mats, int64_t rows, int64_t cols, bf16_t* dst, hipStream_t s) {
  const int64_t chunks_per_mat = (rows + 15) / 16 * (cols / 32) * 64;
  const int64_t n = n_mats * chunks_per_mat;
  if (n <= 0) return hipSuccess;
  pack_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, rows, cols, chunks_per_mat, n, dst);
  return hipGetLastError();
}

}  // namespace moe
