// Weighted combine (page "Step3.5 Flash 大模型技术深度解析", section 3.2.2,
// step 3): the outputs of a token's K routed experts, weighted by their
// router probabilities, are added to the shared expert's output:
//   out[t] = y_shared[t] + sum_{k=0..K-1} prob[t,k] * y_perm[dest[t*K+k]]
// in fp32, in that order, with one final rounding to the output type.
// One block per (token, 1024-column chunk); the K source rows are read with
// 16-byte loads.
#include "moe_internal.h"

namespace moe {

namespace {

template <typename TO>
__device__ __forceinline__ void store4(TO* p, float4 v) {
  store_out(p, v.x);
  store_out(p + 1, v.y);
  store_out(p + 2, v.z);
  store_out(p + 3, v.w);
}

template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *(float4*)p = v;
}

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
  *(uint2*)p = make_uint2(lo, hi);
}

// The expert outputs are read once: non-temporal loads keep them from
// displacing anything in L2 (measured 50 us less per prefill step).
__device__ __forceinline__ float4 load_stream4(const float* p) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}

template <typename TO>
__global__ void __launch_bounds__(256) combine_kernel(int D, int K, const float* __restrict__ y_perm, int64_t n_perm,
                                                      const int32_t* __restrict__ dest, const float* __restrict__ prob,
                                                      const float* __restrict__ y_shared, TO* __restrict__ out) {
  __shared__ int64_t s_row[64];
  __shared__ float s_p[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int c0 = (int)blockIdx.y * 1024;  // this block's column chunk
  const int c1 = D < c0 + 1024 ? D : c0 + 1024;
  if (tid < K) {
    const int64_t d = dest[t * K + tid];
    s_row[tid] = (d >= 0 && d < n_perm) ? d : -1;
    s_p[tid] = prob[t * K + tid];
  }
  __syncthreads();
  if ((D & 3) == 0) {
    for (int c = c0 + tid * 4; c < c1; c += 1024) {
      float4 acc = y_shared ? *(const float4*)(y_shared + t * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      // eight rows per batch, all loads issued before the first add (a
      // skipped pair reads row 0 and is not added); adds stay in k order
      for (int k0 = 0; k0 < K; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + u;
          const int64_t r = (k < K && s_row[k] >= 0) ? s_row[k] : 0;
          v[u] = load_stream4(y_perm + r * D + c);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + u;
          if (k < K && s_row[k] >= 0) {
            const float w = s_p[k];
            acc.x = fmaf(w, v[u].x, acc.x);
            acc.y = fmaf(w, v[u].y, acc.y);
            acc.z = fmaf(w, v[u].z, acc.z);
            acc.w = fmaf(w, v[u].w, acc.w);
          }
        }
      }
      store4(out + t * D + c, acc);
    }
  } else {
    for (int c = c0 + tid; c < c1; c += 256) {
      float acc = y_shared ? y_shared[t * D + c] : 0.f;
      for (int k = 0; k < K; ++k)
        if (s_row[k] >= 0) acc = fmaf(s_p[k], y_perm[s_row[k] * D + c], acc);
      store_out(out + t * D + c, acc);
    }
  }
}

// The routed rows in the 16-bit expert-output format (moe_internal.h): each
// thread takes 8 consecutive columns, which lie in one 64-column chunk of
// every row; chunk exponent e turns the routing weight into
// w = p * 2^(e - EXP16_BIAS), an exact scaling, so w * q = p * y up to the
// fp16 rounding of y. The shared expert's row stays fp32. Sums run in k order
// in fp32 with one final rounding, as above.
template <typename TO>
__global__ void __launch_bounds__(256) combine16_kernel(int D, int K, const uint16_t* __restrict__ y16,
                                                        const uint8_t* __restrict__ y16_exp, int64_t n_perm,
                                                        const int32_t* __restrict__ dest,
                                                        const float* __restrict__ prob,
                                                        const float* __restrict__ y_shared, TO* __restrict__ out) {
  __shared__ int64_t s_row[64];
  __shared__ float s_p[64];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int c0 = (int)blockIdx.y * 2048;  // this block's column chunk
  const int c1 = D < c0 + 2048 ? D : c0 + 2048;
  const int nch = D >> 6;  // exponent chunks per row
  if (tid < K) {
    const int64_t d = dest[t * K + tid];
    s_row[tid] = (d >= 0 && d < n_perm) ? d : -1;
    s_p[tid] = prob[t * K + tid];
  }
  __syncthreads();
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  for (int c = c0 + tid * 8; c < c1; c += 2048) {
    float acc[8];
    if (y_shared) {
      const float4 a = *(const float4*)(y_shared + t * D + c);
      const float4 b = *(const float4*)(y_shared + t * D + c + 4);
      acc[0] = a.x, acc[1] = a.y, acc[2] = a.z, acc[3] = a.w, acc[4] = b.x, acc[5] = b.y, acc[6] = b.z, acc[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int k0 = 0; k0 < K; k0 += 8) {
      u32x4_t q[8];
      int ex[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // all loads of the batch before the first add
        const int k = k0 + u;
        const int64_t r = (k < K && s_row[k] >= 0) ? s_row[k] : 0;
        q[u] = __builtin_nontemporal_load((const u32x4_t*)(y16 + r * D + c));
        ex[u] = y16_exp[r * nch + (c >> 6)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        if (k < K && s_row[k] >= 0) {
          const float w = ldexpf(s_p[k], ex[u] - EXP16_BIAS);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t bits = q[u][i];
            acc[2 * i] = fmaf(w, (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu)), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, (float)__builtin_bit_cast(_Float16, (uint16_t)(bits >> 16)), acc[2 * i + 1]);
          }
        }
      }
    }
    store4(out + t * D + c, make_float4(acc[0], acc[1], acc[2], acc[3]));
    store4(out + t * D + c + 4, make_float4(acc[4], acc[5], acc[6], acc[7]));
  }
}

}  // namespace

hipError_t launch_combine16(int out_dtype, int64_t T, int D, int K, const uint16_t* y16, const uint8_t* y16_exp,
                            int64_t n_perm_rows, const int32_t* dest, const float* prob, const float* y_shared,
                            void* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (D % 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)T, (unsigned)((D + 2047) / 2048));
  if (out_dtype == MOE_BF16)
    combine16_kernel<bf16_t><<<grid, 256, 0, s>>>(D, K, y16, y16_exp, n_perm_rows, dest, prob, y_shared,
                                                  (bf16_t*)out);
  else
    combine16_kernel<float><<<grid, 256, 0, s>>>(D, K, y16, y16_exp, n_perm_rows, dest, prob, y_shared,
                                                 (float*)out);
  return hipGetLastError();
}

hipError_t launch_combine(int out_dtype, int64_t T, int D, int K, const float* y_perm, int64_t n_perm_rows,
                          const int32_t* dest, const float* prob, const float* y_shared, void* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)T, (unsigned)((D + 1023) / 1024));
  if (out_dtype == MOE_BF16)
    combine_kernel<bf16_t><<<grid, 256, 0, s>>>(D, K, y_perm, n_perm_rows, dest, prob, y_shared, (bf16_t*)out);
  else
    combine_kernel<float><<<grid, 256, 0, s>>>(D, K, y_perm, n_perm_rows, dest, prob, y_shared, (float*)out);
  return hipGetLastError();
}

}  // namespace moe
