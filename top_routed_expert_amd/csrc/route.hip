// Router selection (page "Step3.5 Flash 大模型技术深度解析", section 3.2.2,
// steps 1-2): softmax over all E routed experts' logits, then the K most
// probable experts per token. The linear layer producing the logits is a
// one-group GEMM (grouped_gemm.hip).
//
// One wavefront per token. Lane l holds experts l, l+64, ... (E <= 1024,
// so at most 16 per lane; the kernel is specialised on that count). Each of the K rounds takes the wave maximum of
// the 64-bit key (fp32 probability bits << 32 | ~expert): probabilities are
// non-negative, so their bit patterns order like the values, and on equal
// probabilities the lower expert id wins. The winner's slot is then cleared.
#include <math.h>

#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Sum of nsplit partial logit arrays for one token, one block (4 waves) per
// token: wave w adds slices w, w+4, ... in order, then the four wave sums are
// added in wave order. Result in LDS.
__device__ __forceinline__ void sum_partials(const float* __restrict__ logits, int nsplit, int64_t T, int E,
                                             int64_t t, float* s_logit, float* s_part) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t slice = T * (int64_t)E;
  for (int e = lane; e < E; e += 64) {
    float a = 0.f;
    for (int s = wave; s < nsplit; s += 4) a += logits[s * slice + t * E + e];
    s_part[wave * 1024 + e] = a;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    s_logit[e] = ((s_part[e] + s_part[1024 + e]) + s_part[2048 + e]) + s_part[3072 + e];
  __syncthreads();
}

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int nsplit, int64_t T, int E,
                                                   int K, int32_t* __restrict__ idx, float* __restrict__ prob,
                                                   float* __restrict__ gap) {
  __shared__ float s_logit[1024];
  __shared__ float s_part[4096];
  const int lane = threadIdx.x & 63;
  int64_t t;
  const float* l;
  if (nsplit > 1) {  // one token per block: the four waves add the partial sums
    t = blockIdx.x;
    sum_partials(logits, nsplit, T, E, t, s_logit, s_part);
    if (threadIdx.x >= 64) return;
    l = s_logit;
  } else {           // one token per wave
    t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave
    l = logits + t * E;
  }

  float v[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + 64 * j;
    const float x = e < E ? l[e] : -INFINITY;
    v[j] = x;
    m = fmaxf(m, x);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? expf(v[j] - m) : 0.f;
    s += v[j];
  }
  s = wave_sum(s);

  unsigned long long key[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const unsigned e = (unsigned)(lane + 64 * j);
    const float p = v[j] / s;
    key[j] = e < (unsigned)E ? ((unsigned long long)__float_as_uint(p) << 32) | (0xffffffffu - e) : 0ull;
  }

  float p_last = 0.f;
  for (int r = 0; r <= K; ++r) {
    if (r == K && K == E) break;
    unsigned long long best = key[0];
#pragma unroll
    for (int j = 1; j < VPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const unsigned e = 0xffffffffu - (unsigned)(best & 0xffffffffu);
    const float p = __uint_as_float((unsigned)(best >> 32));
    if (r == K) {
      if (gap && lane == 0) gap[t] = p_last - p;
      break;
    }
    if (lane == 0) {
      idx[t * K + r] = (int32_t)e;
      prob[t * K + r] = p;
    }
    p_last = p;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if ((unsigned)(lane + 64 * j) == e) key[j] = 0ull;
  }
  if (K == E && gap && lane == 0) gap[t] = INFINITY;
}

}  // namespace

hipError_t launch_topk(const float* logits, int nsplit, int64_t T, int E, int K, int32_t* idx, float* prob,
                       float* gap, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(nsplit > 1 ? T : (T + 3) / 4);
  const int vpl = (E + 63) / 64;
#define MOE_TOPK(V) topk_kernel<V><<<blocks, 256, 0, s>>>(logits, nsplit, T, E, K, idx, prob, gap)
  if (vpl <= 1) MOE_TOPK(1);
  else if (vpl <= 2) MOE_TOPK(2);
  else if (vpl <= 3) MOE_TOPK(3);
  else if (vpl <= 5) MOE_TOPK(5);
  else if (vpl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
