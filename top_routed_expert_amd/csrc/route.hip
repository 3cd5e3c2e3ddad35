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

// Wave-wide reductions with DPP lane moves (no LDS round trips): pairs in a
// quad, then half-row and row mirrors give every lane of a 16-lane row the
// row's result; row_bcast:15 / row_bcast:31 fold rows 0-1 and 2-3 so lane 63
// ends with the wave's result, which readlane broadcasts.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xf, false);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp32<0xb1, 0xf>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp32<0x4e, 0xf>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp32<0x141, 0xf>(v));  // row_half_mirror
  v = op(v, dpp32<0x140, 0xf>(v));  // row_mirror
  v = op(v, dpp32<0x142, 0xa>(v));  // row_bcast:15 into rows 1 and 3
  v = op(v, dpp32<0x143, 0xc>(v));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
  const uint32_t lo = dpp32<CTRL, ROW_MASK>((uint32_t)v), hi = dpp32<CTRL, ROW_MASK>((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long max64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  v = max64(v, dpp64<0xb1, 0xf>(v));
  v = max64(v, dpp64<0x4e, 0xf>(v));
  v = max64(v, dpp64<0x141, 0xf>(v));
  v = max64(v, dpp64<0x140, 0xf>(v));
  v = max64(v, dpp64<0x142, 0xa>(v));
  v = max64(v, dpp64<0x143, 0xc>(v));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
}

// Sum of nsplit partial logit arrays for one token, one block (4 waves) per
// token: wave w adds slices w, w+4, ... in order, then the four wave sums are
// added in wave order. Result in LDS. All of a lane's loads for four slices
// are issued before the first add, so the chain of dependent loads is short.
template <int VPL>
__device__ __forceinline__ void sum_partials(const float* __restrict__ logits, int nsplit, int64_t T, int E,
                                             int64_t t, float* s_logit, float* s_part) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t slice = T * (int64_t)E;
  float part[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) part[j] = 0.f;
  const float* base = logits + t * E + lane;
  for (int s0 = wave; s0 < nsplit; s0 += 16) {
    float v[4][VPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + 4 * u;
#pragma unroll
      for (int j = 0; j < VPL; ++j) v[u][j] = (s < nsplit && lane + 64 * j < E) ? base[s * slice + 64 * j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        if (s0 + 4 * u < nsplit) part[j] += v[u][j];
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if (lane + 64 * j < E) s_part[wave * 1024 + lane + 64 * j] = part[j];
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    s_logit[e] = ((s_part[e] + s_part[1024 + e]) + s_part[2048 + e]) + s_part[3072 + e];
  __syncthreads();
}

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int nsplit, int64_t T, int E,
                                                   int K, const int32_t* __restrict__ k_tok,
                                                   int32_t* __restrict__ idx, float* __restrict__ prob,
                                                   float* __restrict__ gap, float* __restrict__ gmass, int G) {
  __shared__ float s_logit[1024];
  __shared__ float s_part[4096];
  const int lane = threadIdx.x & 63;
  int64_t t;
  const float* l;
  if (nsplit > 4) {  // one token per block: the four waves add the partial sums
    t = blockIdx.x;
    sum_partials<VPL>(logits, nsplit, T, E, t, s_logit, s_part);
    if (threadIdx.x >= 64) return;
    l = s_logit;
  } else {           // one token per wave, adding up to four partial sums itself
    t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave
    l = logits + t * E;
  }
  // partial sums this wave adds, in slice order: ((p0 + p1) + p2) + p3
  const int nadd = nsplit > 4 ? 1 : nsplit;
  const int64_t slice = T * (int64_t)E;

  float v[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = lane + 64 * j;
    float x = -INFINITY;
    if (e < E) {
      x = l[e];
      if (nadd > 1) {
        const float x1 = l[slice + e];
        const float x2 = nadd > 2 ? l[2 * slice + e] : 0.f;
        const float x3 = nadd > 3 ? l[3 * slice + e] : 0.f;
        x = ((x + x1) + x2) + x3;
      }
    }
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

  // optional: the token's routing probability mass per expert group (G
  // equal contiguous groups), for the expert-parallel balance statistics
  if (gmass) {
    const int gs = E / G;
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int e = lane + 64 * j;
        if (e < E && e / gs == g) a += v[j] / s;
      }
      a = wave_sum(a);
      if (lane == 0) gmass[t * G + g] = a;
    }
  }

  unsigned long long key[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const unsigned e = (unsigned)(lane + 64 * j);
    const float p = v[j] / s;
    key[j] = e < (unsigned)E ? ((unsigned long long)__float_as_uint(p) << 32) | (0xffffffffu - e) : 0ull;
  }

  // this token's number of experts: K, or k_tok[t] clamped to [0, K]
  int kt = K;
  if (k_tok) {
    kt = k_tok[t];
    kt = kt < 0 ? 0 : (kt > K ? K : kt);
  }
  float p_last = 0.f;
  for (int r = 0; r <= kt; ++r) {
    if (r == kt && (kt == E || !gap)) break;  // round kt only finds the gap
    unsigned long long best = key[0];
#pragma unroll
    for (int j = 1; j < VPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const unsigned e = 0xffffffffu - (unsigned)(best & 0xffffffffu);
    const float p = __uint_as_float((unsigned)(best >> 32));
    if (r == kt) {
      if (gap && lane == 0) gap[t] = kt > 0 ? p_last - p : INFINITY;
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
  if (kt == E && gap && lane == 0) gap[t] = INFINITY;
  // slots past the token's own count: no expert
  if (lane == 0)
    for (int r = kt; r < K; ++r) {
      idx[t * K + r] = -1;
      prob[t * K + r] = 0.f;
    }
}

// Expert-parallel balance statistics (page "Step3.5 Flash 大模型技术深度解析",
// section 3.2.3: 288 experts in G groups, one group per GPU; the balance
// loss L_EP = G * sum_g f_g p_g): out[g] = sum_t p_g(t) (the group's
// probability mass gmass[t][g]) and out[G + g] = #{(t, k): idx[t,k] in group
// g}, in fp64. Two passes, each in a fixed order, so the sums do not depend
// on scheduling: block (b, g) of the first sums tokens b*GS_CHUNK ..
// (b+1)*GS_CHUNK - 1 (thread i takes tokens i, i+256, ..., then a
// fixed-shape tree) into part[g][b]; block g of the second sums part[g][0 ..
// nb-1] the same way (nb = 0: zeros).
constexpr int GS_CHUNK = 1024;

__device__ __forceinline__ void block_sum2(double& m, double& c, double* s_m, double* s_c) {
  const int tid = threadIdx.x;
  s_m[tid] = m;
  s_c[tid] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      s_m[tid] += s_m[tid + w];
      s_c[tid] += s_c[tid + w];
    }
    __syncthreads();
  }
  m = s_m[0];
  c = s_c[0];
}

__global__ void __launch_bounds__(256) group_partials_kernel(const float* __restrict__ gmass,
                                                             const int32_t* __restrict__ idx, int64_t T, int K,
                                                             int E, int G, double* __restrict__ part, int nb) {
  __shared__ double s_m[256], s_c[256];
  const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x, gs = E / G;
  const int64_t t0 = (int64_t)b * GS_CHUNK, t1 = t0 + GS_CHUNK < T ? t0 + GS_CHUNK : T;
  double m = 0.0, c = 0.0;
  for (int64_t t = t0 + tid; t < t1; t += 256) {
    m += (double)gmass[t * G + g];
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      c += (e >= 0 && e < E && e / gs == g) ? 1.0 : 0.0;
    }
  }
  block_sum2(m, c, s_m, s_c);
  if (tid == 0) {
    part[(int64_t)g * nb + b] = m;
    part[(int64_t)(G + g) * nb + b] = c;
  }
}

__global__ void __launch_bounds__(256) group_stats_kernel(const double* __restrict__ part, int nb, int G,
                                                          double* __restrict__ out) {
  __shared__ double s_m[256], s_c[256];
  const int g = blockIdx.x, tid = threadIdx.x;
  double m = 0.0, c = 0.0;
  for (int b = tid; b < nb; b += 256) {
    m += part[(int64_t)g * nb + b];
    c += part[(int64_t)(G + g) * nb + b];
  }
  block_sum2(m, c, s_m, s_c);
  if (tid == 0) {
    out[g] = m;
    out[G + g] = c;
  }
}

}  // namespace

int64_t group_stats_partials(int64_t T, int G) { return (T + GS_CHUNK - 1) / GS_CHUNK * 2 * G; }

hipError_t launch_group_stats(const float* gmass, const int32_t* idx, int64_t T, int K, int E, int G, double* part,
                              double* out, hipStream_t s) {
  const int64_t nb = (T + GS_CHUNK - 1) / GS_CHUNK;
  if (nb > 0) {
    const dim3 grid((unsigned)nb, (unsigned)G);
    group_partials_kernel<<<grid, 256, 0, s>>>(gmass, idx, T, K, E, G, part, (int)nb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  group_stats_kernel<<<G, 256, 0, s>>>(part, (int)nb, G, out);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int nsplit, int64_t T, int E, int K, const int32_t* k_tok, int32_t* idx,
                       float* prob, float* gap, float* gmass, int G, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(nsplit > 4 ? T : (T + 3) / 4);
  const int vpl = (E + 63) / 64;
#define MOE_TOPK(V) \
  topk_kernel<V><<<blocks, 256, 0, s>>>(logits, nsplit, T, E, K, k_tok, idx, prob, gap, gmass, G)
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
