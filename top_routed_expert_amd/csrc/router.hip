// Router of many tokens in one kernel (page "Step3.5 Flash 大模型技术深度解析",
// section 3.2.2, steps 1-2): the linear layer, the softmax over all E routed
// experts and the choice of the K most probable, for 32 tokens per block and
// every expert at once, so the logits never leave the compute unit.
//
// Linear layer: bf16 MFMA 16x16x32 with fp32 accumulation. A block owns 32
// tokens (two 16-row tiles) and all column tiles of 16 experts (up to 20, so
// E <= 320); wave w of four holds column tiles 5w .. 5w+4 for both row tiles
// (40 accumulators per lane). Both operands move HBM/L2 -> LDS through direct
// loads (global_load_lds, 16 bytes per lane) in stages of 64 contraction
// elements through a ring of three 44 KB slots: the token rows (32 x 128
// bytes, chunk q of row r at q ^ ((r >> 1) & 7) so the operand reads are
// conflict-free) and the router's fragments (1 KB each, 40 per stage): copied
// as they are from the packed layout, or gathered lane by lane into the same
// fragment order from row-major weights, so both layouts give the same bits. Per stage every wave issues exactly 11 loads, waits
// for its own loads of the stage with s_waitcnt vmcnt (loads complete in
// order) and then one barrier makes every wave's loads visible and ends the
// reads of the slot about to be refilled. Stages past the end re-load the
// last stage into a slot nobody reads again, so the wait counts are fixed.
// Each router weight byte is read by every block (from L2); a block's time is
// set by that stream, so blocks of 32 tokens keep all compute units busy.
// Blocks start their walk over the contraction at different stages (block b
// of an XCD at stage 2b mod the stage count, wrapping around): a stage's 40
// fragments lie in a few L2 channels, and blocks in lockstep on the same stage
// would all queue on them. The summation order differs from block to block;
// it is fixed for a block, so the results are deterministic.
//
// Selection: the 32 x E logits (plus bias) go to LDS; each token is handled
// by 16 lanes (one DPP row), lane j holding experts j, j+16, ... Row maxima
// and sums take four lane moves (quad permutes, half-row and row mirrors),
// which leave the same value in all 16 lanes. Each of the K rounds takes the
// row maximum of the 64-bit key (fp32 probability bits << 32 | ~expert):
// probabilities are non-negative, so their bits order like the values, and on
// equal probabilities the lower expert id wins; the winner's key is cleared.
#include <math.h>

#include "moe_internal.h"

// The operand-read lambdas capture their asm operands explicitly (clang's
// device pass does not capture names used only as asm operands); the host
// pass, which does not see the asm's use, would warn about those captures.
#pragma clang diagnostic ignored "-Wunused-lambda-capture"

namespace moe {

namespace {

constexpr int RT_ROWS = 32;                         // tokens per block
constexpr int RT_KS = 64;                           // contraction elements per stage
constexpr int RT_NS = 3;                            // slots in the ring
constexpr int RT_CTW = 5;                           // 16-expert column tiles per wave
constexpr int RT_NCT = 4 * RT_CTW;                  // column tiles per block (E <= 320)
constexpr int RT_VPL = RT_NCT;                      // experts per lane in the selection (16 lanes per token)
constexpr int RT_A_BYTES = RT_ROWS * RT_KS * 2;     // 4 KB of token rows per stage
constexpr int RT_B_BYTES = RT_NCT * 2 * 1024;       // 40 fragments of 1 KB per stage
constexpr int RT_STAGE = RT_A_BYTES + RT_B_BYTES;   // 44 KB
constexpr int RT_LOADS = 1 + 2 * RT_CTW;            // direct loads per wave per stage
constexpr int RT_LS = RT_NCT * 16 + 4;              // logit row stride in the epilogue (floats)

typedef __attribute__((address_space(3))) void lds_rt_t;
typedef uint32_t u32x4_rt __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8_rt(u32x4_rt v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ int swz_rt(int row) { return (row >> 1) & 7; }
constexpr int waitcnt_vm_rt(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

// one DPP lane move of a 32-bit value (CTRL: quad_perm / row mirrors)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_rt(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xf, 0xf, false);
}
// Reductions over the 16 lanes of a DPP row; every lane of the row ends with the result.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __uint_as_float(dpp_rt<0xb1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_rt<0x4e>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_rt<0x141>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_rt<0x140>(__float_as_uint(v))));
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += __uint_as_float(dpp_rt<0xb1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_rt<0x4e>(__float_as_uint(v)));
  v += __uint_as_float(dpp_rt<0x141>(__float_as_uint(v)));
  v += __uint_as_float(dpp_rt<0x140>(__float_as_uint(v)));
  return v;
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64_rt(unsigned long long v) {
  const uint32_t lo = dpp_rt<CTRL>((uint32_t)v), hi = dpp_rt<CTRL>((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long max64_rt(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long row_max16_u64(unsigned long long v) {
  v = max64_rt(v, dpp64_rt<0xb1>(v));
  v = max64_rt(v, dpp64_rt<0x4e>(v));
  v = max64_rt(v, dpp64_rt<0x141>(v));
  v = max64_rt(v, dpp64_rt<0x140>(v));
  return v;
}

template <bool PK>
__global__ void __launch_bounds__(256) router_topk_kernel(const bf16_t* __restrict__ x, int64_t T, int D,
                                                          const bf16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int E, int K,
                                                          const int32_t* __restrict__ k_tok,
                                                          int32_t* __restrict__ idx, float* __restrict__ prob,
                                                          float* __restrict__ gap, float* __restrict__ gmass,
                                                          int G) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[RT_NS * RT_STAGE];  // the epilogue's logits reuse it
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * RT_ROWS;
  const int nst = D / RT_KS;
  const int ct_last = (E + 15) / 16 - 1;
  const int rot = (int)((blockIdx.x >> 3) * 2u % (unsigned)nst);  // first stage of this block's walk

  // direct-load sources: token rows wave*8 + lane/8 (rows past T read row T-1,
  // never stored), physical chunk lane%8 = logical chunk (lane%8) ^ swz(row);
  // router fragments f = wave*10 + i: column tile f/2 (tiles past E clamped,
  // never stored), contraction half f%2 of the stage; lane l = c + 16q of a
  // fragment holds expert 16*tile + c, contraction elements 32*half + 8q .. +7
  // (row-major: experts past E read expert E-1, never stored)
  const int arow = wave * 8 + (lane >> 3);
  const int64_t asrc_row = row0 + arow < T ? row0 + arow : T - 1;
  const bf16_t* asrc = x + asrc_row * D + (((lane & 7) ^ swz_rt(arow)) << 3);
  const bf16_t* bsrc[2 * RT_CTW];
#pragma unroll
  for (int i = 0; i < 2 * RT_CTW; ++i) {
    const int f = wave * 2 * RT_CTW + i;
    const int ct = (f >> 1) < ct_last ? (f >> 1) : ct_last;
    if constexpr (PK) {
      bsrc[i] = wr + packed_offset(ct, f & 1, lane, D);
    } else {
      const int e = ct * 16 + (lane & 15) < E ? ct * 16 + (lane & 15) : E - 1;
      bsrc[i] = wr + (int64_t)e * D + (f & 1) * 32 + (lane >> 4) * 8;
    }
  }
  auto issue = [&](int step, int slot) {  // step-th stage of the walk
    const int stage = step + rot < nst ? step + rot : step + rot - nst;
    uint8_t* base = lds + slot * RT_STAGE;
    __builtin_amdgcn_global_load_lds((const void*)(asrc + stage * RT_KS), (lds_rt_t*)(base + wave * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < 2 * RT_CTW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(bsrc[i] + stage * (PK ? 2 * PACKED_FRAG : RT_KS)),
                                       (lds_rt_t*)(base + RT_A_BYTES + (wave * 2 * RT_CTW + i) * 1024), 16, 0, 0);
  };

  // operand reads: lane (r = lane & 15, q = lane >> 4); row tile 1 at +2048,
  // column tile j of contraction half h at fragment (5*wave + j)*2 + h
  const int rq = lane >> 4, rr = lane & 15;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_rt_t*)&lds[0];
  const uint32_t aoff0 = (uint32_t)(rr * 128 + ((rq ^ swz_rt(rr)) << 4));
  const uint32_t aoff1 = (uint32_t)(rr * 128 + (((rq + 4) ^ swz_rt(rr)) << 4));
  const uint32_t boff = (uint32_t)RT_A_BYTES + (uint32_t)(wave * RT_CTW * 2) * 1024u + (uint32_t)lane * 16u;
  f32x4 acc[2][RT_CTW];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < RT_CTW; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int slot) {
    const uint32_t sb = lds_base + (uint32_t)slot * RT_STAGE;
    const uint32_t a0 = sb + aoff0, a1 = sb + aoff1, bb = sb + boff;
    u32x4_rt A0[2], A1[2], B0[RT_CTW], B1[RT_CTW];
    // half 0 first (7 reads), then half 1 (7 reads)
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(A0[0]) : "v"(a0), "n"(0));
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(A0[1]) : "v"(a0), "n"(2048));
    static_for<0, RT_CTW>([&B0, bb](auto J) {
      constexpr int j = decltype(J)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(B0[j]) : "v"(bb), "n"(j * 2048));
    });
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(A1[0]) : "v"(a1), "n"(0));
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(A1[1]) : "v"(a1), "n"(2048));
    static_for<0, RT_CTW>([&B1, bb](auto J) {
      constexpr int j = decltype(J)::value;
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(B1[j]) : "v"(bb), "n"(j * 2048 + 1024));
    });
    // the first seven reads have landed once at most seven are pending
    asm volatile("s_waitcnt lgkmcnt(7)" : "+v"(A0[0]), "+v"(A0[1]), "+v"(B0[0]), "+v"(B0[1]), "+v"(B0[2]),
                 "+v"(B0[3]), "+v"(B0[4]));
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < RT_CTW; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_rt(A0[m]), as_bf16x8_rt(B0[j]), acc[m][j], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // the first half's multiplies stay ahead of the second wait
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(A1[0]), "+v"(A1[1]), "+v"(B1[0]), "+v"(B1[1]), "+v"(B1[2]),
                 "+v"(B1[3]), "+v"(B1[4]));
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < RT_CTW; ++j)
        acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8_rt(A1[m]), as_bf16x8_rt(B1[j]), acc[m][j], 0, 0, 0);
  };

  issue(0, 0);
  issue(1, 1);  // nst >= 2: the contraction is at least 128
#pragma unroll 1
  for (int s = 0; s < nst; ++s) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_rt(RT_LOADS));  // stage s landed (stage s+1 may be in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int nxt = s + 2 < nst ? s + 2 : nst - 1;  // past the end: the last stage again, never read
    issue(nxt, (s + 2) % RT_NS);
    compute(s % RT_NS);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_rt(0));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // logits (+ bias) of the block's tokens into LDS: accumulator lane holds
  // column lane & 15 of each tile, rows 4*(lane >> 4) + v
  float* s_l = (float*)lds;
#pragma unroll
  for (int j = 0; j < RT_CTW; ++j) {
    const int col = (wave * RT_CTW + j) * 16 + (lane & 15);
    if (col < E) {
      const float b = bias ? bias[col] : 0.f;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) s_l[(m * 16 + 4 * (lane >> 4) + v) * RT_LS + col] = acc[m][j][v] + b;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // selection: wave w takes tokens 8w .. 8w+7, four at a time (16 lanes each)
  const int j16 = lane & 15;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const int tk = wave * 8 + pass * 4 + (lane >> 4);
    const int64_t t = row0 + tk;
    const bool real = t < T;
    float v[RT_VPL];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < RT_VPL; ++i) {
      const int e = j16 + 16 * i;
      v[i] = e < E ? s_l[tk * RT_LS + e] : -INFINITY;
      m = fmaxf(m, v[i]);
    }
    m = row_max16(m);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < RT_VPL; ++i) {
      const int e = j16 + 16 * i;
      v[i] = e < E ? expf(v[i] - m) : 0.f;
      sum += v[i];
    }
    sum = row_sum16(sum);
    // optional: the token's routing probability mass per expert group (G equal
    // contiguous groups), for the expert-parallel balance statistics
    if (gmass) {
      const int gs = E / G;
#pragma unroll 1
      for (int g = 0; g < G; ++g) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < RT_VPL; ++i) {
          const int e = j16 + 16 * i;
          if (e < E && e / gs == g) a += v[i] / sum;
        }
        a = row_sum16(a);
        if (real && j16 == 0) gmass[t * G + g] = a;
      }
    }
    unsigned long long key[RT_VPL];
#pragma unroll
    for (int i = 0; i < RT_VPL; ++i) {
      const unsigned e = (unsigned)(j16 + 16 * i);
      key[i] = e < (unsigned)E ? ((unsigned long long)__float_as_uint(v[i] / sum) << 32) | (0xffffffffu - e) : 0ull;
    }
    // this token's number of experts: K, or k_tok[t] clamped to [0, K]
    int kt = K;
    if (k_tok) {
      kt = k_tok[real ? t : 0];
      kt = kt < 0 ? 0 : (kt > K ? K : kt);
    }
    // kt is uniform over the token's 16 lanes; rounds run to the wave's largest kt, a row whose
    // count is reached only reduces (its lanes agree, so its moves stay inside the row)
    float p_last = 0.f;
    const bool store = real && j16 == 0;
    const int rounds = gap ? K + 1 : K;  // the last round only finds the gap
#pragma unroll 1
    for (int r = 0; r < rounds; ++r) {
      unsigned long long best = key[0];
#pragma unroll
      for (int i = 1; i < RT_VPL; ++i) best = key[i] > best ? key[i] : best;
      best = row_max16_u64(best);
      const unsigned e = 0xffffffffu - (unsigned)(best & 0xffffffffu);
      const float p = __uint_as_float((unsigned)(best >> 32));
      if (r == kt) {
        if (gap && store) gap[t] = (kt > 0 && kt < E) ? p_last - p : INFINITY;
      } else if (r < kt) {
        if (store) {
          idx[t * K + r] = (int32_t)e;
          prob[t * K + r] = p;
        }
        p_last = p;
#pragma unroll
        for (int i = 0; i < RT_VPL; ++i)
          if ((unsigned)(j16 + 16 * i) == e) key[i] = 0ull;
      }
    }
    // slots past the token's own count: no expert
    if (store)
      for (int r = kt; r < K; ++r) {
        idx[t * K + r] = -1;
        prob[t * K + r] = 0.f;
      }
  }
}

}  // namespace

// Above 12288 tokens the two-kernel route is faster: every 32 tokens here read
// the whole router matrix again (d_model 4096, 288 experts: 119.5 against
// 107 us at 16384 tokens, 494 against 431 us at 65536; 59.7 against 75.9 us
// at 8192). Up to 6144 tokens the router GEMM with its contraction split over
// the idle compute units, then top-k over the partial sums, is faster too: a
// block here walks the whole contraction for its 32 tokens, about 62 us
// however few blocks there are.
bool router_topk_fits(int64_t T, int D, int E, int K) {
  return T > 6144 && T <= 12288 && E <= 20 * 16 && K <= E && D % RT_KS == 0 && D >= 2 * RT_KS;
}

hipError_t launch_router_topk(const bf16_t* x, int64_t T, int D, const bf16_t* w_router, bool packed,
                              const float* bias, int E, int K, const int32_t* k_tok, int32_t* idx, float* prob,
                              float* gap, float* gmass, int G, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (E > RT_NCT * 16 || K > E || D % RT_KS || D < 2 * RT_KS) return hipErrorInvalidValue;
  if (gmass && (G < 1 || E % G)) return hipErrorInvalidValue;
  const int64_t blocks = (T + RT_ROWS - 1) / RT_ROWS;
  if (packed)
    router_topk_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(x, T, D, w_router, bias, E, K, k_tok, idx, prob, gap,
                                                              gmass, G);
  else
    router_topk_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(x, T, D, w_router, bias, E, K, k_tok, idx, prob, gap,
                                                               gmass, G);
  return hipGetLastError();
}

}  // namespace moe
