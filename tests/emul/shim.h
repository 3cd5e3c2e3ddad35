// Host build of a HIP kernel source for bounds checking: the kernel body
// runs as plain C++, one lane at a time, and every global or LDS access it
// makes lands in an exact-size host buffer, so AddressSanitizer reports any
// access outside it. Matrix-core results are not computed (the accumulators
// pass through unchanged); the index arithmetic is the kernel's own.
#pragma once
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define __restrict__
struct uint4 { uint32_t x, y, z, w; };
struct float4 { float x, y, z, w; };
struct int4 { int x, y, z, w; };
struct uint2 { uint32_t x, y; };
inline uint2 make_uint2(uint32_t x, uint32_t y) { return uint2{x, y}; }
inline float4 make_float4(float x, float y, float z, float w) { return float4{x, y, z, w}; }
inline uint4 make_uint4(uint32_t x, uint32_t y, uint32_t z, uint32_t w) { return uint4{x, y, z, w}; }
struct emul_dim3 { unsigned x = 0, y = 0, z = 0; };
extern thread_local emul_dim3 threadIdx, blockIdx;
extern emul_dim3 gridDim, blockDim;
#define __align__(n) __attribute__((aligned(n)))
struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
typedef int hipError_t;
typedef void* hipStream_t;
constexpr int hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorInvalidDevice = 101;
inline int hipGetLastError() { return 0; }
inline int hipGetDevice(int* d) { *d = 0; return 0; }
typedef int hipDevice_t;
inline int hipStreamGetDevice(hipStream_t, hipDevice_t* d) { *d = 0; return 0; }
constexpr int hipDeviceAttributeMultiprocessorCount = 0;
inline int hipDeviceGetAttribute(int* v, int, int) { *v = 256; return 0; }
inline const char* hipGetErrorString(int) { return "emulated HIP error"; }
// a device variable's address is its host stand-in's address in the emulation
#define HIP_SYMBOL(x) ((const void*)&(x))
inline int hipGetSymbolAddress(void** p, const void* sym) { *p = (void*)sym; return 0; }
inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
inline float __expf(float x) { return expf(x); }
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
template <class T> T min(T a, T b) { return a < b ? a : b; }
template <class T> T max(T a, T b) { return a > b ? a : b; }
// Block barrier: a real barrier when the block runs one OS thread per lane
// (tests/emul/runner.h), nothing when lanes run one after another.
void emul_syncthreads();
inline void __syncthreads() { emul_syncthreads(); }
// Lane exchange within a wave (needs the one-thread-per-lane mode).
void emul_wave_sync();
extern thread_local long long* emul_wave_slots;  // 1024 slots of the running block
template <class T> T __shfl_up(T v, unsigned delta, int width) {
  (void)width;  // always the whole wave (64) in this library
  const unsigned lane = threadIdx.x & 63;
  long long slot = 0;
  memcpy(&slot, &v, sizeof(T));
  emul_wave_slots[threadIdx.x] = slot;
  emul_wave_sync();
  T r = v;
  if (lane >= delta) memcpy(&r, &emul_wave_slots[threadIdx.x - delta], sizeof(T));
  emul_wave_sync();
  return r;
}
inline int atomicAdd(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
// DPP lane moves of one 32-bit value (the controls this library uses: quad
// permutes, row half-mirror, row mirror, row_bcast:15, row_bcast:31): lane i
// takes the value of its source lane when its row is enabled in row_mask and
// the source exists, else keeps `old`. And readlane.
inline int emul_dpp_source(int lane, int ctrl) {
  if (ctrl <= 0xff) return (lane & ~3) + ((ctrl >> (2 * (lane & 3))) & 3);  // quad_perm
  if (ctrl == 0x140) return (lane & ~15) + (15 - (lane & 15));              // row_mirror
  if (ctrl == 0x141) return (lane & ~7) + (7 - (lane & 7));                 // row_half_mirror
  if (ctrl == 0x142) return lane >= 16 ? (lane & ~15) - 1 : -1;             // row_bcast:15
  if (ctrl == 0x143) return lane >= 32 ? 31 : -1;                           // row_bcast:31
  fprintf(stderr, "DPP control 0x%x is not emulated\n", ctrl);
  abort();
}
// Lane by lane (kernels whose lane moves feed values only, not addresses), a
// move returns the lane's own value.
bool emul_lanes_synced();
inline int emul_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
  (void)bank_mask, (void)bound_ctrl;  // all banks enabled in this library
  if (!emul_lanes_synced()) return old;
  const int lane = threadIdx.x & 63;
  emul_wave_slots[threadIdx.x] = src;
  emul_wave_sync();
  const int from = emul_dpp_source(lane, ctrl);
  int r = old;
  if (((row_mask >> (lane >> 4)) & 1) && from >= 0) r = (int)emul_wave_slots[(threadIdx.x & ~63) + from];
  emul_wave_sync();
  return r;
}
inline int emul_readlane(int v, int l) {
  emul_wave_slots[threadIdx.x] = v;
  emul_wave_sync();
  const int r = (int)emul_wave_slots[(threadIdx.x & ~63) + l];
  emul_wave_sync();
  return r;
}
inline unsigned long long __ballot(int pred) {  // bit l: lane l of the wave holds pred != 0
  emul_wave_slots[threadIdx.x] = pred != 0;
  emul_wave_sync();
  unsigned long long m = 0;
  for (int l = 0; l < 64; ++l)
    if (emul_wave_slots[(threadIdx.x & ~63) + l]) m |= 1ull << l;
  emul_wave_sync();
  return m;
}
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) emul_update_dpp((old), (src), (ctrl), (rm), (bm), (bc))
// mov_dpp: lanes without a source (or in disabled rows) get 0 with bound_ctrl, else keep src
inline int emul_mov_dpp(int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl) {
  if (!emul_lanes_synced()) return src;
  return emul_update_dpp(bound_ctrl ? 0 : src, src, ctrl, row_mask, bank_mask, bound_ctrl);
}
#define __builtin_amdgcn_mov_dpp(src, ctrl, rm, bm, bc) emul_mov_dpp((src), (ctrl), (rm), (bm), (bc))
#define __builtin_amdgcn_readlane(v, l) emul_readlane((v), (l))

// LDS addresses taken as 32-bit values become region * 2^20 + offset.
void* emul_lds_region_ptr(uint32_t vaddr, int bytes);
uint32_t emul_lds_base(void* p, size_t bytes);
// A direct global -> LDS load: lane l writes `bytes` at dst + l * bytes.
void emul_global_load_lds(const void* src, void* dst, int bytes);
extern long long emul_loads;

template <class V> inline V emul_ds_read(uint32_t vaddr) {
  V v;
  memcpy(&v, emul_lds_region_ptr(vaddr, sizeof(V)), sizeof(V));
  return v;
}
#define __builtin_amdgcn_global_load_lds(src, dst, size, off, aux) emul_global_load_lds((src), (dst), (size))
#define __builtin_amdgcn_s_waitcnt(x) ((void)0)
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
#define __builtin_amdgcn_readfirstlane(x) (x)
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) (c)
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) (c)
typedef float emul_f32x2 __attribute__((ext_vector_type(2)));
inline emul_f32x2 emul_cvt_pk_f32_fp8(int w, bool hi) {  // values are not needed, only the call's shape
  (void)w, (void)hi;
  return emul_f32x2{0.f, 0.f};
}
#define __builtin_amdgcn_cvt_pk_f32_fp8(w, hi) emul_cvt_pk_f32_fp8((w), (hi))
inline uint32_t emul_cvt_scalef32_pk_bf16_fp8(uint32_t w, float scale, bool hi) {  // shape only, as above
  (void)w, (void)scale, (void)hi;
  return 0u;
}
#define __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, hi) emul_cvt_scalef32_pk_bf16_fp8((w), (scale), (hi))
