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
inline uint4 make_uint4(uint32_t x, uint32_t y, uint32_t z, uint32_t w) { return uint4{x, y, z, w}; }
struct emul_dim3 { unsigned x = 0, y = 0, z = 0; };
extern thread_local emul_dim3 threadIdx, blockIdx;
extern emul_dim3 gridDim, blockDim;
typedef int hipError_t;
typedef void* hipStream_t;
constexpr int hipSuccess = 0, hipErrorInvalidValue = 1;
inline int hipGetLastError() { return 0; }
inline int hipGetDevice(int* d) { *d = 0; return 0; }
constexpr int hipDeviceAttributeMultiprocessorCount = 0;
inline int hipDeviceGetAttribute(int* v, int, int) { *v = 256; return 0; }
inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
inline float __expf(float x) { return expf(x); }
template <class T> T min(T a, T b) { return a < b ? a : b; }
template <class T> T max(T a, T b) { return a > b ? a : b; }
inline void __syncthreads() {}

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
