// Kernel launches of the host build (tests/emul): every lane of every block
// runs the kernel body as plain C++ under AddressSanitizer.
//
// Two modes:
//   - lane by lane: the blocks of a grid are spread over 8 host threads, and
//     inside a block the lanes run one after another. For kernels whose
//     control flow and addresses do not depend on what other lanes wrote to
//     LDS (the GEMMs: their LDS holds operand values only); barriers are no-ops.
//   - one OS thread per lane: each block runs with blockDim OS threads and a
//     real barrier behind __syncthreads (and a per-wave barrier behind wave
//     shuffles), for kernels that scan or count through LDS (tile builder,
//     permutation). Blocks run one after another, so the kernel's static LDS
//     arrays belong to one block at a time.
// Also the LDS address space of the inline-asm reads and the direct
// global -> LDS loads (see shim.h).
#pragma once
#include <atomic>
#include <mutex>
#include <thread>
#include <vector>

thread_local emul_dim3 threadIdx, blockIdx;
emul_dim3 gridDim, blockDim;
long long emul_loads = 0;  // direct loads into LDS of the last lane-by-lane launch

// ---- barriers ----
struct EmulBarrier {  // sense counter plus generation; waiters sleep on the generation (futex)
  std::atomic<unsigned> count{0}, gen{0};
  unsigned n = 0;
  void reset(unsigned parties) { n = parties, count = 0; }
  void wait() {
    const unsigned g = gen.load(std::memory_order_acquire);
    if (count.fetch_add(1, std::memory_order_acq_rel) + 1 == n) {
      count.store(0, std::memory_order_relaxed);
      gen.fetch_add(1, std::memory_order_acq_rel);
      gen.notify_all();
    } else {
      gen.wait(g, std::memory_order_acquire);
    }
  }
};
static thread_local bool emul_sync_mode = false;
static EmulBarrier g_block_barrier;
static EmulBarrier g_wave_barrier[16];
static long long g_wave_slots[1024];
thread_local long long* emul_wave_slots = g_wave_slots;
bool emul_lanes_synced() { return emul_sync_mode; }
void emul_syncthreads() {
  if (emul_sync_mode) g_block_barrier.wait();
}
void emul_wave_sync() {
  if (!emul_sync_mode) {
    fprintf(stderr, "wave shuffle in a kernel run lane by lane\n");
    abort();
  }
  g_wave_barrier[threadIdx.x >> 6].wait();
}

// ---- LDS regions: one per LDS array of each kernel instantiation ----
// Registered once (under a lock) and never removed, so readers need no lock.
static void* g_regions[64];
static size_t g_sizes[64];
static std::atomic<int> g_nreg{0};
static std::mutex g_reg_mu;
uint32_t emul_lds_base(void* p, size_t bytes) {
  const int n = g_nreg.load(std::memory_order_acquire);
  for (int i = 0; i < n; ++i)
    if (g_regions[i] == p) return (uint32_t)i << 20;
  std::lock_guard<std::mutex> lk(g_reg_mu);
  const int m = g_nreg.load(std::memory_order_relaxed);
  for (int i = 0; i < m; ++i)
    if (g_regions[i] == p) return (uint32_t)i << 20;
  if (m == 64) { fprintf(stderr, "too many LDS regions\n"); abort(); }
  g_regions[m] = p;
  g_sizes[m] = bytes;
  g_nreg.store(m + 1, std::memory_order_release);
  return (uint32_t)m << 20;
}
void* emul_lds_region_ptr(uint32_t vaddr, int bytes) {
  const int n = g_nreg.load(std::memory_order_acquire);
  const int r = (int)(vaddr >> 20);
  const uint32_t off = vaddr & 0xfffff;
  if (r >= n || off + bytes > g_sizes[r]) {
    fprintf(stderr, "LDS read out of range: region %d offset %u (+%d); block %u thread %u\n", r, off, bytes,
            blockIdx.x, threadIdx.x);
    abort();
  }
  return (char*)g_regions[r] + off;
}
// direct loads counted per host thread (summed by emul_direct_loads)
static std::atomic<long long> g_loads_done{0};
static thread_local long long t_loads = 0;
void emul_global_load_lds(const void* src, void* dst, int bytes) {
  const int lane = threadIdx.x & 63;
  memcpy((char*)dst + lane * bytes, src, bytes);
  ++t_loads;
}
static void emul_flush_loads() {
  g_loads_done.fetch_add(t_loads);
  t_loads = 0;
}

// ---- launches ----
inline dim3 emul_grid(dim3 g) { return g; }
inline dim3 emul_grid(unsigned x) { return dim3(x); }
inline dim3 emul_grid(int x) { return dim3((unsigned)x); }
inline dim3 emul_grid(long x) { return dim3((unsigned)x); }

template <class K, class... A>
void emul_run(bool sync, K kernel, dim3 grid, unsigned threads, A... args) {
  gridDim.x = grid.x, gridDim.y = grid.y, gridDim.z = 1;
  blockDim.x = threads, blockDim.y = 1, blockDim.z = 1;
  const unsigned nblocks = grid.x * grid.y;
  if (nblocks == 0) return;
  if (sync) {
    g_block_barrier.reset(threads);
    for (unsigned w = 0; w < (threads + 63) / 64; ++w) g_wave_barrier[w].reset(threads - 64 * w < 64 ? threads - 64 * w : 64);
    std::vector<std::thread> th;
    for (unsigned t = 0; t < threads; ++t)
      th.emplace_back([&, t] {
        emul_sync_mode = true;
        for (unsigned b = 0; b < nblocks; ++b) {
          blockIdx.x = b % grid.x, blockIdx.y = b / grid.x;
          threadIdx.x = t;
          kernel(args...);
          g_block_barrier.wait();  // the block's LDS arrays are reused by the next block
        }
      });
    for (auto& t : th) t.join();
  } else {
    std::vector<std::thread> th;
    g_loads_done = 0;
    for (int w = 0; w < 8; ++w)
      th.emplace_back([&, w] {
        for (unsigned b = w; b < nblocks; b += 8)
          for (unsigned t = 0; t < threads; ++t) {
            blockIdx.x = b % grid.x, blockIdx.y = b / grid.x;
            threadIdx.x = t;
            kernel(args...);
          }
        emul_flush_loads();
      });
    for (auto& t : th) t.join();
    emul_loads = g_loads_done.load();
  }
}
