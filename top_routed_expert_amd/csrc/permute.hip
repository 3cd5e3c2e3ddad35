// Permutation of the (token, choice) pairs into per-expert row segments, so
// each expert's FFN (page "Step3.5 Flash 大模型技术深度解析", section 3.2.1:
// independent FFN per expert) runs on one contiguous block of rows.
//
// Pairs are numbered token-major (j = t*K + k). Row of pair j:
//   dest[j] = offsets[e] + #{ j' < j : idx[j'] == e },   e = idx[j]
// which is stable and unique, so the result is independent of scheduling.
//
//  1. rank: one block of 1024 threads per expert walks all pairs in order, a
//     block-wide prefix sum of match flags per 16384-pair chunk giving each
//     matching pair its rank; the total is the expert's count. No atomics.
//  2. place: every block rebuilds the exclusive scan of the E counts in LDS,
//     then maps each pair to dest and writes sorted_token[dest] = t; block 0
//     also writes the tile table of the expert GEMMs when asked.
// Small batches take a single-block path that also builds the tile table of
// the expert GEMMs (one launch instead of three).
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int PR_PER = 16;             // pairs per thread per chunk
constexpr int PR_THREADS = 1024;       // threads of a rank block
constexpr int PR_CHUNK = PR_THREADS * PR_PER;

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int w = __shfl_up(v, o, 64);
    if (lane >= o) v += w;
  }
  return v;
}

// Block b ranks the pairs of experts 2b and 2b+1 (one block per two experts,
// so 288 experts fit one round of the compute units): per chunk, each thread
// counts its pairs of both experts in one int (expert 2b in the low 16 bits,
// 2b+1 in the high 16; a chunk holds at most 16384 pairs, so the low half
// never carries into the high one), one block scan serves both, and each
// expert's running total across chunks is kept apart.
__global__ void __launch_bounds__(PR_THREADS) permute_rank_kernel(const int32_t* __restrict__ idx, int64_t P, int E,
                                                                  int32_t* __restrict__ rank,
                                                                  int32_t* __restrict__ counts) {
  __shared__ int s_wave[PR_THREADS / 64];
  const int e0 = 2 * (int)blockIdx.x, e1 = e0 + 1 < E ? e0 + 1 : -2;  // -2: no second expert
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int running0 = 0, running1 = 0;
  for (int64_t base = 0; base < P; base += PR_CHUNK) {
    const int64_t j0 = base + (int64_t)tid * PR_PER;
    int v[PR_PER];
    if (j0 + PR_PER <= P) {
#pragma unroll
      for (int i = 0; i < PR_PER; i += 4) {
        const int4 q = *(const int4*)(idx + j0 + i);
        v[i] = q.x;
        v[i + 1] = q.y;
        v[i + 2] = q.z;
        v[i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < PR_PER; ++i) v[i] = j0 + i < P ? idx[j0 + i] : -1;
    }
    int c = 0;
#pragma unroll
    for (int i = 0; i < PR_PER; ++i) c += (v[i] == e0) + ((v[i] == e1) << 16);
    const int incl = wave_incl_scan(c, lane);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < PR_THREADS / 64; ++w) {
      before += w < wave ? s_wave[w] : 0;
      total += s_wave[w];
    }
    const int excl = before + incl - c;
    int r0 = running0 + (excl & 0xffff), r1 = running1 + (excl >> 16);
#pragma unroll
    for (int i = 0; i < PR_PER; ++i) {
      if (v[i] == e0) rank[j0 + i] = r0++;
      else if (v[i] == e1) rank[j0 + i] = r1++;
    }
    running0 += total & 0xffff;
    running1 += total >> 16;
    __syncthreads();
  }
  if (tid == 0) {
    counts[e0] = running0;
    if (e1 >= 0) counts[e1] = running1;
  }
}

__global__ void __launch_bounds__(256) permute_place_kernel(const int32_t* __restrict__ idx, int64_t P, int K, int E,
                                                            const int32_t* __restrict__ rank,
                                                            const int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_token,
                                                            int32_t* __restrict__ dest,
                                                            int32_t* __restrict__ offsets_ext, int32_t extra_rows,
                                                            Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                            int32_t max_tiles, int BM) {
  __shared__ int s_off[1025];
  __shared__ int s_wave[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // exclusive scan of counts: thread owns experts 4*tid .. 4*tid+3
  int c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    c[i] = e < E ? counts[e] : 0;
    sum += c[i];
  }
  const int incl = wave_incl_scan(sum, lane);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w = 0; w < wave; ++w) run += s_wave[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    if (e < E) s_off[e] = run;
    run += c[i];
  }
  if (tid == 255) s_off[E] = run;  // the last thread ends on the total
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += 256) {
      if (offsets) offsets[e] = s_off[e];
      if (offsets_ext) offsets_ext[e] = s_off[e];
    }
    if (offsets_ext && tid == 0) {  // rows of pairs without an expert, then the extra rows
      offsets_ext[E + 1] = (int32_t)P;
      offsets_ext[E + 2] = (int32_t)P + extra_rows;
    }
    if (tiles) {
      // the expert GEMMs' tile table over the E routed segments and, with
      // extra_rows, group E (rows of pairs without an expert: no tiles) and
      // group E+1 (the extra rows): thread tid owns groups 4*tid .. 4*tid+3,
      // thread 255 also group E+1
      int g0[5], g1[5], nt[5], mine = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int g = i < 4 ? 4 * tid + i : E + 1;
        g0[i] = g1[i] = 0;
        if (i < 4 && g < E) {
          g0[i] = s_off[g];
          g1[i] = s_off[g + 1];
        } else if (i == 4 && tid == 255 && extra_rows > 0) {
          g0[i] = (int)P;
          g1[i] = (int)P + extra_rows;
        }
        nt[i] = (g1[i] - g0[i] + BM - 1) / BM;
        mine += nt[i];
      }
      __syncthreads();  // s_wave is reused
      const int incl2 = wave_incl_scan(mine, lane);
      if (lane == 63) s_wave[wave] = incl2;
      __syncthreads();
      int slot = incl2 - mine, n_all = 0;
      for (int w = 0; w < 4; ++w) {
        slot += w < wave ? s_wave[w] : 0;
        n_all += s_wave[w];
      }
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int g = i < 4 ? 4 * tid + i : E + 1;
        const int first = slot;
        for (int row = g0[i]; row < g1[i]; row += BM, ++slot)
          if (slot < max_tiles) tiles[slot] = Tile{g, row, row + BM < g1[i] ? row + BM : g1[i], first, nt[i], 0, 0, 0};
      }
      if (tid == 0) *n_tiles = n_all < max_tiles ? n_all : max_tiles;
    }
  }
  for (int64_t j = (int64_t)blockIdx.x * 256 + tid; j < P; j += (int64_t)gridDim.x * 256) {
    const int e = idx[j];
    if (e >= 0 && e < E) {
      const int d = s_off[e] + rank[j];
      dest[j] = d;
      sorted_token[d] = (int32_t)(j / K);
    } else {
      dest[j] = -1;
    }
  }
}

__global__ void __launch_bounds__(256) gather_rows_kernel(const uint4* __restrict__ x, int row_vecs,
                                                          const int32_t* __restrict__ sorted_token, int64_t T,
                                                          uint4* __restrict__ x_perm) {
  const int64_t r = blockIdx.x;
  int64_t t = sorted_token[r];
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);
  for (int i = threadIdx.x; i < row_vecs; i += 256) x_perm[r * row_vecs + i] = x[t * row_vecs + i];
}

__global__ void __launch_bounds__(256) gather_rows_bytes_kernel(const uint8_t* __restrict__ x, int row_bytes,
                                                                const int32_t* __restrict__ sorted_token, int64_t T,
                                                                uint8_t* __restrict__ x_perm) {
  const int64_t r = blockIdx.x;
  int64_t t = sorted_token[r];
  t = t < 0 ? 0 : (t >= T ? T - 1 : t);
  for (int i = threadIdx.x; i < row_bytes; i += 256) x_perm[r * row_bytes + i] = x[t * row_bytes + i];
}

// Exclusive prefix sum over a block of 1024 threads (16 waves): wave scans,
// then the 16 wave totals scanned by wave 0. s_tot holds 16 ints; *total
// receives the sum. Two barriers; every thread of the block must call it.
__device__ __forceinline__ int block1024_excl_scan(int v, int* s_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v, lane);
  if (lane == 63) s_tot[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? s_tot[lane] : 0;
    w = wave_incl_scan(w, lane);
    if (lane < 16) s_tot[lane] = w;
  }
  __syncthreads();
  *total = s_tot[15];
  return (wave ? s_tot[wave - 1] : 0) + incl - v;
}

// Small batches (T*K <= 1024, E <= 1022): the whole permutation and the
// expert-GEMM tile table in one block of 1024 threads (pair p = thread p, so
// wave w holds pairs 64w .. 64w+63). A pair's stable rank among the earlier
// pairs of its expert is (pairs of that expert in earlier waves) + (lanes
// below it in its own wave with the same expert). Each lane counts the
// second term, and the wave's total for its expert, over the wave's 64 ids
// in LDS; the wave's first lane of each expert writes that total to
// s_cnt[w][e] (no atomics), and thread e turns column e of s_cnt into an
// exclusive scan over the waves and the expert's total. So the result is
// the same stable permutation as the two-kernel path.
__global__ void __launch_bounds__(1024) permute_small_kernel(const int32_t* __restrict__ idx, int P, int K, int E,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_token,
                                                             int32_t* __restrict__ dest,
                                                             int32_t* __restrict__ offsets_ext, int32_t extra_rows,
                                                             Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                             int32_t max_tiles, int BM) {
  __shared__ int s_cnt[16 * 1024];  // [wave][expert]
  __shared__ __attribute__((aligned(16))) int s_idx[1024];
  __shared__ int s_off[1025];
  __shared__ int s_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e_raw = tid < P ? idx[tid] : -1;
  const bool valid = e_raw >= 0 && e_raw < E;
  const int e_mine = valid ? e_raw : -1;
  s_idx[tid] = e_mine;
  for (int i = tid; i < 16 * E; i += 1024) s_cnt[i] = 0;
  __syncthreads();
  // this wave's lanes with the same expert: below this one (r_wave) and in all (n_wave), from
  // the wave's 64 ids in LDS, four per read
  int r_wave = 0, n_wave = 0;
  const int4* w4 = (const int4*)&s_idx[wave * 64];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int4 q = w4[j];
    const int b = 4 * j;
    r_wave += (b < lane && q.x == e_mine) + (b + 1 < lane && q.y == e_mine) + (b + 2 < lane && q.z == e_mine) +
              (b + 3 < lane && q.w == e_mine);
    n_wave += (q.x == e_mine) + (q.y == e_mine) + (q.z == e_mine) + (q.w == e_mine);
  }
  if (valid && r_wave == 0) s_cnt[wave * E + e_mine] = n_wave;  // the wave's first lane of the expert
  __syncthreads();
  // column e: exclusive scan over the waves, total = the expert's pair count
  int c = 0;
  if (tid < E)
    for (int w = 0; w < 16; ++w) {
      const int v = s_cnt[w * E + tid];
      s_cnt[w * E + tid] = c;
      c += v;
    }
  int total;
  const int off_mine = block1024_excl_scan(c, s_tot, &total);
  if (tid < E) s_off[tid] = off_mine;  // s_off now holds offsets
  if (tid == 0) s_off[E] = total;
  __syncthreads();
  if (tid <= E) {
    if (offsets) offsets[tid] = s_off[tid];
    if (offsets_ext) offsets_ext[tid] = s_off[tid];
  }
  if (tid == 0 && offsets_ext) {  // rows of pairs without an expert, then the extra rows
    offsets_ext[E + 1] = P;
    offsets_ext[E + 2] = P + extra_rows;
  }
  if (tid < P) {
    if (valid) {
      const int d = s_off[e_mine] + s_cnt[wave * E + e_mine] + r_wave;
      dest[tid] = d;
      sorted_token[d] = tid / K;
    } else {
      dest[tid] = -1;
    }
  }
  if (tiles == nullptr) return;
  // tile table over the E routed groups and, with extra_rows, group E (rows
  // of pairs without an expert: no tiles) and group E+1 (the extra rows)
  int seg0 = 0, seg1 = 0;
  if (tid < E) {
    seg0 = s_off[tid];
    seg1 = s_off[tid + 1];
  } else if (tid == E + 1 && extra_rows > 0) {
    seg0 = P;
    seg1 = P + extra_rows;
  }
  const int mine = (seg1 - seg0 + BM - 1) / BM;
  int n_all;
  __syncthreads();  // s_tot is reused
  int slot = block1024_excl_scan(mine, s_tot, &n_all);
  const int first = slot;
  for (int row = seg0; row < seg1; row += BM, ++slot)
    if (slot < max_tiles) tiles[slot] = Tile{tid, row, row + BM < seg1 ? row + BM : seg1, first, mine, 0, 0, 0};
  if (tid == 1023) *n_tiles = n_all < max_tiles ? n_all : max_tiles;
}

// Receive plan of one GPU's share under expert parallelism (page "Step3.5
// Flash 大模型技术深度解析", section 3.2.3: the experts in G groups, one group
// per GPU). The receive buffer of the dispatch exchange holds one chunk per
// (source rank r, local expert e), r-major, counts[r * n_local + e] rows each,
// rows in the source's token order. Expert-major order takes the experts in
// turn, inside an expert the sources in turn, inside a chunk its rows in turn:
// expert-major row q reads receive row gather[q], receive row i holds
// expert-major row scatter[i], and offsets [n_local+1] bound the experts'
// segments. Every block rebuilds both chunk scans in LDS (at most 1024
// chunks), then maps receive rows grid-stride, finding each row's chunk by
// binary search. Rows at or past max_rows are not written.
__global__ void __launch_bounds__(1024) ep_plan_kernel(const int32_t* __restrict__ counts, int n_src, int n_local,
                                                       int64_t max_rows, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ gather, int32_t* __restrict__ scatter) {
  __shared__ int s_rcv[1025];  // receive-order start of chunk c = r * n_local + e; s_rcv[n] = total
  __shared__ int s_em[1024];   // expert-major start of chunk c
  __shared__ int s_tot[16];
  const int tid = threadIdx.x, n = n_src * n_local;
  const int cnt = tid < n ? max(counts[tid], 0) : 0;
  int total;
  const int rcv = block1024_excl_scan(cnt, s_tot, &total);
  if (tid < n) s_rcv[tid] = rcv;
  if (tid == 0) s_rcv[n] = total;
  __syncthreads();  // s_tot is reused
  // expert-major position p = e * n_src + r holds chunk r * n_local + e
  const int pe = tid / n_src, pr = tid - pe * n_src;
  const int cnt_em = tid < n ? max(counts[pr * n_local + pe], 0) : 0;
  int total_em;
  const int em = block1024_excl_scan(cnt_em, s_tot, &total_em);
  if (tid < n) s_em[pr * n_local + pe] = em;
  if (blockIdx.x == 0) {
    if (tid < n && pr == 0) offsets[pe] = em;
    if (tid == 0) offsets[n_local] = total_em;
  }
  __syncthreads();
  const int64_t rows = total < max_rows ? total : max_rows;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + tid; i < rows; i += (int64_t)gridDim.x * 1024) {
    int lo = 0, hi = n - 1;  // the last chunk starting at or before i (it holds row i)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_rcv[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int64_t q = (int64_t)s_em[lo] + (i - s_rcv[lo]);
    scatter[i] = (int32_t)q;
    if (q < max_rows) gather[q] = (int32_t)i;
  }
}

}  // namespace

hipError_t launch_ep_plan(const int32_t* counts, int n_src, int n_local, int64_t max_rows, int32_t* offsets,
                          int32_t* gather, int32_t* scatter, hipStream_t s) {
  int64_t blocks = (max_rows + 1023) / 1024;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  ep_plan_kernel<<<(unsigned)blocks, 1024, 0, s>>>(counts, n_src, n_local, max_rows, offsets, gather, scatter);
  return hipGetLastError();
}

bool permute_small_fits(int64_t T, int K, int E) { return T * K <= 1024 && E <= 1022; }

hipError_t launch_permute_small(const int32_t* idx, int64_t T, int K, int E, int32_t* offsets, int32_t* sorted_token,
                                int32_t* dest, int32_t* offsets_ext, int32_t extra_rows, Tile* tiles,
                                int32_t* n_tiles, int32_t max_tiles, int block_rows, hipStream_t s) {
  permute_small_kernel<<<1, 1024, 0, s>>>(idx, (int)(T * K), K, E, offsets, sorted_token, dest, offsets_ext,
                                          extra_rows, tiles, n_tiles, max_tiles, block_rows);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int K, int E, int32_t* rank, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_token, int32_t* dest, int32_t* offsets_ext,
                          int32_t extra_rows, Tile* tiles, int32_t* n_tiles, int32_t max_tiles, int block_rows,
                          hipStream_t s) {
  const int64_t P = T * K;
  permute_rank_kernel<<<(E + 1) / 2, PR_THREADS, 0, s>>>(idx, P, E, rank, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int64_t blocks = (P + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  permute_place_kernel<<<(unsigned)blocks, 256, 0, s>>>(idx, P, K, E, rank, counts, offsets, sorted_token, dest,
                                                        offsets_ext, extra_rows, tiles, n_tiles, max_tiles,
                                                        block_rows);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, int64_t T, int D, int elem_bytes, const int32_t* sorted_token,
                              int64_t rows, void* x_perm, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int row_bytes = D * elem_bytes;
  if (row_bytes % 16 == 0)
    gather_rows_kernel<<<(unsigned)rows, 256, 0, s>>>((const uint4*)x, row_bytes / 16, sorted_token, T,
                                                      (uint4*)x_perm);
  else
    gather_rows_bytes_kernel<<<(unsigned)rows, 256, 0, s>>>((const uint8_t*)x, row_bytes, sorted_token, T,
                                                            (uint8_t*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
