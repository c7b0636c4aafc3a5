// GPU page selection for the sparse decode path, gfx950: an indexer's block
// top-k over a compressed slab, then the pages those blocks touch compacted
// into the fixed-capacity selection array the attention kernel reads, with a
// counter of pages that did not fit (FreeToken PR #499 "Why this works": top-k
// block selection over a compressed slab, GPU-resident, fixed shape; "Design":
// compaction with a drop counter, capacity 2 * block_topk + 8).
//
//  * score_kernel: one thread per block; the dot product of the row's fp16
//    indexer query with the block's fp16 summary, accumulated in fp32 in
//    index order (each fp16 product is exact in fp32, so every step is one
//    rounding and the result is reproducible bit for bit).
//  * select_kernel: one 1024-thread workgroup per row. An exact radix select
//    (8 bits per pass, most significant first, LDS histograms) finds the key
//    of the k-th best score; blocks above it are taken, and of those equal to
//    it the lowest block indices (a prefix count over contiguous per-thread
//    ranges). The pages of the chosen blocks, and the forced first and last
//    pages, are marked in an LDS bitmap, which a popcount prefix scan turns
//    into the ascending page list.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int SCORE_THREADS = 256;
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

// Blocks of a row (ceil(L / BT)), with L clamped into [0, max_pages * P].
__device__ inline int row_blocks(int L, const SelectArgs& a) {
  return L <= 0 ? 0 : (int)(((int64_t)L + a.block_tokens - 1) / a.block_tokens);
}
__device__ inline int clamp_len(int L, const SelectArgs& a) {
  const int64_t cap = (int64_t)a.max_pages * a.page;
  return L < 0 ? 0 : (int)((int64_t)L > cap ? cap : L);
}

__global__ void __launch_bounds__(SCORE_THREADS) score_kernel(const SelectArgs a) {
  extern __shared__ float qs[];  // the row's indexer query in fp32
  const int b = blockIdx.y;
  const int j = blockIdx.x * SCORE_THREADS + threadIdx.x;
  const _Float16* q = reinterpret_cast<const _Float16*>(a.q_idx) + (size_t)b * a.idx_dim;
  for (int i = threadIdx.x; i < a.idx_dim; i += SCORE_THREADS) qs[i] = (float)q[i];
  __syncthreads();
  const int L = clamp_len(a.seq_lens[b], a);
  const int nb = min(row_blocks(L, a), a.max_blocks);
  if (j >= nb) return;
  const h8* s = reinterpret_cast<const h8*>(reinterpret_cast<const _Float16*>(a.slab) +
                                            ((size_t)b * a.max_blocks + j) * a.idx_dim);
  float acc = 0.f;
  for (int c = 0; c < a.idx_dim / 8; ++c) {
    const h8 x = s[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qs[8 * c + e], (float)x[e], acc);
  }
  a.scores[(size_t)b * a.max_blocks + j] = acc;
}

// Score -> key whose unsigned order is the score order; NaN lowest, -0 = +0.
__device__ inline uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (f == 0.f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (every thread passes x; returns the
// sum of x over lower thread ids; *total gets the sum over all).
__device__ inline int block_exclusive_scan(int x, int* wave_sums, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int v = lane < SEL_WAVES ? wave_sums[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(v, o);
      if (lane >= o) v += y;
    }
    if (lane < SEL_WAVES) wave_sums[lane] = v;  // inclusive sums of the waves
  }
  __syncthreads();
  const int before = (wave > 0 ? wave_sums[wave - 1] : 0) + incl - x;
  *total = wave_sums[SEL_WAVES - 1];
  __syncthreads();  // wave_sums is reused by the next scan
  return before;
}

__global__ void __launch_bounds__(SEL_THREADS) select_kernel(const SelectArgs a) {
  __shared__ int hist[256];
  __shared__ int wave_sums[SEL_WAVES];
  __shared__ uint32_t pick[2];  // threshold key, ties to take
  extern __shared__ uint32_t bitmap[];  // one bit per page of the row
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int raw_len = a.seq_lens[b];
  const int L = clamp_len(raw_len, a);
  if (tid == 0 && a.err && (raw_len < 0 || L != raw_len)) atomicAdd(a.err, 1);
  const int nb_all = row_blocks(L, a);
  if (tid == 0 && a.err && nb_all > a.max_blocks) atomicAdd(a.err, 1);
  const int nb = min(nb_all, a.max_blocks);
  const int npages = (int)(((int64_t)L + a.page - 1) / a.page);
  const int nwords = (npages + 31) / 32;
  for (int w = tid; w < nwords; w += SEL_THREADS) bitmap[w] = 0u;

  const float* sc = a.scores + (size_t)b * a.max_blocks;
  // contiguous block range of this thread
  const int per = (nb + SEL_THREADS - 1) / SEL_THREADS;
  const int j0 = min(tid * per, nb), j1 = min(j0 + per, nb);
  const int k = a.block_topk;

  uint32_t thr = 0u;   // take keys > thr, and `ties` of the keys == thr
  int ties = 0;
  const bool all = k >= nb;
  if (!all && k > 0) {
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
      __syncthreads();
      for (int j = j0; j < j1; ++j) {
        const uint32_t key = order_key(sc[j]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int above = 0, d = 255;
        for (; d > 0; --d) {
          if (above + hist[d] >= remaining) break;
          above += hist[d];
        }
        pick[0] = prefix | ((uint32_t)d << shift);
        pick[1] = (uint32_t)(remaining - above);
      }
      __syncthreads();
      prefix = pick[0];
      remaining = (int)pick[1];
      mask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    ties = remaining;
  }

  // ties are taken in block order: rank of this thread's first tie
  int my_ties = 0;
  if (!all && k > 0)
    for (int j = j0; j < j1; ++j) my_ties += order_key(sc[j]) == thr;
  int total_ties;
  int rank = block_exclusive_scan(my_ties, wave_sums, &total_ties);
  __syncthreads();  // bitmap cleared

  if (k > 0) {
    for (int j = j0; j < j1; ++j) {
      bool take = all;
      if (!all) {
        const uint32_t key = order_key(sc[j]);
        take = key > thr || (key == thr && rank < ties);
        rank += key == thr;
      }
      if (take) {
        const int64_t t0 = (int64_t)j * a.block_tokens;
        const int64_t t1 = min((int64_t)(j + 1) * a.block_tokens, (int64_t)L);
        for (int pg = (int)(t0 / a.page); pg <= (int)((t1 - 1) / a.page); ++pg)
          atomicOr(&bitmap[pg >> 5], 1u << (pg & 31));
      }
    }
  }
  // forced pages: the first sink_pages and the last recent_pages
  for (int pg = tid; pg < min(a.sink_pages, npages); pg += SEL_THREADS) atomicOr(&bitmap[pg >> 5], 1u << (pg & 31));
  for (int pg = max(npages - a.recent_pages, 0) + tid; pg < npages; pg += SEL_THREADS)
    atomicOr(&bitmap[pg >> 5], 1u << (pg & 31));
  __syncthreads();

  // compaction: contiguous word ranges per thread, popcount prefix
  const int wper = (nwords + SEL_THREADS - 1) / SEL_THREADS;
  const int w0 = min(tid * wper, nwords), w1 = min(w0 + wper, nwords);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __builtin_popcount(bitmap[w]);
  int total;
  int pos = block_exclusive_scan(cnt, wave_sums, &total);
  int32_t* out = a.sel + (size_t)b * a.max_sel;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = bitmap[w];
    while (bits) {
      const int bit = __builtin_ctz(bits);
      bits &= bits - 1;
      if (pos < a.max_sel) out[pos] = 32 * w + bit;
      ++pos;
    }
  }
  if (tid == 0) {
    a.sel_lens[b] = min(total, a.max_sel);
    if (total > a.max_sel && a.dropped) atomicAdd(a.dropped, total - a.max_sel);
  }
}

}  // namespace

int launch_select(const SelectArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned gx = (unsigned)((a.max_blocks + SCORE_THREADS - 1) / SCORE_THREADS);
  if (gx > 0)
    hipLaunchKernelGGL(score_kernel, dim3(gx, a.rows), dim3(SCORE_THREADS), (size_t)a.idx_dim * sizeof(float), s, a);
  if (hipGetLastError() != hipSuccess) return -4;
  const size_t bitmap_bytes = (size_t)((a.max_pages + 31) / 32) * 4;
  hipLaunchKernelGGL(select_kernel, dim3(a.rows), dim3(SEL_THREADS), bitmap_bytes, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
