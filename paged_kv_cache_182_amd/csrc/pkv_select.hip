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
//    rounding and the result is reproducible bit for bit). Summaries reach
//    the threads through LDS, loaded coalesced.
//  * select_kernel: one 1024-thread workgroup per row. An exact radix select
//    (8 bits per pass, most significant first, LDS histograms fed by one
//    atomic per distinct digit of a wave) finds the key of the k-th best
//    score; blocks above it are taken, and of those equal to it the lowest
//    block indices (ranked by workgroup prefix counts, only when more keys
//    equal it than are needed). The pages of the chosen blocks, and the
//    forced first and last pages, are marked in an LDS bitmap, which a
//    popcount prefix scan turns into the ascending page list.

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
constexpr int KPT = 32;  // keys per thread held in registers (rows up to 32,768 blocks)

// keys[i] for a runtime i (the rare tie-ranking path): a select chain keeps
// the array in registers
__device__ inline uint32_t key_of_reg(const uint32_t* keys, int i) {
  uint32_t v = 0u;
#pragma unroll
  for (int t = 0; t < KPT; ++t) v = t == i ? keys[t] : v;
  return v;
}

// Blocks of a row (ceil(L / BT)), with L clamped into [0, max_pages * P].
__device__ inline int row_blocks(int L, const SelectArgs& a) {
  return L <= 0 ? 0 : (int)(((int64_t)L + a.block_tokens - 1) / a.block_tokens);
}
__device__ inline int clamp_len(int L, const SelectArgs& a) {
  const int64_t cap = (int64_t)a.max_pages * a.page;
  return L < 0 ? 0 : (int)((int64_t)L > cap ? cap : L);
}

// Summaries are staged through LDS 64 dims at a time with coalesced,
// non-temporal (read once) 16-byte loads (a workgroup's 256 rows are
// contiguous in the slab; every thread issues its eight loads of a round
// before storing any), then each thread accumulates its own row in index
// order from LDS.
constexpr int CH = 64;                 // dims per staging round
constexpr int ROW_WORDS = CH / 2 + 4;  // one staged row: 128 bytes + 16 bytes of padding
constexpr int LOADS = CH / 8;          // 16-byte loads per thread per full round

__global__ void __launch_bounds__(SCORE_THREADS) score_kernel(const SelectArgs a) {
  extern __shared__ float qs[];  // the row's indexer query in fp32
  __shared__ __attribute__((aligned(16))) uint32_t stage[SCORE_THREADS * ROW_WORDS];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int j0 = blockIdx.x * SCORE_THREADS;
  const _Float16* q = reinterpret_cast<const _Float16*>(a.q_idx) + (size_t)b * a.idx_dim;
  for (int i = tid; i < a.idx_dim; i += SCORE_THREADS) qs[i] = (float)q[i];
  const int L = clamp_len(a.seq_lens[b], a);
  const int nb = min(row_blocks(L, a), a.max_blocks);
  const int nrows = min(SCORE_THREADS, nb - j0);  // rows of this workgroup (<= 0: none)
  if (nrows <= 0) return;                          // uniform over the workgroup
  const uint8_t* base = reinterpret_cast<const uint8_t*>(a.slab) + ((size_t)b * a.max_blocks + j0) * a.idx_dim * 2;
  const size_t row_bytes = (size_t)a.idx_dim * 2;
  float acc = 0.f;
  for (int d0 = 0; d0 < a.idx_dim; d0 += CH) {
    const int w = min(CH, a.idx_dim - d0);  // dims this round (a multiple of 8)
    const int chunks = w / 8;               // 16-byte chunks per row
    __syncthreads();
    const int total = nrows * chunks;  // <= LOADS * SCORE_THREADS
    u4 x[LOADS];
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int e = tid + k * SCORE_THREADS;
      const int r = e / chunks, c = e % chunks;
      if (e < total) x[k] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(base + r * row_bytes + (size_t)(d0 + 8 * c) * 2));
    }
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      const int e = tid + k * SCORE_THREADS;
      const int r = e / chunks, c = e % chunks;
      if (e < total) *reinterpret_cast<u4*>(&stage[r * ROW_WORDS + 4 * c]) = x[k];
    }
    __syncthreads();
    if (tid < nrows) {
      for (int c = 0; c < chunks; ++c) {
        const h8 x = __builtin_bit_cast(h8, *reinterpret_cast<const u4*>(&stage[tid * ROW_WORDS + 4 * c]));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qs[d0 + 8 * c + e], (float)x[e], acc);
      }
    }
  }
  if (tid < nrows) a.scores[(size_t)b * a.max_blocks + j0 + tid] = acc;
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
  __shared__ int whist[SEL_WAVES][256];  // per-wave histograms (no cross-wave contention)
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
  const int k = a.block_topk;
  const int lane = tid & 63;
  // Keys of blocks j = tid + 1024 i: held in registers when the row has at
  // most KPT * 1024 blocks (all loads issued at once), else re-read per pass.
  const bool in_regs = nb <= KPT * SEL_THREADS;  // uniform
  uint32_t keys[KPT];
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = tid + SEL_THREADS * i;
      keys[i] = j < nb ? order_key(sc[j]) : 0u;
    }
  }
  auto key_of = [&](int i, int j) -> uint32_t { return in_regs ? keys[i] : (j < nb ? order_key(sc[j]) : 0u); };
  const int iters = (nb + SEL_THREADS - 1) / SEL_THREADS;

  uint32_t thr = 0u;   // take keys > thr, and the `ties` lowest blocks of the keys == thr
  int ties = 0;
  const bool all = k >= nb;
  if (!all && k > 0) {
    uint32_t prefix = 0u, mask = 0u;
    int remaining = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < SEL_WAVES * 256; i += SEL_THREADS) (&whist[0][0])[i] = 0;
      __syncthreads();
      int* wh = whist[tid >> 6];
      auto count = [&](uint32_t key, bool valid) {
        if (valid && (key & mask) == prefix) atomicAdd(&wh[(key >> shift) & 255u], 1);
      };
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if (i < iters) count(keys[i], tid + SEL_THREADS * i < nb);
      } else {
        for (int i = 0; i < iters; ++i) {
          const int j = tid + SEL_THREADS * i;
          count(key_of(i, j), j < nb);
        }
      }
      __syncthreads();
      if (tid < 256) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < SEL_WAVES; ++w) t += whist[w][tid];
        hist[tid] = t;
      }
      __syncthreads();
      if (tid < 64) {
        // the bin holding the remaining-th largest key: lane l holds bins
        // 4l .. 4l+3; counts above each bin come from a suffix scan over the
        // lanes; the highest bin with (above + count >= remaining) is it
        const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
        int suf = c0 + c1 + c2 + c3;  // inclusive suffix sum over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_down(suf, o);
          if (lane + o < 64) suf += y;
        }
        const int s3 = suf - (c0 + c1 + c2 + c3);  // keys in bins above 4l+3
        const int s2 = s3 + c3, s1 = s2 + c2, s0 = s1 + c1;
        int best = -1, best_above = 0;
        if (s0 + c0 >= remaining) { best = 4 * lane; best_above = s0; }
        if (s1 + c1 >= remaining) { best = 4 * lane + 1; best_above = s1; }
        if (s2 + c2 >= remaining) { best = 4 * lane + 2; best_above = s2; }
        if (s3 + c3 >= remaining) { best = 4 * lane + 3; best_above = s3; }
        const uint64_t hit = __ballot(best >= 0);
        const int top = 63 - __builtin_clzll(hit);  // hit != 0: remaining <= keys with the prefix
        const int d = __builtin_amdgcn_readlane(best, top);
        const int above = __builtin_amdgcn_readlane(best_above, top);
        if (lane == 0) {
          pick[0] = prefix | ((uint32_t)d << shift);
          pick[1] = (uint32_t)(remaining - above);
        }
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
  const bool sel_some = !all && k > 0;
  // do the keys equal to the threshold all go in? (usually one key equals it)
  int total_ties = 0;
  if (sel_some) {
    int mine = 0;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) mine += tid + SEL_THREADS * i < nb && keys[i] == thr;
    } else {
      for (int i = 0; i < iters; ++i) {
        const int j = tid + SEL_THREADS * i;
        mine += j < nb && key_of(i, j) == thr;
      }
    }
    block_exclusive_scan(mine, wave_sums, &total_ties);
  }
  const bool rank_ties = sel_some && total_ties > ties;  // uniform
  __syncthreads();  // bitmap cleared

  auto mark = [&](int j) {
    const int64_t t0 = (int64_t)j * a.block_tokens;
    const int64_t t1 = min((int64_t)(j + 1) * a.block_tokens, (int64_t)L);
    for (int pg = (int)(t0 / a.page); pg <= (int)((t1 - 1) / a.page); ++pg)
      atomicOr(&bitmap[pg >> 5], 1u << (pg & 31));
  };
  if (k > 0) {
    if (!rank_ties) {
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          const int j = tid + SEL_THREADS * i;
          if (j < nb && (all || keys[i] >= thr)) mark(j);
        }
      } else {
        for (int i = 0; i < iters; ++i) {
          const int j = tid + SEL_THREADS * i;
          if (j < nb && (all || key_of(i, j) >= thr)) mark(j);
        }
      }
    } else {
      int rank = 0;  // ties in lower blocks
      for (int i = 0; i < iters; ++i) {
        const int j = tid + SEL_THREADS * i;
        const uint32_t key = j < nb ? (in_regs ? key_of_reg(keys, i) : key_of(i, j)) : 0u;
        const int t = j < nb && key == thr;
        int round_total;
        const int before = block_exclusive_scan(t, wave_sums, &round_total);
        if (j < nb && (key > thr || (t && rank + before < ties))) mark(j);
        rank += round_total;
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
