// GPU page selection for the sparse decode path, gfx950: an indexer's block
// top-k over a compressed slab, then the pages those blocks touch compacted
// into the fixed-capacity selection array the attention kernel reads, with a
// counter of pages that did not fit (FreeToken PR #499 "Why this works": top-k
// block selection over a compressed slab, GPU-resident, fixed shape; "Design":
// compaction with a drop counter, capacity 2 * block_topk + 8).
//
//  * score_kernel: one lane per block; the dot product of the row's fp16
//    indexer query with the block's fp16 summary, accumulated in fp32 in
//    index order (each fp16 product is exact in fp32, so every step is one
//    rounding and the result is reproducible bit for bit). A wave streams 64
//    blocks at a time through a private LDS slot, loaded coalesced.
//  * select_kernel: one 1024-thread workgroup per row. The key of the k-th
//    best score is found exactly. First a lower bound of it from the waves'
//    lane maxima keeps only the keys that can reach it (usually a few
//    hundred) as candidates in LDS; one wave then finds the key one bit at a
//    time from the top, a bit kept when at least k candidates reach it
//    (per-lane counts summed by DPP). Short rows, large k and candidate sets
//    over the cap take the same bit search over all the row's keys (wave
//    ballots summed across the waves through LDS). Blocks above the key are
//    taken, and of those equal to it the lowest block indices (ranked by
//    workgroup prefix counts, only when more keys equal it than are needed). The pages of the chosen blocks, and the forced
//    first and last pages, are marked in an LDS bitmap, which a popcount
//    prefix scan turns into the ascending page list.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int SCORE_WAVES = 4;
constexpr int SCORE_THREADS = 64 * SCORE_WAVES;
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int KPT_MAX = 32;  // keys per thread held in registers: rows of up to 32,768 blocks

// keys[i] for a runtime i (the rare tie-ranking path): a select chain keeps
// the array in registers
template <int KPT>
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

// Scores. One wave scores 64 consecutive blocks of a row at a time (a chunk),
// one block per lane, in rounds of up to 64 dims. A round's summaries arrive
// by coalesced 16-byte loads (consecutive lanes read consecutive bytes of the
// chunk), go through a wave-private LDS slot, and each lane reads its own
// block's summary back and accumulates its dot product in index order. The
// next round's loads are in flight while the current round is accumulated.
// The waves split the rows' chunks evenly, in order, so that the grid is one
// round of resident workgroups; no workgroup barrier is used.
constexpr int SC_DIMS = 64;                 // dims per round
constexpr int SC_PITCH = SC_DIMS * 2 + 16;  // LDS bytes per staged block: 128 + 16 of padding
constexpr int SC_SLOT = 64 * SC_PITCH;      // one wave's slot
constexpr int SC_LOADS = SC_DIMS / 8;       // 16-byte loads per lane in a full round
constexpr uint32_t SC_OFF_NONE = 0xFFFFFFF0u;  // past any row: reads zero, no traffic

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Piece i of lane `lane` in a round whose rows are cw 16-byte pieces long:
// piece e = lane + 64 i is piece c of block r (of the chunk); pieces past the
// round's 64 * cw are flagged by r = -1. FULL: every round has 64 dims.
template <bool FULL>
__device__ inline void sc_piece(int lane, int i, int cw, int& r, int& c) {
  const int e = lane + 64 * i;
  if (FULL || cw == SC_LOADS) {
    r = e >> 3;
    c = e & 7;
  } else {
    r = e / cw;
    c = e - r * cw;
    if (i >= cw) r = -1;
  }
}

struct ScoreUnit {
  int row, j0, d0, rnd;  // row, first block of the chunk, first dim, round
  int nb;                // blocks of the row
};

__device__ inline int sgpr(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <bool FULL>
__global__ void __launch_bounds__(SCORE_THREADS) __attribute__((amdgpu_waves_per_eu(4))) score_kernel(
    const SelectArgs a, const int64_t chunks, const int64_t nwaves) {
  __shared__ __attribute__((aligned(16))) uint8_t slots[SCORE_WAVES * SC_SLOT];
  __shared__ __attribute__((aligned(16))) float qslots[SCORE_WAVES * SC_DIMS];
  const int lane = threadIdx.x & 63;
  const int wave = sgpr(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * SCORE_WAVES + wave;
  if (gw >= nwaves) return;  // uniform over the wave
  const int64_t g0 = chunks * gw / nwaves, g1 = chunks * (gw + 1) / nwaves;
  const int rounds = (a.idx_dim + SC_DIMS - 1) / SC_DIMS;
  const int units = sgpr((int)(g1 - g0) * rounds);
  if (units <= 0) return;  // uniform over the wave; nothing below synchronises the workgroup
  const int cpr = (a.max_blocks + 63) >> 6;  // chunks per row
  const uint32_t row_bytes = (uint32_t)a.idx_dim * 2u;
  uint8_t* slot = slots + wave * SC_SLOT;
  float* qs = qslots + wave * SC_DIMS;

  // the units (chunk, round) of this wave in order; a row's block count is
  // read when the walk enters the row
  ScoreUnit nx;
  nx.row = sgpr((int)(g0 / cpr));
  nx.j0 = sgpr((int)(g0 - (int64_t)nx.row * cpr)) * 64;
  nx.d0 = 0;
  nx.rnd = 0;
  nx.nb = -1;
  auto blocks_of = [&](int row) {
    const int L = clamp_len(a.seq_lens[row], a);
    return sgpr(min(row_blocks(L, a), a.max_blocks));
  };
  // past the last unit: loads through zero-size ranges (no traffic), so every
  // iteration issues the same loads and the wait counts stay exact
  auto next_unit = [&](bool live) {
    if (!live) {
      ScoreUnit z = nx;
      z.nb = 0;
      return z;
    }
    ScoreUnit u = nx;
    if (u.nb < 0) u.nb = blocks_of(u.row);
    nx.nb = u.nb;
    if (++nx.rnd == rounds) {
      nx.rnd = 0;
      nx.j0 += 64;
      if (nx.j0 >= 64 * cpr) {
        nx.j0 = 0;
        ++nx.row;
        nx.nb = -1;
      }
    }
    nx.d0 = nx.rnd * SC_DIMS;
    return u;
  };
  // a round's loads: blocks past the row's end and pieces past the round read
  // zeros through the buffer bounds; the query's dims of the round as raw fp16
  auto issue = [&](const ScoreUnit& u, u4 (&x)[SC_LOADS], uint32_t& qh) {
    const int cw = FULL ? SC_LOADS : min(SC_DIMS, a.idx_dim - u.d0) / 8;
    const rsrc_t rs = make_rsrc(reinterpret_cast<const uint8_t*>(a.slab) + (size_t)u.row * a.max_blocks * row_bytes,
                                (uint32_t)u.nb * row_bytes);
#pragma unroll
    for (int i = 0; i < SC_LOADS; ++i) {
      int r, c;
      sc_piece<FULL>(lane, i, cw, r, c);
      const uint32_t off = r < 0 ? SC_OFF_NONE : (uint32_t)(u.j0 + r) * row_bytes + (uint32_t)(u.d0 + 8 * c) * 2u;
      x[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 2));
    }
    const rsrc_t rq = make_rsrc(reinterpret_cast<const uint8_t*>(a.q_idx) + (size_t)u.row * row_bytes,
                                u.nb > 0 ? row_bytes : 0u);
    qh = __builtin_amdgcn_raw_buffer_load_b16(rq, (int)((u.d0 + lane) * 2), 0, 0);
  };
  float acc = 0.f;
  auto consume = [&](const ScoreUnit& u, const u4 (&x)[SC_LOADS], uint32_t qh) {
    const int cw = FULL ? SC_LOADS : min(SC_DIMS, a.idx_dim - u.d0) / 8;
#pragma unroll
    for (int i = 0; i < SC_LOADS; ++i) {
      int r, c;
      sc_piece<FULL>(lane, i, cw, r, c);
      if (r >= 0) *reinterpret_cast<u4*>(slot + r * SC_PITCH + 16 * c) = x[i];
    }
    qs[lane] = (float)__builtin_bit_cast(_Float16, (uint16_t)qh);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int c = 0; c < cw; ++c) {
      const h8 v = __builtin_bit_cast(h8, *reinterpret_cast<const u4*>(slot + lane * SC_PITCH + 16 * c));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qs[8 * c + e], (float)v[e], acc);
    }
    if (u.rnd == rounds - 1) {
      // blocks past the row's end fall outside the range: not stored
      const rsrc_t ro = make_rsrc(a.scores + (size_t)u.row * a.max_blocks, (uint32_t)u.nb * 4u);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), ro, (u.j0 + lane) * 4, 0, 0);
      acc = 0.f;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };

  u4 xa[SC_LOADS], xb[SC_LOADS];
  uint32_t qa, qb;
  ScoreUnit ua = next_unit(true), ub;
  issue(ua, xa, qa);
  for (int t = 0; t < units; t += 2) {
    ub = next_unit(t + 1 < units);
    issue(ub, xb, qb);
    consume(ua, xa, qa);
    if (t + 1 >= units) break;
    ua = next_unit(t + 2 < units);
    issue(ua, xa, qa);
    consume(ub, xb, qb);
  }
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

// Sum / maximum over the 64 lanes of a wave, returned to every lane: DPP
// steps within each row of 16 lanes, then the four rows' results read out.
template <int CTRL>
__device__ inline uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ inline int wave_sum(int x) {
  uint32_t v = (uint32_t)x;
  v += dpp<0xB1>(v);   // quad lanes 1 0 3 2
  v += dpp<0x4E>(v);   // quad lanes 2 3 0 1
  v += dpp<0x141>(v);  // half-row mirror
  v += dpp<0x140>(v);  // row mirror
  return (int)(__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
               __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ inline uint32_t wave_max(uint32_t v) {
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x141>(v));
  v = max(v, dpp<0x140>(v));
  return max(max((uint32_t)__builtin_amdgcn_readlane(v, 0), (uint32_t)__builtin_amdgcn_readlane(v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane(v, 32), (uint32_t)__builtin_amdgcn_readlane(v, 48)));
}

// KPT: keys per thread held in registers (16 when the rows have at most
// 16,384 blocks, else 32)
constexpr int CAND_CAP = 64 * 16;  // candidates the final search holds (16 registers of one wave)

template <int KPT>
__global__ void __launch_bounds__(SEL_THREADS) select_kernel(const SelectArgs a) {
  __shared__ __attribute__((aligned(16))) int wcount[2][SEL_WAVES];  // the waves' counts of one search step
  __shared__ int wave_sums[SEL_WAVES];
  __shared__ uint32_t cands[CAND_CAP];  // keys that can hold the k-th best (see below)
  __shared__ int cand_total;
  __shared__ uint32_t pick[3];          // threshold, keys above it, keys equal to it
  extern __shared__ uint32_t bitmap[];  // one bit per page of the row
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* sc = a.scores + (size_t)b * a.max_blocks;
  // Keys of blocks j = tid + 1024 i are held in registers when the row has
  // at most KPT * 1024 blocks, else re-read per pass. Where every row fits,
  // the loads go out before the row's length is known (they read within the
  // row's max_blocks scores, or zero through the buffer bounds past them).
  uint32_t raw[KPT];
  const bool early = a.max_blocks <= KPT * SEL_THREADS;  // uniform
  const rsrc_t rs = make_rsrc(sc, (uint32_t)a.max_blocks * 4u);
  if (early) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) raw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (tid + SEL_THREADS * i) * 4, 0, 0);
  }
  const int raw_len = a.seq_lens[b];
  const int L = clamp_len(raw_len, a);
  if (tid == 0 && a.err && (raw_len < 0 || L != raw_len)) atomicAdd(a.err, 1);
  const int nb_all = row_blocks(L, a);
  if (tid == 0 && a.err && nb_all > a.max_blocks) atomicAdd(a.err, 1);
  const int nb = min(nb_all, a.max_blocks);
  const int npages = (int)(((int64_t)L + a.page - 1) / a.page);
  const int nwords = (npages + 31) / 32;
  for (int w = tid; w < nwords; w += SEL_THREADS) bitmap[w] = 0u;
  if (tid == 0) cand_total = 0;

  const int k = a.block_topk;
  const bool in_regs = nb <= KPT * SEL_THREADS;  // uniform
  uint32_t keys[KPT];
  if (in_regs) {
    if (!early) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) raw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (tid + SEL_THREADS * i) * 4, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int j = tid + SEL_THREADS * i;
      keys[i] = j < nb ? order_key(__builtin_bit_cast(float, raw[i])) : 0u;  // blocks past the row's end: key 0
    }
  }
  auto key_of = [&](int i, int j) -> uint32_t { return in_regs ? keys[i] : (j < nb ? order_key(sc[j]) : 0u); };
  const int iters = (nb + SEL_THREADS - 1) / SEL_THREADS;
  // keys >= t among this wave's keys held in registers
  auto wave_count_ge = [&](uint32_t t) -> int {
    int c = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(keys[i] >= t));
    return c;
  };

  uint32_t thr = 0u;   // take keys > thr, and the `ties` lowest blocks of the keys == thr
  int ties = 0;
  int total_ties = -1;  // keys equal to thr, when the search counted them
  const bool all = k >= nb;
  // keys >= t over the workgroup (t >= 1: the key 0 of a block past the row's
  // end never counts): per wave by ballots, then the waves' counts summed
  // through LDS; the two count buffers alternate, so one barrier per count
  int par = 0;
  auto count_ge = [&](uint32_t t) -> int {
    int c = 0;
    if (in_regs) {
      c = wave_count_ge(t);
    } else {
      for (int i = 0; i < iters; ++i) {
        const int j = tid + SEL_THREADS * i;
        c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key_of(i, j) >= t));
      }
    }
    if (lane == 0) wcount[par][wave] = c;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < SEL_WAVES; w += 4) {
      const int4 v = *reinterpret_cast<const int4*>(&wcount[par][w]);
      total += v.x + v.y + v.z + v.w;
    }
    par ^= 1;
    return total;
  };
  __syncthreads();  // cand_total cleared
  bool searched = false;
  if (!all && k > 0 && in_regs && nb >= SEL_THREADS && k <= 64 * SEL_WAVES) {
    // A lower bound T of the row's k-th largest key. Every lane holds at
    // least one block's key (nb >= 1024). A wave's q-th largest lane maximum
    // (q = ceil(k / 16)) is reached by at least q of its keys, so the
    // smallest of the 16 waves' is reached by at least k keys of the row:
    // T is at most the k-th largest key, and every key at or above that key
    // is a candidate (a key >= max(T, 1)).
    const int q = (k + SEL_WAVES - 1) / SEL_WAVES;
    uint32_t mx = keys[0];
#pragma unroll
    for (int i = 1; i < KPT; ++i) mx = max(mx, keys[i]);
    uint32_t tq = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tq | (1u << bit);
      if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(mx >= cand)) >= q) tq = cand;
    }
    if (lane == 0) wcount[0][wave] = (int)tq;
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < SEL_WAVES; w += 4) {
      const int4 v = *reinterpret_cast<const int4*>(&wcount[0][w]);
      lo = min(lo, min(min((uint32_t)v.x, (uint32_t)v.y), min((uint32_t)v.z, (uint32_t)v.w)));
    }
    lo = max(lo, 1u);
    const int n = wave_count_ge(lo);
    int base = 0;
    if (lane == 0) base = atomicAdd(&cand_total, n);
    base = __builtin_amdgcn_readfirstlane(base);
    if (base + n <= CAND_CAP) {  // uniform
      int pos = base;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool take = keys[i] >= lo;
        const uint64_t m = __builtin_amdgcn_ballot_w64(take);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (take) cands[pos + before] = keys[i];
        pos += __builtin_popcountll(m);
      }
    }
    __syncthreads();
    const int total = cand_total;  // uniform
    if (total <= CAND_CAP) {
      if (wave == 0) {
        // register r of lane l holds candidate 64 r + l (0 past the last)
        uint32_t c[CAND_CAP / 64];
        uint32_t cmax = 0u;
#pragma unroll
        for (int r = 0; r < CAND_CAP / 64; ++r) {
          c[r] = 64 * r + lane < total ? cands[64 * r + lane] : 0u;
          cmax = max(cmax, c[r]);
        }
        const int groups = (total + 255) / 256;  // groups of 4 registers in use
        // candidates >= t: per lane, then summed over the wave
        auto cand_count_ge = [&](uint32_t t) -> int {
          int cl = 0;
#pragma unroll
          for (int g = 0; g < CAND_CAP / 256; ++g) {
            if (g < groups) {
#pragma unroll
              for (int r = 4 * g; r < 4 * g + 4; ++r) cl += c[r] >= t ? 1 : 0;
            }
          }
          return wave_sum(cl);
        };
        cmax = wave_max(cmax);
        // The k-th largest key lies in [lo, cmax] when at least k candidates
        // exist (else it is below lo: a NaN score's key 0). Keys of that
        // range share their bits above the highest bit where lo and cmax
        // differ; the rest is found one bit at a time from the top.
        uint32_t t = 0u;
        if (total >= k) {
          const uint32_t diff = lo ^ cmax;
          const int h = diff ? 31 - __builtin_clz(diff) : -1;
          t = h < 0 ? lo : lo & ~((2u << h) - 1u);  // 2u << 31 wraps to 0: no common bits
          for (int bit = h; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            if (cand_count_ge(cand) >= k) t = cand;
          }
        }
        const int gt = t == 0xFFFFFFFFu ? 0 : (t == 0u ? -1 : cand_count_ge(t + 1u));
        const int ge = t >= 1u ? cand_count_ge(t) : -1;  // key 0 also marks blocks past the end: not counted here
        if (lane == 0) {
          pick[0] = t;
          pick[1] = (uint32_t)gt;
          pick[2] = (uint32_t)(ge < 0 ? -1 : ge - gt);
        }
      }
      __syncthreads();
      thr = pick[0];
      if (thr != 0u) {
        ties = k - (int)pick[1];  // keys equal to thr that go in
        total_ties = (int)pick[2];
        searched = true;
      }
    }
  }
  if (!all && k > 0 && !searched) {
    // the k-th largest key over all the row's keys: the largest t with
    // count_ge(t) >= k, one bit at a time from the top (t = 0 needs no count:
    // every block has a key >= 0)
    uint32_t t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (count_ge(cand) >= k) t = cand;
    }
    thr = t;
    ties = k - (thr == 0xFFFFFFFFu ? 0 : count_ge(thr + 1u));  // keys equal to thr that go in
  }
  const bool sel_some = !all && k > 0;
  // do the keys equal to the threshold all go in? (usually one key equals it)
  if (sel_some && total_ties < 0) {
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

  // block j covers tokens [j BT, min((j + 1) BT, L)); j < nb, so j BT < L
  // < 2^31 and the positions fit 32 bits
  auto mark = [&](int j) {
    if (a.block_tokens == a.page) {  // uniform: block j is page j
      atomicOr(&bitmap[j >> 5], 1u << (j & 31));
      return;
    }
    const uint32_t t0 = (uint32_t)j * (uint32_t)a.block_tokens;
    const uint32_t t1 = min(t0 + (uint32_t)a.block_tokens, (uint32_t)L);
    for (uint32_t pg = t0 / (uint32_t)a.page; pg <= (t1 - 1u) / (uint32_t)a.page; ++pg)
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
        const uint32_t key = j < nb ? (in_regs ? key_of_reg<KPT>(keys, i) : key_of(i, j)) : 0u;
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
  // one round of resident score workgroups (four per compute unit: LDS),
  // at most one wave per chunk of 64 blocks
  const int64_t chunks = (int64_t)a.rows * ((a.max_blocks + 63) / 64);
  const int64_t nwaves = std::min<int64_t>(chunks, (int64_t)a.cus * 4 * SCORE_WAVES);
  if (nwaves > 0)
    hipLaunchKernelGGL(a.idx_dim % SC_DIMS == 0 ? score_kernel<true> : score_kernel<false>, dim3((unsigned)((nwaves + SCORE_WAVES - 1) / SCORE_WAVES)), dim3(SCORE_THREADS), 0,
                       s, a, chunks, nwaves);
  if (hipGetLastError() != hipSuccess) return -4;
  const size_t bitmap_bytes = (size_t)((a.max_pages + 31) / 32) * 4;
  hipLaunchKernelGGL(a.max_blocks <= 16 * SEL_THREADS ? select_kernel<16> : select_kernel<KPT_MAX>, dim3(a.rows), dim3(SEL_THREADS), bitmap_bytes, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
