// Write side of the paged cache, gfx950: token append into 16-bit pages and
// re-encoding (demotion) of full 16-bit pages to FP8 / INT8 / INT4 / INT2 /
// 1-bit / 16-bit.
//
// Recent pages stay FP16 while they fill; full older pages are re-encoded
// into a compact codec (ARGUS "Adaptive activation" and "v0.5"). FP8 pages
// hold e4m3 codes with one fp32 scale per (page, KV head, plane) (FreeToken
// PR #499 update, item 1); INT8/INT4 pages hold one fp16 scale per token and
// group of 32 dims (GGML Q8/Q4 pages, ARGUS "Direct paged attention"). The
// INT2 and 1-bit tiers of ARGUS's cascade (intro): INT2 as the unsigned-affine
// 2-bit kind of its "Pluggable tiers" (an fp16 offset and step per token and
// group), 1-bit as the sign with one fp16 scale (the mean magnitude) per token
// and group.
//
// In-page layout (the library's definition; the decode kernels read it).
// A plane is the codes of every KV head, head after head, then for INT8/INT4
// fp16 scales [Hkv][P][D/32]. One head's codes are P/16 tiles of 16 tokens.
// Each tile is the register image of the 64 lanes that consume it: lane L
// owns a run of D/4 elements (R = D*bits/32 bytes); with R >= 16 the runs are
// interleaved in 16-byte chunks (chunk i of lane L at i*1024 + 16*L), else
// run L sits at R*L. Run element e of lane L is
//  * K, one-scale codecs (FP16/BF16/FP8): token L%16, dim (D/4)(L/16) + e;
//  * K, group-scale codecs (INT8/INT4):   token L%16, dim 32(e/8) + 8(L/16) + e%8;
//  * V, every codec: token 4(L/16) + e%4, dim 16(e/4) + L%16.
// Codes of fewer than 8 bits fill a run in units of min(32, run bits) bits,
// m codes each: code r of a unit at slot (r%2)*(m/2) + r/2 (INT4: eight per
// word; INT2: sixteen; BIT1: thirty-two, or sixteen in a 16-bit unit). The
// group-scale codecs (INT8, INT4, INT2, BIT1) use the grouped K order; INT2
// planes hold fp16 offsets [Hkv][P][D/32] after the scales.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

enum : int { W_FP16 = 0, W_BF16 = 1, W_FP8 = 2, W_INT8 = 3, W_INT4 = 4, W_INT2 = 5, W_BIT1 = 6 };

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int wbits(int c) {
  return c <= W_BF16 ? 16 : (c == W_INT4 ? 4 : (c == W_INT2 ? 2 : (c == W_BIT1 ? 1 : 8)));
}
__device__ inline bool w16(int c) { return c == W_FP16 || c == W_BF16; }
// symmetric integer codes: c = clip(rint(x / s), -qmax, qmax)
__host__ __device__ constexpr bool wint(int c) { return c == W_INT8 || c == W_INT4; }
// codecs with one fp16 scale per (token, 32 dims), in the grouped K order
__host__ __device__ constexpr bool wgrp(int c) { return wint(c) || c == W_INT2 || c == W_BIT1; }
__host__ __device__ constexpr bool wsub(int c) { return c == W_INT2 || c == W_BIT1; }

__device__ inline uint64_t wplane_bytes(int c, int hkv, int page, int d) {
  const uint64_t codes = (uint64_t)hkv * page * d * wbits(c) / 8;
  const uint64_t groups = (uint64_t)hkv * page * (d / 32) * 2;
  return codes + (wgrp(c) ? groups : 0) + (c == W_INT2 ? groups : 0);
}

// (token in tile, dim) of run element e of lane L.
__device__ inline void run_elem(int L, int e, int D, bool is_v, bool grouped, int& tt, int& d) {
  if (is_v) {
    tt = 4 * (L >> 4) + (e & 3);
    d = 16 * (e >> 2) + (L & 15);
  } else if (grouped) {
    tt = L & 15;
    d = 32 * (e >> 3) + 8 * (L >> 4) + (e & 7);
  } else {
    tt = L & 15;
    d = (D / 4) * (L >> 4) + e;
  }
}

// Byte offset inside a tile of run byte rb of lane L (R = run bytes).
__device__ inline uint32_t run_byte(int L, int rb, int R) {
  return R >= 16 ? (uint32_t)((rb >> 4) * 1024 + 16 * L + (rb & 15)) : (uint32_t)(R * L + rb);
}

__device__ inline float h16_to_f(uint16_t c, int codec) {
  if (codec == W_FP16) return (float)__builtin_bit_cast(_Float16, c);
  return __builtin_bit_cast(float, (uint32_t)c << 16);
}

// float (exactly an fp16 value, or any finite float) -> bf16 code, nearest even.
__device__ inline uint16_t f_to_bf16(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ inline void count_err(int32_t* err) {
  if (err) atomicAdd(err, 1);
}

// A plane at byte offset `off` in codec c: 16-byte aligned and inside the pool.
__device__ inline bool plane_fits(uint64_t off, int c, int hkv, int page, int d, uint64_t pool_bytes) {
  return (off & 15) == 0 && off <= pool_bytes && pool_bytes - off >= wplane_bytes(c, hkv, page, d);
}

__device__ inline bool disjoint(uint64_t a, uint64_t an, uint64_t b, uint64_t bn) { return a + an <= b || b + bn <= a; }

// Checks of encode pair i, for both planes at once (a pair with one bad plane
// is skipped whole): ids in range and distinct, a 16-bit source in both
// planes, every plane aligned and inside the pool, no destination plane
// overlapping a source plane or the other destination plane. Returns the
// answer (the same in every lane and every unit of the pair) and, for
// `plane`, the destination id, the source and destination codecs and the
// source and destination plane offsets.
__device__ inline bool check_pair(const EncodeArgs& a, int i, int plane, int D, int& dst, int& scodec, int& dcodec,
                                  uint64_t& so, uint64_t& dof) {
  const int P = a.page, hkv = a.hkv;
  const int src = a.src[i];
  dst = a.dst[i];
  const int dk = a.dst_codec & 15, dv = (a.dst_codec >> 4) & 15;
  dcodec = plane ? dv : dk;
  scodec = 0;
  so = 0;
  dof = 0;
  if (!((unsigned)src < (unsigned)a.num_pages && (unsigned)dst < (unsigned)a.num_pages && src != dst)) return false;
  const int cb = a.codec[src];
  const int sk = cb & 15, sv = cb >> 4;
  const uint64_t sko = a.koff[src], svo = a.voff[src], dko = a.koff[dst], dvo = a.voff[dst];
  scodec = plane ? sv : sk;
  so = plane ? svo : sko;
  dof = plane ? dvo : dko;
  if (!(w16(sk) && w16(sv))) return false;
  const uint64_t skb = wplane_bytes(sk, hkv, P, D), svb = wplane_bytes(sv, hkv, P, D);
  const uint64_t dkb = wplane_bytes(dk, hkv, P, D), dvb = wplane_bytes(dv, hkv, P, D);
  const bool fit = plane_fits(sko, sk, hkv, P, D, a.pool_bytes) && plane_fits(svo, sv, hkv, P, D, a.pool_bytes) &&
                   plane_fits(dko, dk, hkv, P, D, a.pool_bytes) && plane_fits(dvo, dv, hkv, P, D, a.pool_bytes);
  return fit && disjoint(dko, dkb, sko, skb) && disjoint(dko, dkb, svo, svb) && disjoint(dvo, dvb, sko, skb) &&
         disjoint(dvo, dvb, svo, svb) && disjoint(dko, dkb, dvo, dvb);
}

// OR the code of run element e (E elements of BITS bits) into the run's words.
template <int BITS, int E>
__device__ inline void put_code(uint32_t* word, int e, uint32_t code) {
  if constexpr (BITS == 16) {
    word[e >> 1] |= (code & 0xFFFFu) << (16 * (e & 1));
  } else if constexpr (BITS == 8) {
    word[e >> 2] |= (code & 0xFFu) << (8 * (e & 3));
  } else {
    constexpr int UB = E * BITS < 32 ? E * BITS : 32;  // unit bits
    constexpr int M = UB / BITS;                        // codes per unit
    const int r = e % M;
    const int bit = (e / M) * UB + BITS * ((r & 1) * (M / 2) + (r >> 1));
    word[bit >> 5] |= (code & ((1u << BITS) - 1u)) << (bit & 31);
  }
}

// Store a destination run of RD bytes (lane L's run at its layout position).
template <int RD, bool NT>
__device__ inline void store_run_words(uint8_t* td, const uint32_t* word, int lane) {
  if constexpr (RD >= 16) {
#pragma unroll
    for (int c = 0; c < RD / 16; ++c) {
      const u4 x = {word[4 * c], word[4 * c + 1], word[4 * c + 2], word[4 * c + 3]};
      u4* p = reinterpret_cast<u4*>(td + (c * 1024 + 16 * lane));
      if constexpr (NT) __builtin_nontemporal_store(x, p); else *p = x;
    }
  } else if constexpr (RD == 8) {
    u2* p = reinterpret_cast<u2*>(td + 8 * lane);
    if constexpr (NT) __builtin_nontemporal_store(u2{word[0], word[1]}, p); else *p = u2{word[0], word[1]};
  } else if constexpr (RD == 4) {
    uint32_t* p = reinterpret_cast<uint32_t*>(td + 4 * lane);
    if constexpr (NT) __builtin_nontemporal_store(word[0], p); else *p = word[0];
  } else {
    static_assert(RD == 2, "run of 2 bytes expected");
    uint16_t* p = reinterpret_cast<uint16_t*>(td + 2 * lane);
    if constexpr (NT) __builtin_nontemporal_store((uint16_t)word[0], p); else *p = (uint16_t)word[0];
  }
}

// INT2 group offset and step from the group's minimum and maximum (fp32):
// z = fp16(lo) saturated to +-65504; s = fp16(RN((hi - z) / 3)) kept inside
// [2^-24, 65504], or 1 when hi - z <= 0. Returned as fp32 values.
__device__ inline void affine2_params(float lo, float hi, float& z, float& st) {
  z = fminf(fmaxf((float)(_Float16)lo, -65504.0f), 65504.0f);
  const float span = hi - z;
  if (span > 0.f) {
    float s = (float)(_Float16)__fdiv_rn(span, 3.0f);
    st = fminf(fmaxf(s, 0x1p-24f), 65504.0f);
  } else {
    st = 1.0f;
  }
}
__device__ inline uint32_t affine2_code(float x, float z, float st) {
  const float q = __builtin_rintf(__fdiv_rn(x - z, st));
  return (uint32_t)(int)fminf(fmaxf(q, 0.0f), 3.0f);
}
// 1-bit group scale from the exact float64 sum of the group's magnitudes:
// fp16(fp32(sum / 32)), capped at 65504 (0 for an all-zero group).
__device__ inline float sign1_scale(double sum) {
  return fminf((float)(_Float16)(float)(sum / 32.0), 65504.0f);
}

// ------------------------------------------------------------------ append
// Grid (row, KV head, plane), 64 threads; thread = dims d, d + 64, ...
__global__ void __launch_bounds__(64) append_kernel(AppendArgs a) {
  const int b = blockIdx.x, h = blockIdx.y, plane = blockIdx.z, tid = threadIdx.x;
  const int D = a.head_dim, P = a.page;
  const int L = a.seq_lens[b];
  bool ok = L >= 0 && L / P < a.max_pages;
  int pp = -1;
  if (ok) {
    pp = a.bt[(size_t)b * a.max_pages + L / P];
    ok = (unsigned)pp < (unsigned)a.num_pages;
  }
  int codec = 0;
  uint64_t off = 0;
  if (ok) {
    // both planes are checked in every unit, so a row with one bad plane
    // writes neither of them (and is counted once)
    const int cb = a.codec[pp];
    const uint64_t ko = a.koff[pp], vo = a.voff[pp];
    ok = w16(cb & 15) && w16(cb >> 4) && plane_fits(ko, cb & 15, a.hkv, P, D, a.pool_bytes) &&
         plane_fits(vo, cb >> 4, a.hkv, P, D, a.pool_bytes);
    codec = plane ? (cb >> 4) : (cb & 15);
    off = plane ? vo : ko;
  }
  if (!ok) {
    if (h == 0 && plane == 0 && tid == 0) count_err(a.err);
    return;
  }
  const int t = L % P, tile = t / 16, tt = t % 16;
  const int R = D / 2;                                  // run bytes of a 16-bit tile
  uint8_t* base = a.pool + off + (size_t)h * P * D * 2 + (size_t)tile * 16 * D * 2;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(plane ? a.v_new : a.k_new) + ((size_t)b * a.hkv + h) * D;
  for (int d = tid; d < D; d += 64) {
    int lane, e;
    if (plane) {
      lane = 16 * (tt / 4) + (d & 15);
      e = 4 * (d >> 4) + (tt & 3);
    } else {
      lane = 16 * (d / (D / 4)) + tt;
      e = d % (D / 4);
    }
    const uint16_t x = src[d];
    const uint16_t code = codec == W_FP16 ? x : f_to_bf16((float)__builtin_bit_cast(_Float16, x));
    *reinterpret_cast<uint16_t*>(base + run_byte(lane, 2 * e, R)) = code;
  }
}

// ------------------------------------------------------------------ encode
// Codes of one destination run (lane L of a tile): D/4 elements from the
// staged tile x[token][dim], written with 16-byte (8 for INT4 at D = 64)
// stores at the run's chunk positions.
template <int D, int DC, bool IS_V>
__device__ __attribute__((always_inline)) inline void emit_run(const float (*x)[D + 1], const float (*sc)[D / 32],
                                                               const float (*zs)[D / 32], float s8, uint8_t* td,
                                                               int lane) {
  constexpr int BITS = wbits(DC);
  constexpr int E = D / 4, RD = D * BITS / 32;
  constexpr int NWD = RD < 4 ? 1 : RD / 4;
  constexpr bool GROUPED = wgrp(DC) && !IS_V;
  constexpr float QMAX = DC == W_INT8 ? 127.0f : 7.0f;
  uint32_t word[NWD];
#pragma unroll
  for (int k = 0; k < NWD; ++k) word[k] = 0;
  if constexpr (DC == W_FP8) {
    // two elements per hardware conversion (OCP e4m3, nearest even) after the
    // correctly rounded quotient is clipped to +-448
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      int tt0, d0, tt1, d1;
      run_elem(lane, e, D, IS_V, GROUPED, tt0, d0);
      run_elem(lane, e + 1, D, IS_V, GROUPED, tt1, d1);
      const float y0 = fminf(fmaxf(__fdiv_rn(x[tt0][d0], s8), -448.0f), 448.0f);
      const float y1 = fminf(fmaxf(__fdiv_rn(x[tt1][d1], s8), -448.0f), 448.0f);
      if ((e >> 1) & 1)
        word[e >> 2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)word[e >> 2], true);
      else
        word[e >> 2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)word[e >> 2], false);
    }
  }
#pragma unroll
  for (int e = 0; e < (DC == W_FP8 ? 0 : E); ++e) {
    int tt, d;
    run_elem(lane, e, D, IS_V, GROUPED, tt, d);
    const float v = x[tt][d];
    uint32_t code;
    if constexpr (DC == W_FP16) {
      code = __builtin_bit_cast(uint16_t, (_Float16)v);
    } else if constexpr (DC == W_BF16) {
      code = f_to_bf16(v);
    } else if constexpr (DC == W_INT2) {
      code = affine2_code(v, zs[tt][d / 32], sc[tt][d / 32]);
    } else if constexpr (DC == W_BIT1) {
      code = v < 0.f ? 1u : 0u;
    } else {
      const float q = __builtin_rintf(__fdiv_rn(v, sc[tt][d / 32]));
      code = (uint32_t)(int)fminf(fmaxf(q, -QMAX), QMAX);
    }
    put_code<BITS, E>(word, e, code);
  }
  store_run_words<RD, false>(td, word, lane);
}

// SUB: the kernel is built for destination pairs with an INT2 or BIT1 plane
// (those codecs only; the other five codecs are built without them).
template <int D, bool IS_V, bool SUB>
__device__ __attribute__((always_inline)) inline void emit_any(int dc, const float (*x)[D + 1], const float (*sc)[D / 32],
                                                               const float (*zs)[D / 32], float s8, uint8_t* td,
                                                               int lane) {
  if constexpr (SUB) {
    if (dc == W_INT2) return emit_run<D, W_INT2, IS_V>(x, sc, zs, s8, td, lane);
    if (dc == W_BIT1) return emit_run<D, W_BIT1, IS_V>(x, sc, zs, s8, td, lane);
  }
  switch (dc) {
    case W_FP16: emit_run<D, W_FP16, IS_V>(x, sc, zs, s8, td, lane); break;
    case W_BF16: emit_run<D, W_BF16, IS_V>(x, sc, zs, s8, td, lane); break;
    case W_FP8: emit_run<D, W_FP8, IS_V>(x, sc, zs, s8, td, lane); break;
    case W_INT8: emit_run<D, W_INT8, IS_V>(x, sc, zs, s8, td, lane); break;
    default: emit_run<D, W_INT4, IS_V>(x, sc, zs, s8, td, lane); break;
  }
}

// Grid (pair i, KV head, plane); TILES tiles of 16 tokens staged at once, one
// 64-lane slot each (TILES = min(4, P/16), so no slot idles on small pages).
template <int D, int TILES, bool SUB>
__global__ void __launch_bounds__(64 * TILES) encode_kernel(EncodeArgs a) {
  constexpr int THREADS = 64 * TILES;
  __shared__ float xs[TILES][16][D + 1];              // staged tiles, [token][dim]
  __shared__ float scs[TILES][16][D / 32];            // group scales (fp32 of the fp16 value)
  __shared__ float zss[TILES][16][D / 32];            // INT2 group offsets
  __shared__ float red[TILES];
  const int i = blockIdx.x, h = blockIdx.y, plane = blockIdx.z, tid = threadIdx.x;
  const int P = a.page, hkv = a.hkv;
  const int lane = tid & 63, slot = tid >> 6;

  // ---- pair checks (every thread of every unit of the pair computes the same answer)
  int dst, scodec, dcodec;
  uint64_t so, dof;
  const bool ok = check_pair(a, i, plane, D, dst, scodec, dcodec, so, dof);
  if (!ok) {
    if (h == 0 && plane == 0 && tid == 0) count_err(a.err);
    return;
  }
  const int dbits = wbits(dcodec);
  const uint8_t* sp = a.pool + so + (size_t)h * P * D * 2;
  uint8_t* dp = a.pool + dof + (size_t)h * P * D * dbits / 8;

  // ---- FP8 scale: from the absmax of the head's whole block. A page that
  // fits one staging round takes it while staging (one read of the page);
  // a longer page takes it in a streaming pass first.
  const int ntiles = P / 16;
  const bool one_round = ntiles <= TILES;
  float s8 = 1.f;
  if (dcodec == W_FP8 && !one_round) {
    float m = 0.f;
    const uint32_t n16 = (uint32_t)(P * D * 2 / 16);
    for (uint32_t c = tid; c < n16; c += THREADS) {
      const u4 w = *reinterpret_cast<const u4*>(sp + 16 * (size_t)c);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m = fmaxf(m, __builtin_fabsf(h16_to_f((uint16_t)(w[k] & 0xFFFF), scodec)));
        m = fmaxf(m, __builtin_fabsf(h16_to_f((uint16_t)(w[k] >> 16), scodec)));
      }
    }
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[slot] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int k = 1; k < TILES; ++k) m = fmaxf(m, red[k]);
    s8 = m == 0.f ? 1.f : __fdiv_rn(m, 448.0f);
    if (tid == 0 && a.scale) a.scale[((size_t)dst * hkv + h) * 2 + plane] = s8;
  } else if (dcodec != W_FP8 && tid == 0 && a.scale) {
    a.scale[((size_t)dst * hkv + h) * 2 + plane] = 1.f;
  }
  if (h == 0 && plane == 0 && tid == 0) a.codec_out[dst] = (uint8_t)a.dst_codec;

  const bool is_v = plane == 1;
  constexpr int RS = D / 2;                              // source run bytes (16-bit)
  constexpr int G = D / 32;
  const float qmax = dcodec == W_INT8 ? 127.0f : 7.0f;

  for (int t0 = 0; t0 < ntiles; t0 += TILES) {
    const int tile = t0 + slot;
    const bool live = tile < ntiles;
    __syncthreads();
    // stage: lane L of this slot reads its source run (16-bit layout, ungrouped K)
    float mloc = 0.f;
    if (live) {
      const uint8_t* ts = sp + (size_t)tile * 16 * D * 2;
#pragma unroll
      for (int c = 0; c < RS / 16; ++c) {
        const u4 w = *reinterpret_cast<const u4*>(ts + run_byte(lane, 16 * c, RS));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          int tt, d;
          run_elem(lane, 8 * c + k, D, is_v, false, tt, d);
          const uint16_t code = (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFF));
          const float v = h16_to_f(code, scodec);
          xs[slot][tt][d] = v;
          mloc = fmaxf(mloc, __builtin_fabsf(v));
        }
      }
    }
    if (dcodec == W_FP8 && one_round) {   // the whole page is staged: its absmax
      for (int o = 32; o >= 1; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
      if (lane == 0) red[slot] = mloc;
    }
    __syncthreads();
    if (dcodec == W_FP8 && one_round) {
      float m = red[0];
#pragma unroll
      for (int k = 1; k < TILES; ++k) m = fmaxf(m, red[k]);
      s8 = m == 0.f ? 1.f : __fdiv_rn(m, 448.0f);
      if (tid == 0 && a.scale) a.scale[((size_t)dst * hkv + h) * 2 + plane] = s8;
    }
    // group scales (and INT2 offsets): one (token, group) per lane of the slot
    if (live && wgrp(dcodec)) {
      for (int q = lane; q < 16 * G; q += 64) {
        const int tt = q / G, g = q % G;
        _Float16 s16, z16 = (_Float16)0.0f;
        if (SUB && dcodec == W_INT2) {
          float lo = xs[slot][tt][32 * g], hi = lo;
#pragma unroll 8
          for (int j = 1; j < 32; ++j) {
            lo = fminf(lo, xs[slot][tt][32 * g + j]);
            hi = fmaxf(hi, xs[slot][tt][32 * g + j]);
          }
          float z, st;
          affine2_params(lo, hi, z, st);
          s16 = (_Float16)st;
          z16 = (_Float16)z;
        } else if (SUB && dcodec == W_BIT1) {
          double sum = 0.0;                       // exact for 16-bit inputs
#pragma unroll 8
          for (int j = 0; j < 32; ++j) sum += (double)__builtin_fabsf(xs[slot][tt][32 * g + j]);
          s16 = (_Float16)sign1_scale(sum);
        } else {
          float m = 0.f;
#pragma unroll 8
          for (int j = 0; j < 32; ++j) m = fmaxf(m, __builtin_fabsf(xs[slot][tt][32 * g + j]));
          // fp16 scale kept inside its positive finite range [2^-24, 65504]
          s16 = (_Float16)__fdiv_rn(m, qmax);
          s16 = s16 == (_Float16)0.0f ? __builtin_bit_cast(_Float16, (uint16_t)0x0001) : s16;
          s16 = s16 > (_Float16)65504.0f ? (_Float16)65504.0f : s16;
          s16 = m == 0.f ? (_Float16)1.0f : s16;
        }
        scs[slot][tt][g] = (float)s16;
        zss[slot][tt][g] = (float)z16;
        const size_t so16 = (size_t)hkv * P * D * dbits / 8 + ((size_t)h * P + 16 * tile + tt) * G * 2 + 2 * g;
        *reinterpret_cast<_Float16*>(a.pool + dof + so16) = s16;
        if (SUB && dcodec == W_INT2)
          *reinterpret_cast<_Float16*>(a.pool + dof + so16 + (size_t)hkv * P * G * 2) = z16;
      }
    }
    __syncthreads();
    if (!live) continue;
    uint8_t* td = dp + (size_t)tile * 16 * D * dbits / 8;
    if (is_v)
      emit_any<D, true, SUB>(dcodec, xs[slot], scs[slot], zss[slot], s8, td, lane);
    else
      emit_any<D, false, SUB>(dcodec, xs[slot], scs[slot], zss[slot], s8, td, lane);
  }
}

// x / s for a scale s with r = RN(1 / s): one product and one correction.
// Equal to the correctly rounded quotient on every code the encoder can
// produce from the inputs it can meet (|x| <= the block's or group's absmax;
// FP8 scales of at least 2^-100): checked exhaustively over every fp16 and
// bf16 source value by tests/division/check_recip_div.c.
__device__ inline float recip_div(float x, float s, float r) {
  const float q0 = __fmul_rn(x, r);
  return __builtin_fmaf(-__builtin_fmaf(q0, s, -x), r, q0);
}
// The same quotient with q0 taken as fma(x, r, 0): equal to RN(x * r) but for
// the sign of a zero product, which leaves q zero alike. Written so, the
// product reads an fp16 x straight from its half of the source word (a mixed-
// precision fma), with no conversion of its own.
__device__ inline float recip_div0(float x, float s, float r) {
  const float q0 = __builtin_fmaf(x, r, 0.0f);
  return __builtin_fmaf(-__builtin_fmaf(q0, s, -x), r, q0);
}

// RN(1 / s) for a stored fp16 group scale s (as float, in [2^-24, 65504]):
// the hardware reciprocal estimate and one Newton step. Exact for every such s
// and every estimate within two units in the last place of the result, checked
// exhaustively by tests/division/check_scale_div.c (which also covers the
// group scale m / qmax taken through recip_div with the constant RN(1 / qmax)).
__device__ inline float recip_fp16_scale(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(r0, __builtin_fmaf(-s, r0, 1.0f), r0);
}

// INT2 code u = clip(rint(RN((x - z) / s)), 0, 3) with the division as
// recip_div by r = RN(1 / s): for an fp16 step s the corrected quotient is
// RN(d / s) for every fp32 d, which tests/division/check_affine2_div.c checks
// for every step over every dividend near the rounding boundaries.
// Computed as for the INT codes: the quotient clamped to [0, 3] by a median of
// three, then 1.5 * 2^23 added (rounds to the nearest integer, ties to even,
// and leaves it in the low bits); d = x - z as fma(x, 1, -z), the same value,
// so an fp16 x is read from its half of the source word.
__device__ inline uint32_t affine2_code_r(float x, float z, float st, float r) {
  const float d = __builtin_fmaf(x, 1.0f, -z);
  const float q = __builtin_amdgcn_fmed3f(recip_div0(d, st, r), 0.0f, 3.0f);
  return __builtin_bit_cast(uint32_t, q + 12582912.0f) & 3u;
}

// ------------------------------------------------------ encode, register path
// Pages of up to four tiles (P <= 64): one wave per unit (page pair, KV head,
// plane), units dealt round-robin over the waves of the grid. The wave holds
// its unit's source in registers -- each lane the 16-byte chunks holding the
// elements of its own destination run (its own source run, except for grouped
// INT K, whose dims come from other lanes' runs) -- takes the FP8 block absmax
// or the INT group maxima by cross-lane reductions, and writes its
// destination run. The next unit's loads are issued before the current unit
// is encoded, so they are in flight meanwhile. No barriers.

constexpr int EW = 4;  // waves per workgroup

__device__ inline float dpp_f(float x, int ctrl) {
  switch (ctrl) {  // the control must be a constant
    case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  }
}
// max over the 16 lanes of this lane's row (quad swaps, then half-row and row mirrors)
__device__ inline float row16_max(float x) {
  x = fmaxf(x, dpp_f(x, 0xB1));
  x = fmaxf(x, dpp_f(x, 0x4E));
  x = fmaxf(x, dpp_f(x, 0x141));
  return fmaxf(x, dpp_f(x, 0x140));
}

// ---- many reductions at once over the 16 lanes of a row (reduce-scatter)
// A lane holds one value per combo. A step pairs lanes whose index differs in
// one bit b (the row mirror pairs l and 15 - l, the half-row mirror l and
// 7 - l inside each 8 lanes, the quad permutes l ^ 2 and l ^ 1) and each lane
// keeps, combined with its partner's copy, the half of its combos whose bit b
// equals its own: N combos over 16 lanes take N - 1 exchanges instead of
// 4 N, and lane l ends with combo l.
template <int CTRL>
__device__ inline uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline double dpp_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint64_t lo = dpp_u<CTRL>((uint32_t)u), hi = dpp_u<CTRL>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}
template <int CTRL>
__device__ inline uint32_t dpp_any(uint32_t x) { return dpp_u<CTRL>(x); }
template <int CTRL>
__device__ inline double dpp_any(double x) { return dpp_d<CTRL>(x); }

// one step on v[0 .. N): v[k] for k < N / 2 becomes op(kept, partner's copy)
// of combo k + N/2 (keep_hi) or k
template <int CTRL, int N, class T, class Op>
__device__ inline void halve(T* v, bool keep_hi, Op op) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const T lo = v[k], hi = v[k + N / 2];
    const T keep = keep_hi ? hi : lo, send = keep_hi ? lo : hi;
    v[k] = op(keep, dpp_any<CTRL>(send));
  }
}
// N = 16 or 8 combos (index = the lane that keeps it); returns combo l16's
// reduction over the row (lanes l16 >= N hold a copy of combo l16 % N's).
template <int N, class T, class Op>
__device__ inline T row16_scatter(T (&v)[N], int l16, Op op) {
  static_assert(N == 8 || N == 16, "8 or 16 combos");
  if constexpr (N == 16) {
    halve<0x140, 16>(v, (l16 & 8) != 0, op);  // row mirror: partners differ in bit 3
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = op(v[k], dpp_any<0x140>(v[k]));  // both halves of the row
  }
  halve<0x141, 8>(v, (l16 & 4) != 0, op);  // half-row mirror: bit 2 (bit 3 kept)
  halve<0x4E, 4>(v, (l16 & 2) != 0, op);   // quad [2,3,0,1]: bit 1
  halve<0xB1, 2>(v, (l16 & 1) != 0, op);   // quad [1,0,3,2]: bit 0
  return v[0];
}

// The same for combos held two to a 32-bit word (combo 2w in the low half of
// word w, 2w + 1 in the high half), combined by a packed operation: returns
// the 16-bit reduction of combo l16 (N = 16 or 8 combos).
template <int N, class Op>
__device__ inline uint32_t row16_scatter_pairs(uint32_t (&w)[N / 2], int l16, Op op) {
  static_assert(N == 8 || N == 16, "8 or 16 combos");
  if constexpr (N == 16) {
    halve<0x140, 8>(w, (l16 & 8) != 0, op);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = op(w[k], dpp_u<0x140>(w[k]));
  }
  halve<0x141, 4>(w, (l16 & 4) != 0, op);
  halve<0x4E, 2>(w, (l16 & 2) != 0, op);
  const uint32_t r = op(w[0], dpp_u<0xB1>(w[0]));  // both halves over the whole row
  return (l16 & 1) ? r >> 16 : r & 0xffffu;
}

// Order-preserving signed 16-bit key of a 16-bit float's bits (FP16 or BF16:
// sign and magnitude): larger values give larger keys; and back.
__device__ inline uint32_t key16(uint32_t u) { return (u & 0x8000u) ? (u ^ 0x7FFFu) : u; }
__device__ inline uint32_t unkey16(uint32_t k) { k &= 0xFFFFu; return (k & 0x8000u) ? (k ^ 0x7FFFu) : k; }
template <bool BF>
__device__ inline float bits16_to_float(uint32_t u) {
  if constexpr (BF) return __builtin_bit_cast(float, u << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)u);
}
__device__ inline uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  typedef short s2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s2, a), __builtin_bit_cast(s2, b)));
}
// bits of element i (0..7) of a 16-byte chunk of 16-bit codes
__device__ inline uint32_t chunk_bits(const u4& x, int i) {
  const uint32_t w = x[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// max (and exact float64 sums of 16-bit magnitudes) over lanes l, l^16, l^32,
// l^48 by the row swaps of gfx950 (no LDS)
template <int ROWS>
__device__ inline void swap_rows_u(uint32_t x, uint32_t& a, uint32_t& b) {
  if constexpr (ROWS == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0]; b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0]; b = r[1];
  }
  asm volatile("" : "+v"(a), "+v"(b));
}
__device__ inline float rows4_max_sw(float x) {
  uint32_t a, b;
  swap_rows_u<16>(__builtin_bit_cast(uint32_t, x), a, b);
  x = fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
  swap_rows_u<32>(__builtin_bit_cast(uint32_t, x), a, b);
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ inline double rows4_sum_sw(double x) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    uint32_t la, lb, ha, hb;
    if (r == 0) {
      swap_rows_u<16>((uint32_t)u, la, lb);
      swap_rows_u<16>((uint32_t)(u >> 32), ha, hb);
    } else {
      swap_rows_u<32>((uint32_t)u, la, lb);
      swap_rows_u<32>((uint32_t)(u >> 32), ha, hb);
    }
    x = __builtin_bit_cast(double, (uint64_t)la | ((uint64_t)ha << 32)) +
        __builtin_bit_cast(double, (uint64_t)lb | ((uint64_t)hb << 32));
  }
  return x;
}

// element i (0..7) of a 16-byte chunk of 16-bit codes (BF16 or FP16), as float
template <bool BF>
__device__ inline float chunk_elem(const u4& x, int i) {
  const uint32_t w = x[i >> 1];
  if constexpr (BF) return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
}

// Source chunks of one unit: tile t, chunk c (elements 8c .. 8c+7 of the lane's
// destination run).
template <int D, int NT>
struct UnitSrc {
  static constexpr int NC = D / 32;
  u4 x[NT][NC];
};

template <int D, int NT>
__device__ inline void load_unit(UnitSrc<D, NT>& u, const uint8_t* sp, bool grouped_k, int lane) {
  constexpr int NC = D / 32;
  constexpr int RS = D / 2;  // 16-bit source run bytes
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint8_t* ts = sp + (size_t)t * 16 * D * 2;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint32_t off;
      if (grouped_k) {  // dims 32c + 8(lane/16) .. +7 of token lane%16, from the lane whose run holds them
        const int d0 = 32 * c + 8 * (lane >> 4);
        const int ls = 16 * (d0 / (D / 4)) + (lane & 15);
        off = run_byte(ls, 2 * (d0 % (D / 4)), RS);
      } else {
        off = run_byte(lane, 16 * c, RS);
      }
      // the source page is read once and the destination written once:
      // non-temporal on both sides (FP8 demotion 315-325 -> 299-300 us)
      u.x[t][c] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(ts + off));
    }
  }
}

// Encode one tile's destination run from the lane's eight-element source
// chunks x[c] (elements 8c .. 8c+7 of the run) and write it. Group
// parameters (INT scale s, its reciprocal r, INT2 offset z) come per chunk:
// gp(g, s, r, z) fills entry j = 0..3 for chunk g, and element 8g + k uses
// entry k % 4 (for V runs: token 4(lane/16) + k % 4, group g; grouped K runs
// fill every j alike). They are fetched when the chunk is encoded, so a V
// run's 16 groups need not stay in registers across the tile.
template <int D, int DC, bool BF, class GP>
__device__ inline void store_run(const u4* x, GP&& gp, float s8, float r8, bool fast8, uint8_t* td, int lane) {
  constexpr int BITS = wbits(DC);
  constexpr int E = D / 4, RD = D * BITS / 32;
  constexpr int NWD = RD < 4 ? 1 : RD / 4;
  constexpr float QMAX = DC == W_INT8 ? 127.0f : 7.0f;
  uint32_t word[NWD];
#pragma unroll
  for (int k = 0; k < NWD; ++k) word[k] = 0;
  if constexpr (DC == W_FP8) {
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const float v0 = chunk_elem<BF>(x[e >> 3], e & 7), v1 = chunk_elem<BF>(x[e >> 3], (e + 1) & 7);
      const float q0 = fast8 ? recip_div0(v0, s8, r8) : __fdiv_rn(v0, s8);
      const float q1 = fast8 ? recip_div0(v1, s8, r8) : __fdiv_rn(v1, s8);
      const float y0 = fminf(fmaxf(q0, -448.0f), 448.0f);
      const float y1 = fminf(fmaxf(q1, -448.0f), 448.0f);
      if ((e >> 1) & 1)
        word[e >> 2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)word[e >> 2], true);
      else
        word[e >> 2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, (int)word[e >> 2], false);
    }
  } else if constexpr (DC == W_INT8 || DC == W_INT4) {
    // code = clip(rint(x / s), +-qmax): the quotient clamped (a median of
    // three, exact: the bounds are integers), then 1.5 * 2^23 added, which
    // rounds it to the nearest integer with ties to even (as rint) and leaves
    // that integer's two's complement in the low bits of the sum
    constexpr float MAGIC = 12582912.0f;
#pragma unroll
    for (int g = 0; g < E / 8; ++g) {
      float s[4], r[4], z[4];
      gp(g, s, r, z);
      uint32_t cw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float q = __builtin_amdgcn_fmed3f(recip_div0(chunk_elem<BF>(x[g], k), s[k & 3], r[k & 3]), -QMAX, QMAX);
        cw[k] = __builtin_bit_cast(uint32_t, q + MAGIC);
      }
      if constexpr (DC == W_INT8) {
        // bytes in element order: elements 4k .. 4k+3 in word k
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t lo = __builtin_amdgcn_perm(cw[4 * h + 1], cw[4 * h], 0x0C0C0400u);
          const uint32_t hi = __builtin_amdgcn_perm(cw[4 * h + 3], cw[4 * h + 2], 0x04000C0Cu);
          word[2 * g + h] = lo | hi;
        }
      } else {
        // eight codes per word: element 2m at bits 4m, element 2m + 1 at 16 + 4m
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t pr = __builtin_amdgcn_perm(cw[2 * m + 1], cw[2 * m], 0x0C040C00u) & 0x000F000Fu;
          word[g] |= pr << (4 * m);
        }
      }
    }
  } else if constexpr (DC == W_INT2) {
#pragma unroll
    for (int g = 0; g < E / 8; ++g) {
      float s[4], r[4], z[4];
      gp(g, s, r, z);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        put_code<BITS, E>(word, 8 * g + k, affine2_code_r(chunk_elem<BF>(x[g], k), z[k & 3], s[k & 3], r[k & 3]));
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = chunk_elem<BF>(x[e >> 3], e & 7);
      uint32_t code;
      if constexpr (DC == W_FP16) {
        code = __builtin_bit_cast(uint16_t, (_Float16)v);
      } else if constexpr (DC == W_BF16) {
        code = f_to_bf16(v);
      } else {
        static_assert(DC == W_BIT1, "INT8, INT4 and INT2 codes are made above");
        code = v < 0.f ? 1u : 0u;
      }
      put_code<BITS, E>(word, e, code);
    }
  }
  store_run_words<RD, true>(td, word, lane);
}

// DK: the destination codec pair (K low nibble, V high nibble) the kernel is
// specialised for (FP8/FP8, INT2/INT2, BIT1/BIT1), else -1 (any pair of FP16,
// BF16, FP8, INT8 and INT4, chosen per plane at run time) or -2 (any other
// pair with an INT2 or BIT1 plane: their reductions and packing are built only
// here and in the two sub-byte specialisations, so the other kernels keep
// their registers). A call has one destination pair. (An INT8/INT4
// specialisation held as many registers as the generic kernel and is not
// built.)
// Waves per SIMD the register kernels are compiled for, where a unit holds at
// most 128 x 16 source elements (measured on demotions of 14,720 16-token
// pages at head_dim 128: the generic kernel at four waves 300-309 us against
// 344-352 at three, INT2/INT2 at four 347-365 us against 364-369 at three,
// BIT1/BIT1 at four 275-284 us against 298-309 at three). Larger units keep
// the compiler's choice.
template <int D, int NT, int DK>
__host__ __device__ constexpr int enc_waves() {
  if (D * NT > 128) return 1;
  if (DK == -1 || DK == (W_INT2 | W_INT2 << 4) || DK == (W_BIT1 | W_BIT1 << 4)) return 4;
  return 1;
}
template <int D, int NT, int DK>
__global__ void __launch_bounds__(64 * EW) __attribute__((amdgpu_waves_per_eu(enc_waves<D, NT, DK>()))) encode_reg_kernel(EncodeArgs a, int nunits) {
  constexpr int NC = D / 32;
  constexpr bool SUBK = DK == -2 || (DK >= 0 && (wsub(DK & 15) || wsub(DK >> 4)));  // builds the INT2/BIT1 paths
  // per wave, the group parameters of its V tile: [row][4 g + j] for group g
  // of the row's token j (chunk-major: one 16-byte read gives a chunk's four)
  __shared__ float sx[EW][4][16];  // INT scales
  __shared__ float rx[EW][4][16];  // their reciprocals RN(1 / s)
  __shared__ float zx[EW][4][16];  // INT2 offsets
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int gw = blockIdx.x * EW + wv, nw = gridDim.x * EW;
  const int P = a.page, hkv = a.hkv;
  const int kq = lane >> 4, l16 = lane & 15;

  auto unit_of = [&](int u, int& i, int& h, int& plane) {
    plane = u & 1;
    h = (u >> 1) % hkv;
    i = (u >> 1) / hkv;
  };
  // the next unit is prefetched while the current one is encoded when both fit
  // in registers (the FP8 kernel, free of the INT scale state, holds two
  // 64-token units at head_dim 128 in 224 VGPRs); larger units are loaded at
  // the start of their turn and other waves hide the latency
  // (INT2/INT2 and BIT1/BIT1 one-tile units at head_dim 128 go without it:
  // they fit four waves per SIMD without spills only so, and other waves
  // hide the load)
  constexpr bool SUB_PAIR = DK == (W_INT2 | W_INT2 << 4) || DK == (W_BIT1 | W_BIT1 << 4);
  constexpr bool PREFETCH = !(SUB_PAIR && D == 128 && NT == 1) &&
                            NT * NC <= (DK == (W_FP8 | W_FP8 << 4) ? 16 : 8);
  UnitSrc<D, NT> cur, nxt;
  int u = gw;
  bool have = false;
  int i = 0, h = 0, plane = 0, dst = 0, scodec = 0, dcodec = 0;
  uint64_t so = 0, dof = 0;
  bool ok = false;
  if (u < nunits) {
    unit_of(u, i, h, plane);
    ok = check_pair(a, i, plane, D, dst, scodec, dcodec, so, dof);
    if (DK >= 0) dcodec = plane ? DK >> 4 : DK & 15;
    if (ok) load_unit<D, NT>(cur, a.pool + so + (size_t)h * P * D * 2, wgrp(dcodec) && plane == 0, lane);
    have = true;
  }
  while (have) {
    // the next unit's checks and loads first
    const int un = u + nw;
    int i2 = 0, h2 = 0, plane2 = 0, dst2 = 0, scodec2 = 0, dcodec2 = 0;
    uint64_t so2 = 0, dof2 = 0;
    bool ok2 = false;
    const bool have2 = un < nunits;
    if (have2) {
      unit_of(un, i2, h2, plane2);
      ok2 = check_pair(a, i2, plane2, D, dst2, scodec2, dcodec2, so2, dof2);
      if (DK >= 0) dcodec2 = plane2 ? DK >> 4 : DK & 15;
      if (PREFETCH && ok2) load_unit<D, NT>(nxt, a.pool + so2 + (size_t)h2 * P * D * 2, wgrp(dcodec2) && plane2 == 0, lane);
    }

    if (!ok) {
      if (h == 0 && plane == 0 && lane == 0) count_err(a.err);
    } else {
      // the unit's work, compiled once per source codec (the choice is per unit)
      const int dcodec_unit = dcodec;
      auto work = [&](auto bf_tag) {
        constexpr bool BF = decltype(bf_tag)::value;
        const bool is_v = plane == 1;
        const int dcodec = DK >= 0 ? (is_v ? DK >> 4 : DK & 15) : dcodec_unit;  // one of two constants when specialised
        const int dbits = wbits(dcodec);
        uint8_t* dp = a.pool + dof + (size_t)h * P * D * dbits / 8;
        // FP8: absmax of the whole (page, head, plane) block
        float s8 = 1.f;
        if (dcodec == W_FP8) {
          float m = 0.f;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
              for (int k = 0; k < 8; ++k) m = fmaxf(m, __builtin_fabsf(chunk_elem<BF>(cur.x[t][c], k)));
          m = rows4_max_sw(row16_max(m));
          s8 = m == 0.f ? 1.f : __fdiv_rn(m, 448.0f);
        }
        const float r8 = __fdiv_rn(1.0f, s8);
        const bool fast8 = s8 >= 0x1p-100f;  // smaller scales keep the correctly rounded division
        // the conversions of the absmax pass are recomputed below, not kept
        // live across it (an empty asm hides the chunks' values)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(cur.x[t][c]));
        if (lane == 0 && a.scale) a.scale[((size_t)dst * hkv + h) * 2 + plane] = s8;
        if (h == 0 && plane == 0 && lane == 0) a.codec_out[dst] = (uint8_t)a.dst_codec;
        const float qmax = dcodec == W_INT8 ? 127.0f : 7.0f;
        const float rqmax = dcodec == W_INT8 ? 1.0f / 127.0f : 1.0f / 7.0f;  // RN(1 / qmax), folded
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const u4* x = cur.x[t];
          float s2[4][NC], r2[4][NC], z2[4][NC];
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < NC; ++g) s2[j][g] = r2[j][g] = 1.f, z2[j][g] = 0.f;
          if (SUBK && wsub(dcodec)) {
            // INT2 (offset and step per group) and BIT1 (mean magnitude per group)
            const size_t sc_base = (size_t)hkv * P * D * dbits / 8 + ((size_t)h * P + 16 * t) * NC * 2;
            const size_t zgap = (size_t)hkv * P * NC * 2;
            const bool aff = dcodec == W_INT2;
            if (is_v) {
              // group g of token 4kq + j: elements 8g + j and 8g + 4 + j on the 16 lanes of row kq;
              // lane l16 < 4 NC of each row keeps combo (j, g) = (l16 / NC, l16 % NC)
              // all 4 NC combos reduced together over the row (reduce-scatter)
              constexpr int NCB = 4 * NC;
              float mine_s = 1.f, mine_z = 0.f;
              if (aff) {
                // max and min at once: keys of x (low half) and of -x (high half)
                uint32_t kw[NCB];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                  for (int g = 0; g < NC; ++g) {
                    const uint32_t u0 = chunk_bits(x[g], j), u1 = chunk_bits(x[g], 4 + j);
                    kw[j * NC + g] = pk_max_i16(key16(u0) | (key16(u0 ^ 0x8000u) << 16),
                                                key16(u1) | (key16(u1 ^ 0x8000u) << 16));
                  }
                const uint32_t r = row16_scatter<NCB>(kw, l16, pk_max_i16);
                affine2_params(-bits16_to_float<BF>(unkey16(r >> 16)), bits16_to_float<BF>(unkey16(r)), mine_z, mine_s);
              } else {
                // fp64 sums of the pairs, reduced eight combos at a time (tokens
                // 4kq, 4kq + 1, then 4kq + 2, 4kq + 3 at head_dim 128): the
                // same lane pairs in the same order as one 16-combo reduction,
                // with half the sums live
                auto add = [](double a, double b) { return a + b; };
                double r[NCB / 8];
#pragma unroll
                for (int h = 0; h < NCB / 8; ++h) {
                  double sm[8];
#pragma unroll
                  for (int c = 0; c < 8; ++c) {
                    const int j = (8 * h + c) / NC, g = (8 * h + c) % NC;
                    sm[c] = (double)__builtin_fabsf(chunk_elem<BF>(x[g], j)) +
                            (double)__builtin_fabsf(chunk_elem<BF>(x[g], 4 + j));
                  }
                  r[h] = row16_scatter<8>(sm, l16, add);
                }
                mine_s = sign1_scale(NCB == 16 && (l16 & 8) ? r[NCB / 8 - 1] : r[0]);
              }
              if (l16 < 4 * NC) {
                const int j = l16 / NC, g = l16 % NC;
                sx[wv][kq][4 * g + j] = mine_s;
                zx[wv][kq][4 * g + j] = mine_z;
                if (aff) rx[wv][kq][4 * g + j] = recip_fp16_scale(mine_s);
                const size_t at = sc_base + ((size_t)(4 * kq + j) * NC + g) * 2;
                *reinterpret_cast<_Float16*>(a.pool + dof + at) = (_Float16)mine_s;
                if (aff) *reinterpret_cast<_Float16*>(a.pool + dof + at + zgap) = (_Float16)mine_z;
              }
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            } else {
              // grouped K: chunk c is group c of token lane%16, spread over the 4 rows
#pragma unroll
              for (int c = 0; c < NC; ++c) {
                float sv = 1.f, zv = 0.f;
                if (aff) {
                  float lo = chunk_elem<BF>(x[c], 0), hi = lo;
#pragma unroll
                  for (int k = 1; k < 8; ++k) {
                    lo = fminf(lo, chunk_elem<BF>(x[c], k));
                    hi = fmaxf(hi, chunk_elem<BF>(x[c], k));
                  }
                  affine2_params(-rows4_max_sw(-lo), rows4_max_sw(hi), zv, sv);
                } else {
                  double m = 0.0;
#pragma unroll
                  for (int k = 0; k < 8; ++k) m += (double)__builtin_fabsf(chunk_elem<BF>(x[c], k));
                  sv = sign1_scale(rows4_sum_sw(m));
                }
                const float rv = aff ? recip_fp16_scale(sv) : 1.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  s2[j][c] = sv;
                  z2[j][c] = zv;
                  r2[j][c] = rv;
                }
                if (kq == (c & 3) && (NC == 4 || kq < NC)) {
                  const size_t at = sc_base + ((size_t)l16 * NC + c) * 2;
                  *reinterpret_cast<_Float16*>(a.pool + dof + at) = (_Float16)sv;
                  if (aff) *reinterpret_cast<_Float16*>(a.pool + dof + at + zgap) = (_Float16)zv;
                }
              }
            }
          }
          if (wint(dcodec)) {
            const size_t sc_base = (size_t)hkv * P * D * dbits / 8 + ((size_t)h * P + 16 * t) * NC * 2;
            auto scale_of = [&](float m) {  // fp16 scale kept inside fp16's finite range
              _Float16 s16 = (_Float16)recip_div(m, qmax, rqmax);  // = RN(m / qmax)
              s16 = s16 == (_Float16)0.0f ? __builtin_bit_cast(_Float16, (uint16_t)0x0001) : s16;
              s16 = s16 > (_Float16)65504.0f ? (_Float16)65504.0f : s16;
              return m == 0.f ? (_Float16)1.0f : s16;
            };
            if (is_v) {
              // group g of token 4kq + j: elements 8g + j and 8g + 4 + j on the 16 lanes of row kq;
              // lane l16 < 4 NC of each row computes combo (j, g) = (l16 / NC, l16 % NC)
              // magnitudes' bits (order-preserving), two combos to a word, all
              // reduced together over the row
              constexpr int NCB = 4 * NC;
              uint32_t kw[NCB / 2];
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) {
                const int j = cb / NC, g = cb % NC;
                const uint32_t a0 = chunk_bits(x[g], j) & 0x7FFFu, a1 = chunk_bits(x[g], 4 + j) & 0x7FFFu;
                const uint32_t m = a0 > a1 ? a0 : a1;
                kw[cb >> 1] = (cb & 1) ? (kw[cb >> 1] | (m << 16)) : m;
              }
              const float mine = bits16_to_float<BF>(row16_scatter_pairs<NCB>(kw, l16, pk_max_i16));
              if (l16 < 4 * NC) {
                const _Float16 s16 = scale_of(mine);
                const int j = l16 / NC, g = l16 % NC;
                sx[wv][kq][4 * g + j] = (float)s16;
                rx[wv][kq][4 * g + j] = recip_fp16_scale((float)s16);
                *reinterpret_cast<_Float16*>(a.pool + dof + sc_base + ((size_t)(4 * kq + j) * NC + g) * 2) = s16;
              }
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            } else {
              // grouped K: chunk c is group c of token lane%16, spread over the 4 rows
#pragma unroll
              for (int c = 0; c < NC; ++c) {
                float m = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) m = fmaxf(m, __builtin_fabsf(chunk_elem<BF>(x[c], k)));
                m = rows4_max_sw(m);
                const _Float16 s16 = scale_of(m);
                const float sf = (float)s16, rf = recip_fp16_scale(sf);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  s2[j][c] = sf;
                  r2[j][c] = rf;
                }
                if (kq == (c & 3) && (NC == 4 || kq < NC))
                  *reinterpret_cast<_Float16*>(a.pool + dof + sc_base + ((size_t)l16 * NC + c) * 2) = s16;
              }
            }
          }
          uint8_t* td = dp + (size_t)t * 16 * D * dbits / 8;
          // group parameters of chunk g: a V tile's from its wave's LDS rows,
          // a grouped K tile's from the lane's registers
          auto gp = [&](int g, float (&gs)[4], float (&gr)[4], float (&gz)[4]) {
            if (is_v) {
              const float4 vs = *reinterpret_cast<const float4*>(&sx[wv][kq][4 * g]);
              const float4 vr = *reinterpret_cast<const float4*>(&rx[wv][kq][4 * g]);
              const float4 vz = *reinterpret_cast<const float4*>(&zx[wv][kq][4 * g]);
              gs[0] = vs.x; gs[1] = vs.y; gs[2] = vs.z; gs[3] = vs.w;
              gr[0] = vr.x; gr[1] = vr.y; gr[2] = vr.z; gr[3] = vr.w;
              gz[0] = vz.x; gz[1] = vz.y; gz[2] = vz.z; gz[3] = vz.w;
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) gs[j] = s2[j][g], gr[j] = r2[j][g], gz[j] = z2[j][g];
            }
          };
          const bool sub = SUBK && wsub(dcodec);
          if (sub) {
            if constexpr (SUBK) {
              if (dcodec == W_INT2) store_run<D, W_INT2, BF>(x, gp, s8, r8, fast8, td, lane);
              else store_run<D, W_BIT1, BF>(x, gp, s8, r8, fast8, td, lane);
            }
          } else {
            switch (dcodec) {
              case W_FP16: store_run<D, W_FP16, BF>(x, gp, s8, r8, fast8, td, lane); break;
              case W_BF16: store_run<D, W_BF16, BF>(x, gp, s8, r8, fast8, td, lane); break;
              case W_FP8: store_run<D, W_FP8, BF>(x, gp, s8, r8, fast8, td, lane); break;
              case W_INT8: store_run<D, W_INT8, BF>(x, gp, s8, r8, fast8, td, lane); break;
              default: store_run<D, W_INT4, BF>(x, gp, s8, r8, fast8, td, lane); break;
            }
          }
          // the V parameters are read above before the next tile or unit
          // writes its own (same wave, in order; the fence orders the compiler)
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      };
      if (scodec == W_BF16) work(std::integral_constant<bool, true>{});
      else work(std::integral_constant<bool, false>{});
    }
    have = have2;
    u = un;
    i = i2; h = h2; plane = plane2; dst = dst2; scodec = scodec2; dcodec = dcodec2; so = so2; dof = dof2; ok = ok2;
    if constexpr (PREFETCH) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) cur.x[t][c] = nxt.x[t][c];
    } else if (have && ok) {
      load_unit<D, NT>(cur, a.pool + so + (size_t)h * P * D * 2, wgrp(dcodec) && plane == 0, lane);
    }
  }
}

}  // namespace

int launch_append(const AppendArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  hipLaunchKernelGGL(append_kernel, dim3(a.rows, a.hkv, 2), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

namespace {

// a destination pair with an INT2 or BIT1 plane
bool sub_byte_dst(int dst_codec) {
  const int k = dst_codec & 15, v = (dst_codec >> 4) & 15;
  return k == W_INT2 || k == W_BIT1 || v == W_INT2 || v == W_BIT1;
}
// Whether such a pair takes the register path for units of NT tiles: its
// tile loop, with the INT2/BIT1 reductions, unrolls (and the unit stays in
// registers) up to 16 chunks of 16 bytes per lane; larger units are staged
// through LDS.
constexpr bool sub_reg_path(int D, int NT) { return NT * D / 32 <= 8; }

template <int D, int NT>
void launch_encode_reg(const EncodeArgs& a, hipStream_t s) {
  const int nunits = a.n * a.hkv * 2;
  int wgs = (nunits + EW - 1) / EW;
  // Waves loop over the units past the grid, prefetching the next one.
  // Measured caps: the FP8 kernel (two waves per SIMD, 512 workgroups
  // resident) is fastest with three rounds of them, the generic kernel with
  // 4,096 workgroups.
  const bool fp8 = a.dst_codec == (W_FP8 | W_FP8 << 4);
  const int cap = fp8 ? 1536 : 4096;
  if (wgs > cap) wgs = cap;
  if (fp8) {
    hipLaunchKernelGGL((encode_reg_kernel<D, NT, W_FP8 | W_FP8 << 4>), dim3(wgs), dim3(64 * EW), 0, s, a, nunits);
  } else if (sub_byte_dst(a.dst_codec)) {
    // the uniform INT2 and BIT1 pairs compile their own path alone (fewer
    // registers, more waves per SIMD than the kernel for any sub-byte pair)
    constexpr int I2 = W_INT2 | W_INT2 << 4, B1 = W_BIT1 | W_BIT1 << 4;
    if constexpr (sub_reg_path(D, NT)) {
      if (a.dst_codec == I2)
        hipLaunchKernelGGL((encode_reg_kernel<D, NT, I2>), dim3(wgs), dim3(64 * EW), 0, s, a, nunits);
      else if (a.dst_codec == B1)
        hipLaunchKernelGGL((encode_reg_kernel<D, NT, B1>), dim3(wgs), dim3(64 * EW), 0, s, a, nunits);
      else
        hipLaunchKernelGGL((encode_reg_kernel<D, NT, -2>), dim3(wgs), dim3(64 * EW), 0, s, a, nunits);
    }
  } else {
    hipLaunchKernelGGL((encode_reg_kernel<D, NT, -1>), dim3(wgs), dim3(64 * EW), 0, s, a, nunits);
  }
}

}  // namespace

int launch_encode(const EncodeArgs& a, void* stream) {
  if (a.n == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int tiles = a.page / 16;  // page is a multiple of 16
  if (a.head_dim != 64 && a.head_dim != 128) return -2;
  const bool staged_sub = sub_byte_dst(a.dst_codec) && !(tiles <= 4 && sub_reg_path(a.head_dim, tiles));
  if (tiles <= 4 && !staged_sub && (long long)a.n * a.hkv * 2 <= 0x7fffffff) {
    // register path: one wave per (pair, head, plane)
#define PKV_REG(DD)                                                   \
  if (tiles == 4) launch_encode_reg<DD, 4>(a, s);                     \
  else if (tiles == 3) launch_encode_reg<DD, 3>(a, s);                \
  else if (tiles == 2) launch_encode_reg<DD, 2>(a, s);                \
  else launch_encode_reg<DD, 1>(a, s);
    if (a.head_dim == 64) {
      PKV_REG(64)
    } else {
      PKV_REG(128)
    }
#undef PKV_REG
    return hipGetLastError() == hipSuccess ? 0 : -4;
  }
  // longer pages: staged through LDS, four tiles at a time
  const dim3 grid(a.n, a.hkv, 2);
  const bool sub = sub_byte_dst(a.dst_codec);
  if (a.head_dim == 64) {
    if (sub) hipLaunchKernelGGL((encode_kernel<64, 4, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((encode_kernel<64, 4, false>), grid, dim3(256), 0, s, a);
  } else {
    if (sub) hipLaunchKernelGGL((encode_kernel<128, 4, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((encode_kernel<128, 4, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
