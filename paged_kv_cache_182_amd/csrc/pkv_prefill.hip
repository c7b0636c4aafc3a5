// Chunked-prefill attention over the mixed-codec paged cache, gfx950, and
// the log-sum-exp fold of one window's result into an accumulator.
//
// A chunk of T new query tokens per row has been appended to the cache; query
// t sits at position L - T + t and attends, causally, the cached keys up to
// its own position, restricted to a key window [kv_begin, kv_end) and, with a
// sliding window of W, to its last W positions (ARGUS v0.5: sliding-window
// masks). The key
// range is cut into partitions attended in parallel and folded by their
// log-sum-exp (FreeToken PR #499 discussion, in-place host K/V design: a
// prefill attends window by window and folds the windows into an fp32
// accumulator; ARGUS "Why decode is slow" for grouped-query attention).
//
// Work unit: one workgroup of four waves owns (partition, KV head, row, group
// of 128 query columns), a column being one (query token, query head of the
// KV head's group) pair; each wave owns 16 NBC (32) columns. The partition's 16-token
// tiles go two at a time: each pair is converted once, by the whole
// workgroup, from its page codes into an fp16 image in LDS (double-buffered,
// one barrier per pair); each wave then reads the image as MFMA operands:
//  * scores: v_mfma_f32_16x16x32_f16 per tile, A = K (row = token, 8 dims
//    per lane), B = q^T (col = query column); lane l gets tokens 4*(l/16) + j
//    of column l % 16. The K image keeps dims in natural order: step c of
//    lane l holds dims 32c + 8(l/16) .. +7, so one 32-dim step is one INT
//    scale group.
//  * one online-softmax update per pair, over the lane's eight scores.
//  * P.V: v_mfma_f32_16x16x32_f16, A = P (the lane's four scores of each
//    tile), B = V (the same tokens of one dim; the V layout of every codec
//    gives a lane those four tokens, so the pair image interleaves the two
//    tiles' runs).
// Codes convert to fp16 exactly, and scales stay in fp32: FP8 K scales
// multiply the scores, INT K group scales weight one score accumulator per
// group, INT V group scales multiply the weights per group (fp16 scales, so a
// weight of 1 stays exact), and the FP8 V page scale s enters the softmax in
// the log domain: log2|s| is added to the tile's scores (the weights then
// carry it; the largest weight stays exactly 1), the weights' sum takes 1/|s|
// and the sign of s flips the tile's weights. So no accumulator is rescaled
// when the page scale changes.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

enum : int { C_FP16 = 0, C_BF16 = 1, C_FP8 = 2, C_INT8 = 3, C_INT4 = 4, C_INT2 = 5, C_BIT1 = 6, C_ANY = 15 };

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int NBC = 2;                    // 16-column blocks per wave
constexpr int COLS = 16 * NBC * WAVES;    // query columns per workgroup
constexpr int PAIR_RING = 1;              // tile pairs of codes in flight per thread
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LN2 = 0.693147180559945309f;

// code width: FP16 and BF16 16 bits, FP8 and INT8 8, INT4 4, INT2 2, BIT1 1
// (log2 of it, three bits per codec, in one constant)
__host__ __device__ constexpr int bits_of(int c) { return 1 << ((0xa6e4u >> (3 * c)) & 7u); }
// one fp16 scale per (token, 32 dims): INT8, INT4, INT2, BIT1
__host__ __device__ constexpr bool is_int(int c) { return c >= C_INT8 && c <= C_BIT1; }
// INT2 (unsigned affine) also holds one fp16 offset per (token, 32 dims)
__host__ __device__ constexpr bool has_zero(int c) { return c == C_INT2; }

__device__ inline uint64_t plane_bytes(int c, int hkv, int page, int d) {
  const uint64_t codes = (uint64_t)hkv * page * d * bits_of(c) / 8;
  const uint64_t groups = (uint64_t)hkv * page * (d / 32) * 2;
  return codes + (is_int(c) ? groups : 0) + (has_zero(c) ? groups : 0);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9-family raw buffer format
constexpr int CPOL_NT = 2;              // non-temporal
constexpr uint32_t OFF_NONE = 0xFFFFFF00u;

__device__ inline rsrc_t make_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, RSRC_WORD3);
}

__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- codes -> fp16
__device__ inline h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }

// bf16 operands. The codes of a BF16 page are not converted: they go to the
// bf16 MFMA as they are, against the query and the softmax weights split in
// bf16 high and low parts, so every product is exact and bf16's whole range
// is kept (ARGUS v0.5: FP16/BF16 direct attention).
__device__ inline f4 mfma32_bf(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}
// Eight fp16 query values as bf16: the high parts (the top 8 of the 11
// significant bits, by truncation) and the low parts (the remaining 3 bits,
// exact in bf16, whose exponent range holds fp16's subnormals).
__device__ inline u4 bf_hi8(h8 x) {
  u4 hi;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __builtin_bit_cast(uint32_t, (float)x[2 * i]), b = __builtin_bit_cast(uint32_t, (float)x[2 * i + 1]);
    hi[i] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
  return hi;
}
__device__ inline u4 bf_lo8(h8 x) {
  u4 lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = (float)x[2 * i], b = (float)x[2 * i + 1];
    const float ra = a - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xffff0000u);
    const float rb = b - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, b) & 0xffff0000u);
    lo[i] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, rb), __builtin_bit_cast(uint32_t, ra), 0x07060302u);
  }
  return lo;
}
// Eight fp32 softmax weights as bf16 high (truncated) and low (the remainder,
// rounded to nearest) parts: 16 significant bits.
__device__ inline void bf_split_w8(const float* p, u4& hi, u4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = p[2 * i], b = p[2 * i + 1];
    const uint32_t ha = __builtin_bit_cast(uint32_t, a) & 0xffff0000u, hb = __builtin_bit_cast(uint32_t, b) & 0xffff0000u;
    const __bf16 la = (__bf16)(a - __builtin_bit_cast(float, ha)), lb = (__bf16)(b - __builtin_bit_cast(float, hb));
    hi[i] = __builtin_amdgcn_perm(hb, ha, 0x07060302u);
    lo[i] = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
  }
}

template <bool HI>
__device__ inline uint32_t fp8x2_to_h2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// four int8 codes -> four fp16 (two words): 0x64XX is 1024 + XX, XX = code + 128
__device__ inline u2 int8x4_to_h4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off;
  const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off;
  return u2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}

// eight int4 codes of one word (element r in nibble slot (r%2)*4 + r/2) ->
// eight fp16 in element order. Masking a nibble under the fp16 pattern of
// 1024 and flipping its top bit gives 1024 + (c + 8) or 1024 + 16 (c + 8).
__device__ inline u4 int4x8_to_h8(uint32_t w) {
  const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 off16 = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t u8 = w >> 8;
  const h2 o0 = as_h2((w & 0x000f000fu) ^ 0x64086408u) - off;
  const h2 o1 = __builtin_elementwise_fma(as_h2((w & 0x00f000f0u) ^ 0x64806480u), s16, -off16);
  const h2 o2 = as_h2((u8 & 0x000f000fu) ^ 0x64086408u) - off;
  const h2 o3 = __builtin_elementwise_fma(as_h2((u8 & 0x00f000f0u) ^ 0x64806480u), s16, -off16);
  return u4{__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1), __builtin_bit_cast(uint32_t, o2),
            __builtin_bit_cast(uint32_t, o3)};
}

// Run words of the sub-byte codecs hold 16 (INT2) or 32 (BIT1) elements, the
// even ones in the low half-word and the odd ones in the high half-word, each
// half in element order; a BIT1 run of head_dim 64 is a 16-bit unit (even
// elements in its low byte), spread here to the two half-words.
__device__ inline uint32_t spread16(uint32_t u) { return (u & 0xffu) | ((u & 0xff00u) << 8); }
// two unsigned 2-bit codes at bits s, s+1 and 16+s, 17+s -> fp16 pair (exact)
__device__ inline uint32_t u2pair(uint32_t w, int s) {
  const h2 off = {(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_bit_cast(uint32_t, as_h2(((w >> s) & 0x00030003u) | 0x64006400u) - off);
}
// two sign codes at bits k and 16+k -> fp16 pair of +-1 (bit set: -1)
__device__ inline uint32_t b1pair(uint32_t w, int k) { return ((w << (15 - k)) & 0x80008000u) | 0x3C003C00u; }
// elements 8c .. 8c+7 of a run (job c) from the run word holding them
__device__ inline u4 int2x8_to_h8(uint32_t w, int c) {
  const int s0 = 8 * (c & 1);
  return u4{u2pair(w, s0), u2pair(w, s0 + 2), u2pair(w, s0 + 4), u2pair(w, s0 + 6)};
}
__device__ inline u4 bit1x8_to_h8(uint32_t w, int c) {
  return u4{b1pair(w, 4 * c), b1pair(w, 4 * c + 1), b1pair(w, 4 * c + 2), b1pair(w, 4 * c + 3)};
}
// the run word of a sub-byte job from its aligned 16-byte chunk
template <int D>
__device__ inline uint32_t sub_word(u4 x, uint32_t off, int bits) {
  const uint32_t k = (off >> 2) & 3;
  const uint32_t w = k == 0 ? x[0] : (k == 1 ? x[1] : (k == 2 ? x[2] : x[3]));
  if (D == 64 && bits == 1) return spread16(((off >> 1) & 1) ? w >> 16 : w & 0xffffu);
  return w;
}

// Eight consecutive run elements, raw (16, 8 or 4 bytes in the low words) ->
// eight fp16.
template <int C>
__device__ inline u4 to_h8_c(u4 r) {
  if constexpr (C == C_FP16) {
    return r;
  } else if constexpr (C == C_BF16) {
    return r;  // kept as bf16 codes: they feed the bf16 MFMA
  } else if constexpr (C == C_FP8) {
    return u4{fp8x2_to_h2<false>(r[0]), fp8x2_to_h2<true>(r[0]), fp8x2_to_h2<false>(r[1]), fp8x2_to_h2<true>(r[1])};
  } else if constexpr (C == C_INT8) {
    const u2 a = int8x4_to_h4(r[0]), b = int8x4_to_h4(r[1]);
    return u4{a[0], a[1], b[0], b[1]};
  } else {
    return int4x8_to_h8(r[0]);
  }
}
__device__ inline u4 to_h8(u4 r, int codec) {
  switch (codec) {
    case C_FP16: return r;
    case C_BF16: return r;  // kept as bf16 codes
    case C_FP8:
      return u4{fp8x2_to_h2<false>(r[0]), fp8x2_to_h2<true>(r[0]), fp8x2_to_h2<false>(r[1]),
                fp8x2_to_h2<true>(r[1])};
    case C_INT8: {
      const u2 a = int8x4_to_h4(r[0]), b = int8x4_to_h4(r[1]);
      return u4{a[0], a[1], b[0], b[1]};
    }
    default: return int4x8_to_h8(r[0]);
  }
}

// ---------------------------------------------------------------- tile staging
// Per-tile values every thread holds alike (wave-uniform, so scalar).
struct TileMeta {
  uint64_t koff, voff;  // plane offsets of the page (0 when dead)
  float sk;             // FP8 K scale of this KV head (1 otherwise)
  float sv;             // FP8 V scale as fp8_v_scale_word (64: none)
  int valid;            // tokens of the tile inside the row (0: dead tile)
  int kc, vc;
  int j0;               // position of the tile's first token
  int sub;              // tile of the page (j0 = page start + 16 sub)
};

// Page descriptor staged in LDS (32 bytes).
// The FP8 V page scale s as 64 + log2|s|, log2|s| clamped to [-40, 40], with
// the sign of s (64: no scale). Below 2^-40 a V value |code s| <= 448 |s|
// moves by less than 4.1e-10; scales above 2^40 are outside the supported
// domain (the encoder's lie in [2^-33, 147]). The clamp keeps every weight
// that matters next to the largest a normal fp32 number.
__device__ inline float fp8_v_scale_word(float s) {
  const float l = fminf(fmaxf(__builtin_amdgcn_logf(fabsf(s)), -40.f), 40.f);  // log2; -inf for 0 clamps
  return __builtin_copysignf(64.f + l, s);
}

struct PDesc {
  uint64_t k, v;   // plane offsets (0 if the page is skipped)
  float sk;        // FP8 K scale of this KV head (1 otherwise)
  float sv;        // FP8 V scale as fp8_v_scale_word (64: none)
  int32_t valid;   // tokens of the page inside the row (0: skipped)
  int32_t codec;   // K codec | V codec << 4
};
constexpr int MAX_DESC = 256;  // page descriptors staged at a time

// Raw codes of one tile held by one thread: its K and V jobs (eight elements
// each) and, for a few threads, 16 bytes of INT group scales.
template <int D>
struct Raw {
  static constexpr int JOBS = D / 64;  // jobs per thread (K and V jobs together)
  u4 x[JOBS];                          // the aligned 16-byte chunk of each job
  uint32_t off[JOBS];                  // byte offset of the job's run bytes
  u4 sc;
};

// Byte offset inside a tile of run byte rb of lane L (R run bytes).
__device__ inline uint32_t run_byte(int L, int rb, int R) {
  return R >= 16 ? (uint32_t)((rb >> 4) * 1024 + 16 * L + (rb & 15)) : (uint32_t)(R * L + rb);
}

// Every job issues the same single 16-byte load (the aligned chunk holding its
// bytes; 8- and 4-byte runs share the chunk with a neighbour lane's, so HBM
// traffic is unchanged), with no control flow around it: the wait counts
// stay exact and the next tile's loads stay in flight. `sel` picks the bytes.
__device__ inline u4 load_chunk(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off & ~15u), 0, CPOL_NT));
}
__device__ inline u4 select_bytes(u4 x, uint32_t off, int bits) {
  if (bits == 16) return x;
  if (bits == 8) return (off & 8) ? u4{x[2], x[3], 0u, 0u} : u4{x[0], x[1], 0u, 0u};
  const uint32_t k = (off >> 2) & 3;
  return u4{k == 0 ? x[0] : (k == 1 ? x[1] : (k == 2 ? x[2] : x[3])), 0u, 0u, 0u};
}

// Load job q of a thread: wave-level job wj = wave + WAVES*q picks the plane
// (K for wj < NC) and the run chunk c = wj % NC, the same for the whole wave,
// so the buffer resource stays uniform; lane L is the consuming lane. K jobs
// gather the eight dims 32c + 8(L/16) .. of token L%16 (natural order) from
// wherever the page's K layout keeps them; V jobs take run elements 8c ..
// 8c+7 of lane L (the V layout of every codec).
template <int D>
__device__ inline uint32_t job_offset(bool is_v, int c, int L, int codec) {
  const int bits = bits_of(codec);
  const int R = D * bits / 32;
  int Ls, e0;
  if (is_v || is_int(codec)) {
    Ls = L;
    e0 = 8 * c;
  } else {
    const int d0 = 32 * c + 8 * (L >> 4);
    Ls = 16 * (d0 / (D / 4)) + (L & 15);
    e0 = d0 % (D / 4);
  }
  return run_byte(Ls, e0 * bits / 8, R);
}

template <int D>
__device__ inline void issue(Raw<D>& raw, const TileMeta& m, const PrefillArgs& a, int h, int wave, int lane) {
  constexpr int NC = D / 32;
  const bool live = m.valid > 0;
  const int P = a.page;
  const rsrc_t rk = make_rsrc(a.pool + m.koff, live ? (uint32_t)plane_bytes(m.kc, a.hkv, P, D) : 0u);
  const rsrc_t rv = make_rsrc(a.pool + m.voff, live ? (uint32_t)plane_bytes(m.vc, a.hkv, P, D) : 0u);
  const int sub = m.sub;
  // INT group scales of the tile, 16 tokens x NC fp16 per plane, 16 bytes
  // per lane in lanes 0 .. 2NC-1: K scales in wave 0, V scales in wave 1, and
  // the INT2 offsets (laid out as the scales, after every head's scales) of
  // K in wave 2 and of V in wave 3
  {
    const bool sv = (wave & 1) != 0;
    const int codec = sv ? m.vc : m.kc;
    const uint32_t zgap = wave >= 2 ? (uint32_t)(a.hkv * P * NC * 2) : 0u;
    const uint32_t base = (uint32_t)((uint64_t)a.hkv * P * D * bits_of(codec) / 8) + zgap +
                          (uint32_t)((h * P + 16 * sub) * NC * 2) + 16 * lane;
    const bool want = lane < 2 * NC && (wave < 2 ? is_int(codec) : has_zero(codec));
    raw.sc = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(sv ? rv : rk, (int)(want ? base : OFF_NONE),
                                                                           0, 0));
  }
#pragma unroll
  for (int q = 0; q < Raw<D>::JOBS; ++q) {
    const int wj = wave + WAVES * q;
    const bool is_v = wj >= NC;
    const int c = is_v ? wj - NC : wj;
    const int codec = is_v ? m.vc : m.kc;
    const int bits = bits_of(codec);
    const uint32_t head = (uint32_t)(h * P * D * bits / 8) + (uint32_t)(sub * 16 * D * bits / 8);
    raw.off[q] = head + job_offset<D>(is_v, c, lane, codec);
    raw.x[q] = load_chunk(is_v ? rv : rk, raw.off[q]);
  }
}

// LDS image of one pair of tiles. K: one fp16 image per tile (chunk c of lane
// L at [c*64 + L]). V: the P.V operand of the pair, dims 16n .. 16n+15 of
// lane L at v[n][L]: tile A's four tokens 4(L/16) .. +3, then tile B's (the
// order of the weights). INT group scales as fp32 [tile][16 tokens][NC].
template <int D>
struct PairStage {
  static constexpr int IMG = 32 * D;  // bytes of one fp16 tile image (16 tokens x D)
  static constexpr int SCL = 16 * (D / 32);
  u4 k[2][IMG / 16];
  u4 v[D / 16][64];
  float ks[2][SCL];
  float vs[2][SCL];
  float kz[2][SCL];  // INT2 offsets (0 for the other codecs)
  float vz[2][SCL];
};

// Job c's eight elements (c: its 8-element chunk of the run) as fp16.
template <int C, int D>
__device__ inline u4 convert(u4 raw, uint32_t off, int codec, int c) {
  if constexpr (C == C_INT2) {
    return int2x8_to_h8(sub_word<D>(raw, off, 2), c);
  } else if constexpr (C == C_BIT1) {
    return bit1x8_to_h8(sub_word<D>(raw, off, 1), c);
  } else if constexpr (C == C_ANY) {
    if (codec == C_INT2) return int2x8_to_h8(sub_word<D>(raw, off, 2), c);
    if (codec == C_BIT1) return bit1x8_to_h8(sub_word<D>(raw, off, 1), c);
    return to_h8(select_bytes(raw, off, bits_of(codec)), codec);
  } else {
    return to_h8_c<C>(select_bytes(raw, off, bits_of(C)));
  }
}

// Zero the V values of tokens past the row (their bytes may be anything): run
// element e = 8c + i of lane L holds token 4(L/16) + i%4; word k holds
// elements 2k and 2k+1.
__device__ inline u4 mask_v_tail(u4 x, int valid, int lane) {
  if (valid >= 16) return x;
  const int nv = min(max(valid - 4 * (lane >> 4), 0), 4);
  const uint32_t m01 = nv >= 2 ? ~0u : (nv == 1 ? 0x0000ffffu : 0u);
  const uint32_t m23 = nv >= 4 ? ~0u : (nv == 3 ? 0x0000ffffu : 0u);
  return u4{x[0] & m01, x[1] & m23, x[2] & m01, x[3] & m23};
}

// INT group scales of one tile into LDS: lanes 0 .. 2NC-1 of wave 0 (K) and
// of wave 1 (V), zero past the row and 1 for the other codecs; INT2 offsets
// from waves 2 (K) and 3 (V), zero past the row and for the other codecs.
template <int D>
__device__ inline void stage_scales(const Raw<D>& raw, const TileMeta& m, float* ks, float* vs, float* kz,
                                    float* vz, int wave, int lane) {
  constexpr int NC = D / 32;
  if (lane < 2 * NC) {
    const bool sv = (wave & 1) != 0, zero = wave >= 2;
    const int codec = sv ? m.vc : m.kc;
    const bool has = zero ? has_zero(codec) : is_int(codec);
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = raw.sc[e >> 1];
      const uint16_t hbits = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
      const int tok = (8 * lane + e) / NC;
      f[e] = !has ? (zero ? 0.0f : 1.0f) : (tok < m.valid ? (float)__builtin_bit_cast(_Float16, hbits) : 0.0f);
    }
    float* dst = (zero ? (sv ? vz : kz) : (sv ? vs : ks)) + 8 * lane;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = f[e];
  }
}

// Convert the codes of a pair of tiles into the pair's LDS image. The thread
// holds the same jobs of both tiles, so it writes the interleaved V operand.
template <int D, int KC, int VC>
__device__ inline void produce_pair(const Raw<D>& ra, const Raw<D>& rb, const TileMeta& ma, const TileMeta& mb,
                                    PairStage<D>& st, int wave, int lane) {
  constexpr int NC = D / 32;
#pragma unroll
  for (int q = 0; q < Raw<D>::JOBS; ++q) {
    const int wj = wave + WAVES * q;
    const bool is_v = wj >= NC;
    const int c = is_v ? wj - NC : wj;
    if (is_v) {
      const u4 xa = mask_v_tail(convert<VC, D>(ra.x[q], ra.off[q], ma.vc, c), ma.valid, lane);
      const u4 xb = mask_v_tail(convert<VC, D>(rb.x[q], rb.off[q], mb.vc, c), mb.valid, lane);
      st.v[2 * c][lane] = u4{xa[0], xa[1], xb[0], xb[1]};
      st.v[2 * c + 1][lane] = u4{xa[2], xa[3], xb[2], xb[3]};
    } else {
      const u4 ka = convert<KC, D>(ra.x[q], ra.off[q], ma.kc, c), kb = convert<KC, D>(rb.x[q], rb.off[q], mb.kc, c);
      st.k[0][64 * c + lane] = ka;
      st.k[1][64 * c + lane] = kb;
    }
  }
  if constexpr (KC == C_ANY || VC == C_ANY || is_int(KC) || is_int(VC)) {
    stage_scales<D>(ra, ma, st.ks[0], st.vs[0], st.kz[0], st.vz[0], wave, lane);
    stage_scales<D>(rb, mb, st.ks[1], st.vs[1], st.kz[1], st.vz[1], wave, lane);
  }
}

__device__ inline f4 mfma32(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// Max and sum over lanes l, l^16, l^32, l^48 (the rows holding one column);
// the swap results are read from the builtin's vector and pinned by an empty
// asm so the optimizer cannot merge the two halves.
template <int ROWS>
__device__ inline void swap_rows(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  uint32_t lo, hi;
  if constexpr (ROWS == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    lo = r[0]; hi = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = r[0]; hi = r[1];
  }
  asm volatile("" : "+v"(lo), "+v"(hi));
  a = __builtin_bit_cast(float, lo);
  b = __builtin_bit_cast(float, hi);
}
__device__ inline float row4_max(float x) {
  float a, b;
  swap_rows<16>(x, a, b);
  swap_rows<32>(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ inline float row4_sum(float x) {
  float a, b;
  swap_rows<16>(x, a, b);
  swap_rows<32>(a + b, a, b);
  return a + b;
}

// Raw scores of one staged tile for the wave's NBC column blocks (lane l:
// tokens 4(l/16) + j of column l % 16), before the K scale. INT K: one
// accumulator per 32-dim group, weighted by the token's fp16 group scale;
// INT2 K adds each group's offset times the column's query sum over the
// group (qsum), the offset's share of the dot product.
// BF16 K (kbf): the codes against the query's bf16 high parts (qhi: qf holds
// them in the BF16 kernel; split from the fp16 query here otherwise) and low
// parts (the wave's LDS copy qlo, [block][chunk][lane]).
template <int D, bool QHI>
__device__ inline void tile_scores(const u4* kimg, const float* ks, const float* kz, bool kint, bool kzero, bool kbf,
                                   const h8 (&qf)[NBC][D / 32], const float (&qsum)[NBC][D / 32], const u4* qlo,
                                   int lane, f4 (&s)[NBC]) {
  constexpr int NC = D / 32;
  const int kq = lane >> 4;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  h8 kf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) kf[c] = __builtin_bit_cast(h8, kimg[64 * c + lane]);
  if (kbf) {
#pragma unroll
    for (int cb = 0; cb < NBC; ++cb) {
      f4 sa = zero;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u4 kr = __builtin_bit_cast(u4, kf[c]);
        const u4 qh = QHI ? __builtin_bit_cast(u4, qf[cb][c]) : bf_hi8(qf[cb][c]);
        sa = mfma32_bf(kr, qlo[(cb * NC + c) * 64 + lane], mfma32_bf(kr, qh, sa));
      }
      s[cb] = sa;
    }
    return;
  }
  if (kint) {
    float ksc[4][NC];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < NC; ++g) ksc[j][g] = ks[(4 * kq + j) * NC + g];
#pragma unroll
    for (int cb = 0; cb < NBC; ++cb) {
      f4 sg[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) sg[c] = mfma32(kf[c], qf[cb][c], zero);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) x += ksc[j][c] * sg[c][j];
        if (kzero) {
#pragma unroll
          for (int c = 0; c < NC; ++c) x += kz[(4 * kq + j) * NC + c] * qsum[cb][c];
        }
        s[cb][j] = x;
      }
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < NBC; ++cb) {
      f4 sa = zero;
#pragma unroll
      for (int c = 0; c < NC; ++c) sa = mfma32(kf[c], qf[cb][c], sa);
      s[cb] = sa;
    }
  }
}

// ---------------------------------------------------------------- kernel
// Waves per SIMD asked of the compiler (its minimum occupancy), as the host
// sizes the partitions: see prefill_waves_per_simd (the per-page dispatch
// variant, one, spilled at two at head_dim 64).
template <int D, int KC, int VC>
__host__ __device__ constexpr int prefill_waves() {
  return prefill_waves_per_simd(D, KC == C_ANY ? -1 : KC, VC == C_ANY ? -1 : VC);
}

template <int D, int KC, int VC>
__global__ void __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(prefill_waves<D, KC, VC>()))) prefill_kernel(const PrefillArgs a) {
  constexpr int NC = D / 32, NB = D / 16;
  __shared__ PairStage<D> stage[2];
  // BF16 K: the query's bf16 low parts, one copy per wave ([block][chunk][lane])
  constexpr bool KB = KC == C_BF16 || KC == C_ANY;
  __shared__ u4 qlo_lds[KB ? WAVES * NBC * NC * 64 : 1];
  __shared__ PDesc desc[MAX_DESC];

  // block -> (partition, column group): the column groups of one partition
  // sit 8 blocks apart, on one XCD (blocks are dealt round-robin over the 8
  // XCDs), so its pages are fetched into that XCD's L2 once.
  const int id = blockIdx.x;
  const int kk = id >> 3;
  const int cg = kk % a.col_groups;
  const int part = (kk / a.col_groups) * 8 + (id & 7);
  if (part >= a.nparts) return;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, kq = lane >> 4;
  const int G = a.group, T = a.tokens, P = a.page;
  const int ncols = T * G;
  // the last column group reaches the furthest keys, so it meets every page
  // any group of this partition reads: it alone reports page errors
  const bool reporter = h == 0 && cg == a.col_groups - 1;

  // ---- row extent
  // Errors are counted per thread and added once at the end.
  int nerr = 0;
  int L = a.seq_lens[b];
  const bool bad_row = L < 0 || (int64_t)L > (int64_t)a.max_pages * P;
  L = min(max(L, 0), a.max_pages * P);
  if (bad_row && part == 0 && tid == 0) ++nerr;

  // ---- key range of this partition, and of this workgroup's columns
  const int p_lo = max(a.part_base + part * a.part_tokens, a.kv_begin);
  const int p_hi = min(min(a.part_base + (part + 1) * a.part_tokens, a.kv_end), L);
  const int c_first = cg * COLS;
  const int c_last = min(c_first + COLS, ncols) - 1;  // >= c_first: the host launches no empty group
  const int wg_hi = min(p_hi, L - T + c_last / G + 1);
  // key limits of the column of query token t: [lo_of(t), hi_of(t))
  auto hi_of = [&](int t) { return min(p_hi, L - T + t + 1); };
  auto lo_of = [&](int t) { return a.window > 0 ? max(p_lo, L - T + t + 1 - a.window) : p_lo; };
  const int wg_lo = lo_of(c_first / G);
  // this wave's columns
  const int w_first = c_first + 16 * NBC * wave;
  const int w_last = min(w_first + 16 * NBC, ncols) - 1;
  const bool wave_live = w_first < ncols;
  const int w_hi_min = hi_of(w_first / G);
  const int w_hi_max = wave_live ? hi_of(w_last / G) : p_lo;
  const int w_lo_min = lo_of(w_first / G);
  const int w_lo_max = wave_live ? lo_of(w_last / G) : p_lo;

  // ---- q (B operand of the score MFMA), natural dim order
  h8 qf[NBC][NC];
  int hi_col[NBC], lo_col[NBC];  // key limits of the lane's column in each block
#pragma unroll
  for (int cb = 0; cb < NBC; ++cb) {
    const int c = w_first + 16 * cb + col;
    const bool real = c < ncols;
    const int t = real ? c / G : 0, g = real ? c % G : 0;
    hi_col[cb] = real ? hi_of(t) : p_lo;
    lo_col[cb] = real ? lo_of(t) : p_lo;
    const _Float16* qrow = reinterpret_cast<const _Float16*>(a.q) + (((size_t)b * T + t) * a.hq + (size_t)h * G + g) * D;
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2)
      qf[cb][c2] = real ? *reinterpret_cast<const h8*>(qrow + 32 * c2 + 8 * kq) : h8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  // BF16 K: the low parts go to the wave's LDS copy (written and read by the
  // wave alone); the BF16 kernel keeps the high parts in qf's registers, the
  // per-page kernel splits them from the fp16 query for its BF16 tiles
  const u4* qlo = KB ? qlo_lds + wave * NBC * NC * 64 : nullptr;
  if constexpr (KB) {
#pragma unroll
    for (int cb = 0; cb < NBC; ++cb)
#pragma unroll
      for (int c2 = 0; c2 < NC; ++c2) {
        qlo_lds[((wave * NBC + cb) * NC + c2) * 64 + lane] = bf_lo8(qf[cb][c2]);
        if constexpr (KC == C_BF16) qf[cb][c2] = __builtin_bit_cast(h8, bf_hi8(qf[cb][c2]));
      }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // INT2 K: the column's query summed over each 32-dim group (fp32)
  constexpr bool KZ = KC == C_ANY || has_zero(KC);
  constexpr bool VZ = VC == C_ANY || has_zero(VC);
  float qsum[NBC][NC];
#pragma unroll
  for (int cb = 0; cb < NBC; ++cb)
#pragma unroll
    for (int c2 = 0; c2 < NC; ++c2) {
      float x = 0.f;
      if constexpr (KZ) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x += (float)qf[cb][c2][e];
        x = row4_sum(x);
      }
      qsum[cb][c2] = x;
    }

  // m_run: the running max of the scores plus log2|s| of FP8 V pages, the
  // reference of l_run (the weights' sum without s) and acc (the P.V sums)
  float m_run[NBC], l_run[NBC];
  f4 acc[NBC][NB];
#pragma unroll
  for (int cb = 0; cb < NBC; ++cb) {
    m_run[cb] = NEG_INF;
    l_run[cb] = 0.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[cb][n] = f4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- tiles [t0, t0 + 16 ntiles): 16-token tiles of the partition up to
  // the last key any column of the workgroup attends
  const int t0 = wg_lo & ~15;
  const int ntiles = wg_hi > wg_lo ? (wg_hi - t0 + 15) / 16 : 0;
  const int t_end = t0 + 16 * ntiles;
  const int tpp = P / 16;

  // Page descriptors of the tiles, MAX_DESC pages at a time, gathered into LDS
  // by the whole workgroup (table reads once per page, validated here); the
  // tile loop then reads one descriptor from LDS per tile.
  for (int g0 = t0 / P; ntiles > 0 && g0 * P < t_end; g0 += MAX_DESC) {
    const int g1 = min(g0 + MAX_DESC, (t_end + P - 1) / P);
    lds_barrier();  // the previous chunk's tiles are consumed
    if (tid < g1 - g0) {
      const int lp = g0 + tid;
      const int pp = a.bt[(size_t)b * a.max_pages + lp];
      bool ok = (unsigned)pp < (unsigned)a.num_pages;
      const int pq = ok ? pp : 0;
      const int cod = a.codec[pq];
      const int kc = cod & 15, vc = cod >> 4;
      const uint64_t ko = a.koff[pq], vo = a.voff[pq];
      ok = ok && kc <= C_BIT1 && vc <= C_BIT1 && (KC == C_ANY || kc == KC) && (VC == C_ANY || vc == VC);
      ok = ok && (a.k_codec < 0 || kc == a.k_codec) && (a.v_codec < 0 || vc == a.v_codec);
      ok = ok && !((kc == C_FP8 || vc == C_FP8) && a.scale == nullptr) && ((ko | vo) & 15) == 0;
      ok = ok && ko <= a.pool_bytes && a.pool_bytes - ko >= plane_bytes(kc, a.hkv, P, D);
      ok = ok && vo <= a.pool_bytes && a.pool_bytes - vo >= plane_bytes(vc, a.hkv, P, D);
      PDesc d;
      d.k = ok ? ko : 0;
      d.v = ok ? vo : 0;
      d.sk = ok && kc == C_FP8 ? a.scale[((size_t)pq * a.hkv + h) * 2 + 0] : 1.f;
      d.sv = ok && vc == C_FP8 ? fp8_v_scale_word(a.scale[((size_t)pq * a.hkv + h) * 2 + 1]) : 64.f;
      d.valid = ok ? min(P, L - lp * P) : 0;
      d.codec = ok ? cod : 0;
      if (!ok) ++nerr;
      desc[tid] = d;
    }
    lds_barrier();

    // tiles of this chunk: [c0, c1)
    const int c0 = max(t0, g0 * P), c1 = min(t_end, g1 * P);
    const int nt = (c1 - c0) / 16;
    int ipg = c0 / P - g0, isub = (c0 % P) / 16;  // page and tile of the next tile issued
    auto meta = [&](int i) {
      TileMeta m;
      m.j0 = c0 + 16 * i;
      m.koff = 0; m.voff = 0; m.sk = 1.f; m.sv = 64.f; m.valid = 0; m.sub = 0;
      m.kc = KC == C_ANY ? 0 : KC;
      m.vc = VC == C_ANY ? 0 : VC;
      if (i >= nt) return m;
      const PDesc& d = desc[ipg];
      const int valid = __builtin_amdgcn_readfirstlane(d.valid) - 16 * isub;
      m.valid = min(max(valid, 0), 16);
      m.koff = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(d.k >> 32)) << 32) |
               __builtin_amdgcn_readfirstlane((uint32_t)d.k);
      m.voff = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(d.v >> 32)) << 32) |
               __builtin_amdgcn_readfirstlane((uint32_t)d.v);
      m.sk = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, d.sk)));
      m.sv = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, d.sv)));
      const int cod = __builtin_amdgcn_readfirstlane(d.codec);
      if (KC == C_ANY) m.kc = cod & 15;
      if (VC == C_ANY) m.vc = cod >> 4;
      m.sub = isub;
      if (++isub == tpp) { isub = 0; ++ipg; }
      return m;
    };

    // Tiles go in pairs, 32 keys per step: one barrier, one online-softmax
    // update and 16x16x32 P.V MFMAs per pair. The ring holds the codes of
    // PAIR_RING pairs: while one pair is consumed the next ones are in flight.
    Raw<D> raw[2 * PAIR_RING];
    TileMeta mt[2 * PAIR_RING];
#pragma unroll
    for (int s = 0; s < 2 * PAIR_RING; ++s) {
      mt[s] = meta(s);
      issue<D>(raw[s], mt[s], a, h, wave, lane);
    }
    for (int it = 0; it < nt; it += 2 * PAIR_RING) {
#pragma unroll
      for (int s = 0; s < PAIR_RING; ++s) {
        const int i = it + 2 * s;
        if (i >= nt) break;
        PairStage<D>& st = stage[(i >> 1) & 1];
        const TileMeta mA = mt[2 * s], mB = mt[2 * s + 1];
        // unconditional: a dead tile converts zeros that are never read, and the
        // ring registers are always consumed before they are loaded again
        produce_pair<D, KC, VC>(raw[2 * s], raw[2 * s + 1], mA, mB, st, wave, lane);
        mt[2 * s] = meta(i + 2 * PAIR_RING);
        issue<D>(raw[2 * s], mt[2 * s], a, h, wave, lane);
        mt[2 * s + 1] = meta(i + 2 * PAIR_RING + 1);
        issue<D>(raw[2 * s + 1], mt[2 * s + 1], a, h, wave, lane);
        lds_barrier();
        // a tile attends nothing for this wave when it is dead or outside every
        // column's key range; the pair is skipped when both do
        const bool offA = mA.valid <= 0 || mA.j0 >= w_hi_max || mA.j0 + 16 <= w_lo_min;
        const bool offB = mB.valid <= 0 || mB.j0 >= w_hi_max || mB.j0 + 16 <= w_lo_min;
        if (!wave_live || (offA && offB)) continue;

        // ---- scores of both tiles (before the K scale)
        const int kcA = KC == C_ANY ? mA.kc : KC, kcB = KC == C_ANY ? mB.kc : KC;
        const int vcA = VC == C_ANY ? mA.vc : VC, vcB = VC == C_ANY ? mB.vc : VC;
        f4 sA[NBC], sB[NBC];
        tile_scores<D, KC == C_BF16>(st.k[0], st.ks[0], st.kz[0], is_int(kcA), KZ && has_zero(kcA), KB && kcA == C_BF16,
                                     qf, qsum, qlo, lane, sA);
        tile_scores<D, KC == C_BF16>(st.k[1], st.ks[1], st.kz[1], is_int(kcB), KZ && has_zero(kcB), KB && kcB == C_BF16,
                                     qf, qsum, qlo, lane, sB);
        // scores in log2 units are raw * f: f > 0 goes into the max and the exp
        const float fA = is_int(kcA) ? a.scale_log2 : a.scale_log2 * mA.sk;
        const float fB = is_int(kcB) ? a.scale_log2 : a.scale_log2 * mB.sk;
        const bool masked = offA || offB || mA.j0 < w_lo_max || mB.j0 + 16 > w_hi_min;

        // ---- FP8 V scales in the log domain (log2|s| = 0, 1/|s| = 1 for the
        // other codecs and for dead tiles)
        const float lsvA = fabsf(mA.sv) - 64.f, lsvB = fabsf(mB.sv) - 64.f;
        const float isvA = lsvA == 0.f ? 1.f : __builtin_amdgcn_exp2f(-lsvA);
        const float isvB = lsvB == 0.f ? 1.f : __builtin_amdgcn_exp2f(-lsvB);
        const bool negA = mA.sv < 0.f, negB = mB.sv < 0.f;
        // BF16 V tiles go to the bf16 MFMA: a pair with one of them and one tile
        // of another codec is split in two halves
        constexpr bool VB = VC == C_BF16 || VC == C_ANY;
        const bool vbfA = VB && vcA == C_BF16, vbfB = VB && vcB == C_BF16;
        const bool split = vbfA != vbfB;

        const bool vint = is_int(vcA) || is_int(vcB);
        // INT2 V (a pair holding one): its value z + s*u is the sum of an offset
        // term and a step term, each of which can far exceed the value, so both
        // go to the MFMA with their weights split in fp16 high and low parts
        // (22 bits): p*s with the codes u, and p with the offsets z
        const bool vzero = VZ && (has_zero(vcA) || has_zero(vcB));

        // ---- online softmax of both column blocks; pa holds the P operand
        // (INT V: the weights times the token's fp16 group scale, one operand
        // per group; the staged scales are 1 for other codecs)
        h8 pa[NBC][NC];
        h8 pl[VZ ? NBC : 1][VZ ? NC : 1];  // INT2 V: low parts of pa
        h8 ph[VZ ? NBC : 1], pq[VZ ? NBC : 1];  // INT2 V: the plain weights, high and low
        u4 pbh[VB ? NBC : 1], pbl[VB ? NBC : 1];  // BF16 V: the weights in bf16, high and low
#pragma unroll
        for (int cb = 0; cb < NBC; ++cb) {
          float s8[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s8[j] = sA[cb][j];
            s8[4 + j] = sB[cb][j];
          }
          if (masked) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int pa_ = mA.j0 + 4 * kq + j, pb_ = mB.j0 + 4 * kq + j;
              s8[j] = (mA.valid > 0 && pa_ >= lo_col[cb] && pa_ < hi_col[cb]) ? s8[j] : NEG_INF;
              s8[4 + j] = (mB.valid > 0 && pb_ >= lo_col[cb] && pb_ < hi_col[cb]) ? s8[4 + j] : NEG_INF;
            }
          }
          const float mxa = __builtin_fmaf(fmaxf(fmaxf(s8[0], s8[1]), fmaxf(s8[2], s8[3])), fA, lsvA);
          const float mxb = __builtin_fmaf(fmaxf(fmaxf(s8[4], s8[5]), fmaxf(s8[6], s8[7])), fB, lsvB);
          const float mx = row4_max(fmaxf(mxa, mxb));
          const float m_new = fmaxf(m_run[cb], mx);
          if (__any(m_new > m_run[cb])) {
            const float alpha = m_new > m_run[cb] ? __builtin_amdgcn_exp2f(m_run[cb] - m_new) : 1.0f;
            l_run[cb] *= alpha;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float aj = __shfl(alpha, 4 * kq + j);
#pragma unroll
              for (int n = 0; n < NB; ++n) acc[cb][n][j] *= aj;
            }
            m_run[cb] = m_new;
          }
          const float mu = m_run[cb] == NEG_INF ? 0.f : m_run[cb];
          float p[8];
          const float oA = lsvA - mu, oB = lsvB - mu;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s8[j], fA, oA));
            p[4 + j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s8[4 + j], fB, oB));
          }
          l_run[cb] += __builtin_fmaf((p[0] + p[1]) + (p[2] + p[3]), isvA, ((p[4] + p[5]) + (p[6] + p[7])) * isvB);
          // a negative FP8 V scale flips its tile's weights
          if (negA) {
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = -p[j];
          }
          if (negB) {
#pragma unroll
            for (int j = 4; j < 8; ++j) p[j] = -p[j];
          }
          if constexpr (VB) {
            if (vbfA || vbfB) bf_split_w8(p, pbh[cb], pbl[cb]);
          }
          bool done = false;
          if constexpr (VZ) {
            if (vzero) {
#pragma unroll
              for (int g = 0; g < NC; ++g)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                  const float wv = p[j] * st.vs[j >> 2][(4 * kq + (j & 3)) * NC + g];
                  const _Float16 hi = (_Float16)wv;
                  pa[cb][g][j] = hi;
                  pl[cb][g][j] = (_Float16)(wv - (float)hi);
                }
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const _Float16 hi = (_Float16)p[j];
                ph[cb][j] = hi;
                pq[cb][j] = (_Float16)(p[j] - (float)hi);
              }
              done = true;
            }
          }
          if (done) {
          } else if (vint) {
#pragma unroll
            for (int g = 0; g < NC; ++g)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                pa[cb][g][j] = (_Float16)(p[j] * st.vs[0][(4 * kq + j) * NC + g]);
                pa[cb][g][4 + j] = (_Float16)(p[4 + j] * st.vs[1][(4 * kq + j) * NC + g]);
              }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) pa[cb][0][j] = (_Float16)p[j];
          }
        }

        // ---- P.V, dims 16n .. 16n+15 at a time. INT2 V: the offsets of the
        // lane's eight tokens (the same for the 16 dims of a block) as B.
        auto vfrag = [&](int n) { return __builtin_bit_cast(h8, st.v[n][lane]); };
        h8 zf[VZ ? NC : 1];
        if constexpr (VZ) {
          if (vzero) {
#pragma unroll
            for (int g = 0; g < NC; ++g)
#pragma unroll
              for (int j = 0; j < 8; ++j) zf[g][j] = (_Float16)st.vz[j >> 2][(4 * kq + (j & 3)) * NC + g];
          }
        }
        // one pass over the dims with the weights of the tokens picked by keep
        // (both tiles, or one of them when the pair is split)
        auto pv = [&](auto keep, auto keepu, bool bfh) {
          if constexpr (VB) {
            if (bfh) {
#pragma unroll
              for (int n = 0; n < NB; ++n) {
                const u4 vr = st.v[n][lane];
#pragma unroll
                for (int cb = 0; cb < NBC; ++cb)
                  acc[cb][n] = mfma32_bf(keepu(pbl[cb]), vr, mfma32_bf(keepu(pbh[cb]), vr, acc[cb][n]));
              }
              return;
            }
          }
#pragma unroll
          for (int n = 0; n < NB; ++n) {
            const h8 vf = vfrag(n);
            const int g = vint ? n / 2 : 0;
#pragma unroll
            for (int cb = 0; cb < NBC; ++cb) {
              acc[cb][n] = mfma32(keep(pa[cb][g]), vf, acc[cb][n]);
              if constexpr (VZ) {
                if (vzero) {
                  acc[cb][n] = mfma32(keep(pl[cb][g]), vf, acc[cb][n]);
                  acc[cb][n] = mfma32(keep(ph[cb]), zf[n / 2], acc[cb][n]);
                  acc[cb][n] = mfma32(keep(pq[cb]), zf[n / 2], acc[cb][n]);
                }
              }
            }
          }
        };
        if (!split) {
          pv([](h8 w) { return w; }, [](u4 w) { return w; }, vbfA);
        } else {
          const _Float16 z = 0;
          pv([z](h8 w) { return h8{w[0], w[1], w[2], w[3], z, z, z, z}; }, [](u4 w) { return u4{w[0], w[1], 0u, 0u}; },
             vbfA);
          pv([z](h8 w) { return h8{z, z, z, z, w[4], w[5], w[6], w[7]}; }, [](u4 w) { return u4{0u, 0u, w[2], w[3]}; },
             vbfB);
        }
      }
    }
  }
  if (reporter && nerr > 0 && a.err) atomicAdd(a.err, nerr);
  if (!wave_live) return;

  // ---- results: lane holds out[column 16cb + 4kq + j][dim 16n + col]
#pragma unroll
  for (int cb = 0; cb < NBC; ++cb) {
    const float l_tot = row4_sum(l_run[cb]);
    // own column (lanes of row 0 write lse / (m, l))
    {
      const int c = w_first + 16 * cb + col;
      if (kq == 0 && c < ncols) {
        const int t = c / G, g = c % G;
        const size_t r = ((size_t)b * T + t) * a.hq + (size_t)h * G + g;
        if (a.final_out) {
          a.lse[r] = l_tot > 0.f ? m_run[cb] * LN2 + logf(l_tot) : NEG_INF;
        } else {
          const size_t pi = r * a.nparts + part;
          a.part_ml[2 * pi + 0] = l_tot > 0.f ? m_run[cb] * LN2 : NEG_INF;
          a.part_ml[2 * pi + 1] = l_tot;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lj = __shfl(l_tot, 4 * kq + j);
      const int c = w_first + 16 * cb + 4 * kq + j;
      if (c >= ncols) continue;
      const int t = c / G, g = c % G;
      const size_t r = ((size_t)b * T + t) * a.hq + (size_t)h * G + g;
      if (a.final_out) {
#pragma unroll
        for (int n = 0; n < NB; ++n) a.out[r * D + 16 * n + col] = lj > 0.f ? acc[cb][n][j] / lj : 0.f;
      } else {
        float* dst = a.part_acc + (r * a.nparts + part) * D;
#pragma unroll
        for (int n = 0; n < NB; ++n) dst[16 * n + col] = acc[cb][n][j];
      }
    }
  }
}

// acc <- fold(acc, (out, lse)); one 64-lane block per row.
__global__ void __launch_bounds__(64) fold_into_kernel(int rows, int D, float* acc_out, float* acc_lse,
                                                       const float* out, const float* lse) {
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const float la = acc_lse[r], lb = lse[r];
    const float M = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f;
    if (M != NEG_INF) {
      wa = la == NEG_INF ? 0.f : expf(la - M);
      wb = lb == NEG_INF ? 0.f : expf(lb - M);
    }
    const float den = wa + wb;
    for (int d = threadIdx.x; d < D; d += 64) {
      // an empty side contributes nothing, whatever its values hold
      const size_t i = (size_t)r * D + d;
      const float x = (wa > 0.f ? wa * acc_out[i] : 0.f) + (wb > 0.f ? wb * out[i] : 0.f);
      acc_out[i] = M == NEG_INF ? 0.f : x / den;
    }
    if (threadIdx.x == 0) acc_lse[r] = M == NEG_INF ? NEG_INF : M + logf(den);
  }
}

}  // namespace

namespace {

template <int D, int KC, int VC>
int launch_prefill_t(const PrefillArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, KC, VC>), grid, dim3(THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Kernels specialised for one codec pair (the codec dispatch compiled away),
// and the per-page dispatch variant for any other declaration.
template <int D>
int launch_prefill_d(const PrefillArgs& a, dim3 grid, hipStream_t s) {
  const int kc = a.k_codec < 0 ? C_ANY : a.k_codec;
  const int vc = a.v_codec < 0 ? C_ANY : a.v_codec;
#define PKV_PAIR(K, V) \
  if (kc == K && vc == V) return launch_prefill_t<D, K, V>(a, grid, s);
  PKV_PAIR(C_FP16, C_FP16)
  PKV_PAIR(C_BF16, C_BF16)
  PKV_PAIR(C_FP8, C_FP8)
  PKV_PAIR(C_INT8, C_INT4)
#undef PKV_PAIR
  return launch_prefill_t<D, C_ANY, C_ANY>(a, grid, s);
}

}  // namespace

int launch_prefill(const PrefillArgs& a, int head_dim, void* stream) {
  if (a.rows == 0 || a.tokens == 0) return 0;
  const long long gx = (long long)((a.nparts + 7) / 8) * 8 * a.col_groups;
  const dim3 grid((unsigned)gx, a.hkv, a.rows);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (head_dim == 64) return launch_prefill_d<64>(a, grid, s);
  if (head_dim == 128) return launch_prefill_d<128>(a, grid, s);
  return -2;
}

int launch_fold_into(int rows, int head_dim, float* acc_out, float* acc_lse, const float* out, const float* lse,
                     void* stream) {
  if (rows == 0) return 0;
  const int grid = rows < 65536 ? rows : 65536;
  hipLaunchKernelGGL(fold_into_kernel, dim3(grid), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), rows,
                     head_dim, acc_out, acc_lse, out, lse);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
