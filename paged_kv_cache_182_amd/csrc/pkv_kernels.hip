// Decode attention over a mixed-codec paged KV cache, gfx950 (CDNA4).
//
// One workgroup of four 64-lane waves owns one (partition, KV head, row).
// It first gathers the partition's page descriptors (selection entry ->
// block table -> codec, plane offsets, FP8 scales) into LDS, then each wave
// walks 16-token tiles of those pages: exact conversion of the codes to fp16
// in registers, MFMA for the q.K scores and for P.V, and an exact online
// softmax (ARGUS "Direct paged attention": tile-by-tile online softmax over
// an SoA page table; FreeToken PR #499 "Design": block-table translation).
// The waves' states are merged through LDS; a row split into several
// partitions leaves (acc, max, sum) partials that a second kernel folds by
// log-sum-exp (PR #499 discussion, in-place host K/V design).
//
// Tile layout seen by one wave (lane l, col = l % 16, kq = l / 16):
//  * scores use v_mfma_f32_16x16x32_f16 with A = K (row = token col of the
//    tile, 8 dims per lane) and B = q^T (col = query head of the group);
//    lane l receives scores of tokens 4*kq + j (j = 0..3) for head col.
//  * P.V uses v_mfma_f32_16x16x16_f16 with A = P (those same four scores,
//    which is exactly the A operand layout) and B = V (4 tokens of one dim,
//    which the V plane layout stores contiguously per lane); lane l
//    accumulates out[head 4*kq + j][dim 16*n + col].
// Every code converts to fp16 exactly (FP8 e4m3, int8, int4, the unsigned
// 2-bit steps, the 1-bit signs and -- within fp16 range -- bf16), so each
// product is exact and accumulates in fp32; scales are applied in fp32 to the
// scores (K) or folded into P (V). The 2-bit codec's group offsets add one
// term per group to the scores (offset times the group's query sum) and one
// MFMA with the offsets as B operand to P.V.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

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
typedef short s4 __attribute__((ext_vector_type(4)));

enum : int { C_FP16 = 0, C_BF16 = 1, C_FP8 = 2, C_INT8 = 3, C_INT4 = 4, C_INT2 = 5, C_BIT1 = 6, C_FLT = 14, C_ANY = 15 };
constexpr int C_LAST = C_BIT1;  // highest codec id a page may hold
// C_ANY: any codec per page and plane. C_FLT: per page one of FP16, BF16, FP8,
// the same for K and V (no group scales: a smaller kernel than C_ANY's).
__host__ __device__ constexpr bool per_page(int c) { return c == C_ANY || c == C_FLT; }

#ifndef PKV_RING_WORDS
#define PKV_RING_WORDS 32  // 32-bit words of tile codes a wave keeps in flight
#endif

constexpr int WAVES = 4;
constexpr int THREADS = 64 * WAVES;
constexpr int MAX_DESC = 256;  // page descriptors staged in LDS at a time
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LN2 = 0.693147180559945309f;

// log2 of the code width, three bits per codec (FP16 and BF16 16 bits, FP8
// and INT8 8, INT4 4, INT2 2, BIT1 1): a shift of one constant, where a chain
// of compares on a codec known only at run time compiles to branches
__host__ __device__ constexpr int lg_bits(int c) { return c < 0 ? 4 : (int)((0xa6e4u >> (3 * c)) & 7u); }
__host__ __device__ constexpr int bits_of(int c) { return 1 << lg_bits(c); }
// codecs with one fp16 scale per (token, 32 dims): INT8, INT4, INT2, BIT1
__host__ __device__ constexpr bool is_int(int c) { return (unsigned)(c - C_INT8) <= (unsigned)(C_BIT1 - C_INT8); }
// INT2 (unsigned affine) also holds one fp16 offset per (token, 32 dims)
__host__ __device__ constexpr bool has_zero(int c) { return c == C_INT2; }

// Bytes of one plane (codes of every head, then INT group scales).
__host__ __device__ inline uint64_t plane_bytes(int c, int hkv, int page, int d) {
  const uint64_t codes = ((uint64_t)hkv * page * (d / 8)) << lg_bits(c);
  const uint64_t groups = (uint64_t)hkv * page * (d / 32) * 2;
  return codes + (is_int(c) ? groups : 0) + (has_zero(c) ? groups : 0);
}

// Raw buffer loads through a per-plane resource: the base and size live in
// scalar registers, every lane supplies a 32-bit offset, and an offset past
// the size reads zeros instead of faulting. A skipped tile gets size 0, so
// every tile issues the same loads and the wait counts stay exact.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_WORD3 = 0x00020000;  // gfx9-family raw buffer format

__device__ inline rsrc_t make_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, RSRC_WORD3);
}
constexpr int CPOL_NT = 2;  // non-temporal: page codes are read once
template <int CPOL = 0>
__device__ inline u4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL));
}
template <int CPOL = 0>
__device__ inline u2 bload8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, CPOL));
}
template <int CPOL = 0>
__device__ inline uint32_t bload4(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, CPOL);
}
constexpr uint32_t OFF_NONE = 0xFFFFFF00u;  // past any plane: reads zero, no traffic
constexpr int VMCNT0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left free (gfx9 encoding)

// Page descriptor staged in LDS (32 bytes).
struct Desc {
  uint64_t k;      // byte offset of the K plane in the pool (0 if the page is skipped)
  uint64_t v;      // byte offset of the V plane
  float sk, sv;    // FP8 scales of this KV head (1 for other codecs)
  int32_t valid;   // attended tokens of the page (0 if skipped): slots [lo, valid)
  int32_t codec;   // K codec | V codec << 4 | lo << 8, lo = leading slots before a sliding window
};
static_assert(sizeof(Desc) == 32 && offsetof(Desc, v) == 8 && offsetof(Desc, sk) == 16 && offsetof(Desc, valid) == 24 &&
                  offsetof(Desc, codec) == 28,
              "a descriptor is read as two 16-byte words");

// Raw codes of one 16-token tile for one lane. Sizes per codec class; the
// per-page dispatch variant (C_ANY) reserves the largest.
template <int D, int KC, int VC>
struct Tile {
  static constexpr int KB = per_page(KC) ? 16 : bits_of(KC);
  static constexpr int VB = per_page(VC) ? 16 : bits_of(VC);
  static constexpr int KW = D * KB < 128 ? 1 : D * KB / 128;  // 32-bit words of K codes per lane
  static constexpr int VW = D * VB < 128 ? 1 : D * VB / 128;
  static constexpr int SW = D / 16;        // words of 4 tokens x D/32 fp16 scales
  static constexpr bool KS = KC == C_ANY || is_int(KC);
  static constexpr bool VS = VC == C_ANY || is_int(VC);
  static constexpr bool GS = KS || VS;     // some plane may carry group scales
  static constexpr bool KZ = KC == C_ANY || has_zero(KC);  // and group offsets
  static constexpr bool VZ = VC == C_ANY || has_zero(VC);
  uint32_t k[KW];
  uint32_t v[VW];
  // Group scales of the tile, one word per lane: the 16 tokens x D/32 fp16
  // K scales in lanes 0 .. D/4-1 (sk), the V scales in lanes 32 .. 32+D/4-1
  // (sv); the INT2 offsets in the other half of each: K offsets in lanes
  // 32 .. 32+D/4-1 of sk, V offsets in lanes 0 .. D/4-1 of sv; zero
  // elsewhere. Spread to the lanes that use them through LDS.
  uint32_t sk[1];
  uint32_t sv[1];
};

#ifndef PKV_RING_WORDS_GS
#define PKV_RING_WORDS_GS PKV_RING_WORDS  // the same for kernels with group-scale planes
#endif

template <int D, int KC, int VC>
__host__ __device__ constexpr int ring_depth() {
  using T = Tile<D, KC, VC>;
  constexpr int words = T::KW + T::VW + (T::KS ? 1 : 0) + (T::VS ? 1 : 0);
  constexpr int d = (T::GS ? PKV_RING_WORDS_GS : PKV_RING_WORDS) / words;
  return d < 2 ? 2 : (d > 8 ? 8 : d);
}

// Occupancy asked of the compiler: four waves per SIMD (a whole 1024-
// workgroup grid resident at once) where the tile ring is small enough,
// three for the codecs with group scales (more state per tile).
template <int D, int KC, int VC>
__host__ __device__ constexpr int waves_per_eu() {
#ifdef PKV_WAVES
  return PKV_WAVES;
#else
  return decode_waves_per_simd(D, KC == C_ANY ? -1 : (KC == C_FLT ? -2 : KC), VC == C_ANY ? -1 : (VC == C_FLT ? -2 : VC));
#endif
}

// Upper bound of the occupancy range: the same for the per-page kernels
// (their registers are at the edge: aiming higher spills them), open for the
// fixed pairs.
template <int D, int KC, int VC>
__host__ __device__ constexpr int max_waves_per_eu() {
  return per_page(KC) ? waves_per_eu<D, KC, VC>() : 8;
}

struct TileInfo {
  int valid;  // tokens of the tile to attend: [lo, valid) (valid 0: skip the tile)
  int lo;     // leading tokens before a sliding window
  int kc, vc;
  float sk, sv;
};

__device__ inline void count_error(int32_t* err) {
  if (err) atomicAdd(err, 1);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// accesses, not for its global loads in flight (q, tiles), which
// __syncthreads would also drain.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline uint64_t uni64(uint64_t x) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline float unif(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// ---------------------------------------------------------------- loads
// A 1-bit run of 16 codes (head_dim 64) is one 16-bit unit: even codes in
// bits 0..7, odd codes in bits 8..15. Moving the odd byte to bits 16..23 gives
// the layout of a 32-code word (even codes low, odd codes from bit 16), so
// both head dims decode alike.
__device__ inline uint32_t spread16(uint32_t u) { return (u & 0xffu) | ((u & 0xff00u) << 8); }

// The lane's run of one 16-token tile: R = D*bits/32 bytes. Tiles are stored
// as the image of the 64 lanes' registers, 16-byte chunks interleaved over the
// lanes (chunk i of lane L at i*1024 + 16*L), so every load instruction of a
// wave covers 1 KB of consecutive bytes: whole cache lines, read once, which
// is what lets the non-temporal hint pay off. The run holds, for K, token
// lane%16 and dims (D/4)(lane/16) + e (one scale per page) or 32c + 8(lane/16)
// + j (group scales); for V, tokens 4(lane/16) + j of dim 16n + lane%16.
template <int D, int BITS>
__device__ inline void load_run(uint32_t* w, rsrc_t r, uint32_t head, int sub, int lane) {
  constexpr int R = D * BITS / 32;
  constexpr int TB = 16 * D * BITS / 8;
  const uint32_t base = head + (uint32_t)sub * TB;
  if constexpr (R >= 16) {
#pragma unroll
    for (int i = 0; i < R / 16; ++i) {
      const u4 x = bload16<CPOL_NT>(r, base + 1024 * i + 16 * lane);
      w[4 * i + 0] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
    }
  } else if constexpr (R == 8) {
    const u2 x = bload8<CPOL_NT>(r, base + 8 * lane);
    w[0] = x[0]; w[1] = x[1];
  } else if constexpr (R == 4) {
    w[0] = bload4<CPOL_NT>(r, base + 4 * lane);
  } else {
    static_assert(R == 2, "run of 2 bytes expected");
    const uint32_t x = bload4<CPOL_NT>(r, base + 4 * (lane >> 1));
    w[0] = spread16((lane & 1) ? x >> 16 : x & 0xffffu);
  }
}

// ---------------------------------------------------------------- decode
__device__ inline h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }

// two OCP e4m3 codes (bytes 0,1 or 2,3 of w) -> two fp16 (exact)
template <bool HI>
__device__ inline h2 fp8x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// four int8 codes -> four fp16 (exact): 0x64XX is 1024 + XX, XX = code + 128
__device__ inline h4 int8x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;
  const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off;
  h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off;
  return h4{a[0], a[1], b[0], b[1]};
}

// eight int4 codes of one word -> fp16 pairs (elements 0,1 | 2,3 | 4,5 | 6,7).
// Element pair s sits in bits 4s..4s+3 of each 16-bit half. Masking a nibble
// in place under the fp16 pattern of 1024 and flipping its top bit gives
// 1024 + (c + 8) (bits 0..3) or 1024 + 16 (c + 8) (bits 4..7); one packed
// subtract or fused multiply-add (1/16, -72) then yields c exactly.
__device__ inline void int4x8(uint32_t w, h2* o) {
  const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 off16 = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t u8 = w >> 8;
  o[0] = as_h2((w & 0x000f000fu) ^ 0x64086408u) - off;
  o[1] = __builtin_elementwise_fma(as_h2((w & 0x00f000f0u) ^ 0x64806480u), s16, -off16);
  o[2] = as_h2((u8 & 0x000f000fu) ^ 0x64086408u) - off;
  o[3] = __builtin_elementwise_fma(as_h2((u8 & 0x00f000f0u) ^ 0x64806480u), s16, -off16);
}

// two unsigned 2-bit codes at bits s, s+1 and 16+s, 17+s -> fp16 pair (exact):
// placed under the fp16 pattern of 1024 (0x6400), then 1024 subtracted
__device__ inline h2 u2pair(uint32_t w, int s) {
  const h2 off = {(_Float16)1024.0f, (_Float16)1024.0f};
  return as_h2(((w >> s) & 0x00030003u) | 0x64006400u) - off;
}
// two sign codes at bits k and 16+k -> fp16 pair of +-1 (bit set: -1): each
// bit moved into an fp16 sign bit over the pattern of 1.0 (0x3C00)
__device__ inline h2 b1pair(uint32_t w, int k) {
  return as_h2(((w << (15 - k)) & 0x80008000u) | 0x3C003C00u);
}

// A operand of the score MFMA: dims 32c + 8kq .. +7 of the lane's token.
// (BF16 codes do not come here: they go to the bf16 MFMA as they are.)
template <int C, int D>
__device__ inline h8 k_frag(const uint32_t* w, int c) {
  static_assert(C != C_BF16, "BF16 runs feed the bf16 MFMA");
  if constexpr (C == C_FP16) {
    return __builtin_bit_cast(h8, u4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]});
  } else if constexpr (C == C_FP8) {
    h2 a = fp8x2<false>(w[2 * c]), b = fp8x2<true>(w[2 * c]);
    h2 d = fp8x2<false>(w[2 * c + 1]), e = fp8x2<true>(w[2 * c + 1]);
    return h8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  } else if constexpr (C == C_INT8) {
    h4 a = int8x4(w[2 * c]), b = int8x4(w[2 * c + 1]);
    return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else if constexpr (C == C_INT4) {
    h2 o[4];
    int4x8(w[c], o);
    return h8{o[0][0], o[0][1], o[1][0], o[1][1], o[2][0], o[2][1], o[3][0], o[3][1]};
  } else if constexpr (C == C_INT2) {
    // elements 8(c % 2) + j of word c / 2: pair j, j + 1 at slots 4(c % 2) + j/2 and 8 + that
    const uint32_t x = w[c >> 1];
    const int s0 = 8 * (c & 1);
    h2 a = u2pair(x, s0), b = u2pair(x, s0 + 2), d = u2pair(x, s0 + 4), e = u2pair(x, s0 + 6);
    return h8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  } else {
    // elements 8c + j of the run's word: pair j, j + 1 at bits 4c + j/2 and 16 + that
    const uint32_t x = w[0];
    h2 a = b1pair(x, 4 * c), b = b1pair(x, 4 * c + 1), d = b1pair(x, 4 * c + 2), e = b1pair(x, 4 * c + 3);
    return h8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  }
}

// B operand of the P.V MFMA: tokens 4kq .. +3 of dim 16n + col (16-bit runs:
// FP16 as they are; BF16 runs go to the bf16 MFMA, the same words).
template <int C, int D>
__device__ inline h4 v_frag(const uint32_t* w, int n) {
  if constexpr (C == C_FP16 || C == C_BF16) {
    return __builtin_bit_cast(h4, u2{w[2 * n], w[2 * n + 1]});
  } else if constexpr (C == C_FP8) {
    h2 a = fp8x2<false>(w[n]), b = fp8x2<true>(w[n]);
    return h4{a[0], a[1], b[0], b[1]};
  } else if constexpr (C == C_INT8) {
    return int8x4(w[n]);
  } else if constexpr (C == C_INT4) {
    h2 o[4];
    int4x8(w[n / 2], o);
    return (n & 1) ? h4{o[2][0], o[2][1], o[3][0], o[3][1]} : h4{o[0][0], o[0][1], o[1][0], o[1][1]};
  } else if constexpr (C == C_INT2) {
    // elements 4(n % 4) + j of word n / 4: tokens 0, 1 at bits 4(n % 4) and 16 + that,
    // tokens 2, 3 two bits higher
    const uint32_t x = w[n >> 2];
    h2 a = u2pair(x, 4 * (n & 3)), b = u2pair(x, 4 * (n & 3) + 2);
    return h4{a[0], a[1], b[0], b[1]};
  } else {
    // elements 4n + j: tokens 0, 1 at bits 2n and 16 + 2n, tokens 2, 3 one bit higher
    h2 a = b1pair(w[0], 2 * n), b = b1pair(w[0], 2 * n + 1);
    return h4{a[0], a[1], b[0], b[1]};
  }
}

// Runtime-dispatched variants for pages of mixed codecs (BF16 runs are
// taken before: they feed the bf16 MFMA).
template <int D>
__device__ inline h8 k_frag_any(const uint32_t* w, int c, int codec) {
  switch (codec) {
    case C_FP16: return k_frag<C_FP16, D>(w, c);
    case C_FP8: return k_frag<C_FP8, D>(w, c);
    case C_INT8: return k_frag<C_INT8, D>(w, c);
    case C_INT4: return k_frag<C_INT4, D>(w, c);
    case C_INT2: return k_frag<C_INT2, D>(w, c);
    default: return k_frag<C_BIT1, D>(w, c);
  }
}
template <int D>
__device__ inline h4 v_frag_any(const uint32_t* w, int n, int codec) {
  switch (codec) {
    case C_FP16: return v_frag<C_FP16, D>(w, n);
    case C_FP8: return v_frag<C_FP8, D>(w, n);
    case C_INT8: return v_frag<C_INT8, D>(w, n);
    case C_INT4: return v_frag<C_INT4, D>(w, n);
    case C_INT2: return v_frag<C_INT2, D>(w, n);
    default: return v_frag<C_BIT1, D>(w, n);
  }
}

// Whether K runs hold a contiguous stretch of dims (codecs with one scale per
// page) rather than 8 dims of each 32-dim group (group-scale codecs).
template <int KC>
__host__ __device__ constexpr bool k_perm() {
  return KC != C_ANY && !is_int(KC);  // C_FLT: one-scale codecs only
}
// log2 code width of a page's codec in a kernel built for PC: the float
// kernel's pages hold only FP16, BF16 or FP8 (one compare instead of the
// table lookup).
template <int PC>
__device__ inline int lg_page(int codec) {
  return PC == C_FLT ? (codec == C_FP8 ? 3 : 4) : lg_bits(PC == C_ANY ? codec : PC);
}
// Bytes of a page's plane (fits 32 bits: the host checks plane sizes).
template <int PC, int D>
__device__ inline uint32_t plane_bytes_page(int codec, int hkv, int page) {
  if constexpr (PC == C_FLT) return (uint32_t)(hkv * page * (D / 8)) << lg_page<PC>(codec);
  else return (uint32_t)plane_bytes(PC == C_ANY ? codec : PC, hkv, page, D);
}
// Byte offset of head h's codes inside a plane.
template <int D>
__device__ inline uint32_t head_off(int codec, int h, int page) {
  return (uint32_t)(h * page * (D / 8)) << lg_bits(codec);
}

// The lane's run of a plane whose codec is known only at run time: the same
// D/32 16-byte loads for every codec, branch-free, so the compiler's wait
// counts stay exact across pages of different codecs. Loads past the run
// (codes of 8 bits or fewer) read through an offset beyond the plane: zeros,
// no traffic. A run of R < 16 bytes (R = D * bits / 32) arrives inside the
// 16-byte chunk that holds it (16 / R lanes per chunk, the same cache lines);
// short_run() moves it to the first words when the tile is consumed (doing it
// here would wait for the loads just issued).
template <int D, int PC>
__device__ inline void load_run_any(uint32_t* w, rsrc_t r, int codec, int h, int page, int sub, int lane) {
  constexpr int NL = D / 32;  // 16-byte loads of a 16-bit run
  const int lg = lg_page<PC>(codec);
  const uint32_t head = (uint32_t)(h * page * (D / 8)) << lg;
  const uint32_t base = head + ((uint32_t)sub * (uint32_t)(2 * D) << lg);
  const int R = (D / 32) << lg;  // bytes of the lane's run
  const int nreal = R >= 16 ? R >> 4 : 1;
  const uint32_t lane_off = R >= 16 ? 16u * (uint32_t)lane : 16u * (uint32_t)((lane * R) >> 4);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const u4 x = bload16<CPOL_NT>(r, i < nreal ? base + 1024u * i + lane_off : OFF_NONE);
    w[4 * i + 0] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
  }
}

// Move a short run (R < 16 bytes) from its place in the loaded 16-byte chunk
// to the first words: R = 8 at word 2 (odd lanes), R = 4 at word lane % 4,
// R = 2 in half-word lane % 8 (then spread as a 16-bit unit). Selects on
// register values only (an index into the tile array would move the tile
// ring to scratch memory).
template <int D>
__device__ inline void short_run(uint32_t* w, int codec, int lane) {
  const int R = (D / 32) << lg_bits(codec);
  if (R >= 16) return;
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
  if (R == 8) {
    const bool odd = lane & 1;
    w[0] = odd ? w2 : w0;
    w[1] = odd ? w3 : w1;
  } else {
    const int q = ((lane * R) & 15) >> 2;          // word of the chunk holding the run
    const uint32_t lo = (q & 1) ? w1 : w0, hi = (q & 1) ? w3 : w2;
    const uint32_t x = (q & 2) ? hi : lo;
    w[0] = R == 4 ? x : spread16((lane & 1) ? x >> 16 : x & 0xffffu);
  }
}

// Issue the loads of tile `k` of the staged pages into `t`. Every call issues
// the same loads: a tile with nothing to attend reads through a zero-size
// resource (zeros, no fault) and is skipped when consumed.
template <int D, int KC, int VC>
__device__ inline TileInfo issue_tile(Tile<D, KC, VC>& t, const Desc* desc, int k, int tpp,
                                      const DecodeArgs& a, int h, int lane, bool dead = false) {
  // page of the tile and tile within the page: a shift when tiles per page
  // is a power of two (every usual page size), else a division
  const int i = a.tile_shift >= 0 ? k >> a.tile_shift : k / tpp;
  const int sub = k - i * tpp;
  TileInfo ti;
  // the descriptor as two 16-byte LDS reads issued together (one wait)
  const u4* dp = reinterpret_cast<const u4*>(desc + i);
  const u4 d0 = dp[0], d1 = dp[1];
  const int codec = uni((int)d1[3]);
  ti.lo = min(max((codec >> 8) - 16 * sub, 0), 16);
  ti.valid = dead ? 0 : min(max(uni((int)d1[2]) - 16 * sub, 0), 16);
  ti.valid = ti.valid > ti.lo ? ti.valid : 0;  // wholly before the window: skip
  ti.kc = per_page(KC) ? (codec & 15) : KC;
  ti.vc = per_page(VC) ? ((codec >> 4) & 15) : VC;
  ti.sk = __builtin_bit_cast(float, uni((int)d1[0]));
  ti.sv = __builtin_bit_cast(float, uni((int)d1[1]));
  const uint64_t koff = ((uint64_t)(uint32_t)uni((int)d0[1]) << 32) | (uint32_t)uni((int)d0[0]);
  const uint64_t voff = ((uint64_t)(uint32_t)uni((int)d0[3]) << 32) | (uint32_t)uni((int)d0[2]);
  const bool live = ti.valid > 0;
  const int page = a.page;
  const rsrc_t rk = make_rsrc(a.pool + koff, live ? plane_bytes_page<KC, D>(ti.kc, a.hkv, page) : 0u);
  const rsrc_t rv = make_rsrc(a.pool + voff, live ? plane_bytes_page<VC, D>(ti.vc, a.hkv, page) : 0u);
  // group scales first: loads complete in order and the scores need them early
  if constexpr (Tile<D, KC, VC>::GS) {
    constexpr int NW = D / 4;  // words of one tile's scales (16 tokens x D/32 fp16)
    const uint32_t blk = (uint32_t)((h * page + 16 * sub) * (D / 32) * 2);
    // INT2 offsets follow every head's scales, laid out as the scales; they
    // go to the other half of the lanes of the same word
    const uint32_t zgap = (uint32_t)(a.hkv * page * (D / 32) * 2);
    const int hl = lane & 31;
    if constexpr (Tile<D, KC, VC>::KS) {
      const uint32_t base = ((uint32_t)(a.hkv * page * (D / 8)) << lg_bits(ti.kc)) + blk;
      const bool want = lane < 32 ? is_int(ti.kc) : (Tile<D, KC, VC>::KZ && has_zero(ti.kc));
      t.sk[0] = bload4(rk, want && hl < NW ? base + (lane < 32 ? 0u : zgap) + 4 * hl : OFF_NONE);
    }
    if constexpr (Tile<D, KC, VC>::VS) {
      const uint32_t base = ((uint32_t)(a.hkv * page * (D / 8)) << lg_bits(ti.vc)) + blk;
      const bool want = lane >= 32 ? is_int(ti.vc) : (Tile<D, KC, VC>::VZ && has_zero(ti.vc));
      t.sv[0] = bload4(rv, want && hl < NW ? base + (lane >= 32 ? 0u : zgap) + 4 * hl : OFF_NONE);
    }
  }
  if constexpr (per_page(KC)) {
    load_run_any<D, KC>(t.k, rk, ti.kc, h, page, sub, lane);
  } else {
    load_run<D, bits_of(KC)>(t.k, rk, head_off<D>(KC, h, page), sub, lane);
  }
  if constexpr (per_page(VC)) {
    load_run_any<D, VC>(t.v, rv, ti.vc, h, page, sub, lane);
  } else {
    load_run<D, bits_of(VC)>(t.v, rv, head_off<D>(VC, h, page), sub, lane);
  }
  return ti;
}

__device__ inline f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// The bf16 forms, for BF16 pages: their codes go in as they are, so values
// of bf16's whole range (beyond fp16's 65504, below its 2^-24) stay exact.
__device__ inline f4 mfma32_bf(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}
__device__ inline f4 mfma16_bf(u2 a, u2 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
}
// Eight fp16 query values as bf16 high and low parts, x = hi + lo exactly:
// hi keeps the top 8 of x's 11 significant bits (truncation), the rest, at
// most 3 bits, is exact in bf16 (whose exponent range holds fp16's
// subnormals); each products of a bf16 code with hi and with lo is exact.
__device__ inline void bf_split8(h8 x, u4& hi, u4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = (float)x[2 * i], b = (float)x[2 * i + 1];
    const uint32_t ha = __builtin_bit_cast(uint32_t, a) & 0xffff0000u, hb = __builtin_bit_cast(uint32_t, b) & 0xffff0000u;
    const uint32_t la = __builtin_bit_cast(uint32_t, a - __builtin_bit_cast(float, ha));
    const uint32_t lb = __builtin_bit_cast(uint32_t, b - __builtin_bit_cast(float, hb));
    hi[i] = __builtin_amdgcn_perm(hb, ha, 0x07060302u);
    lo[i] = __builtin_amdgcn_perm(lb, la, 0x07060302u);
  }
}
// Four fp32 softmax weights as bf16 high (truncated) and low (the remainder
// rounded to nearest) parts: 16 significant bits, more than the fp16 weights
// of the other one-scale codecs.
__device__ inline void bf_split4(const float* p, u2& hi, u2& lo) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float a = p[2 * i], b = p[2 * i + 1];
    const uint32_t ha = __builtin_bit_cast(uint32_t, a) & 0xffff0000u, hb = __builtin_bit_cast(uint32_t, b) & 0xffff0000u;
    const __bf16 la = (__bf16)(a - __builtin_bit_cast(float, ha)), lb = (__bf16)(b - __builtin_bit_cast(float, hb));
    hi[i] = __builtin_amdgcn_perm(hb, ha, 0x07060302u);
    lo[i] = (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
  }
}

// Max and sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows
// that hold one column), with the row-swapping permutes of gfx950: swapping
// the odd rows of one copy with the even rows of another (16-lane rows, then
// 32-lane halves) leaves each lane its own value in one result and its
// partner row's value in the other. The two results are read straight from
// the builtin's vector and pass through an empty asm: reading them through a
// bit cast of the pair has been seen to let the optimizer merge them.
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

// Zero the V codes of this lane's tokens 4*kq + j, j >= nv (past the end of
// the sequence): their bytes may be anything, even NaN codes, and 0 * NaN
// would poison the MFMA. A zero code decodes to 0 in every codec. Word n of
// an 8-bit run holds tokens j in bytes j; 16-bit runs hold tokens 0,1 in even
// and 2,3 in odd words; an int4 word holds token j in the nibbles below.
// 2- and 1-bit codes decode to finite values whatever their bits (their
// scales and offsets of such tokens are zeroed instead), so they are left.
// Tokens j of the lane's four are kept for a <= j < b (a > 0: before a
// sliding window).
__device__ inline void mask_v_run(uint32_t* v, int words, int bits, int a, int b) {
  const bool k0 = a <= 0 && b > 0, k1 = a <= 1 && b > 1, k2 = a <= 2 && b > 2, k3 = a <= 3 && b > 3;
  if (bits == 8) {
    const uint32_t m = (k0 ? 0x000000ffu : 0u) | (k1 ? 0x0000ff00u : 0u) | (k2 ? 0x00ff0000u : 0u) |
                       (k3 ? 0xff000000u : 0u);
    for (int i = 0; i < words; ++i) v[i] &= m;
  } else if (bits == 16) {
    const uint32_t m0 = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
    const uint32_t m1 = (k2 ? 0x0000ffffu : 0u) | (k3 ? 0xffff0000u : 0u);
    for (int i = 0; i < words; ++i) v[i] &= (i & 1) ? m1 : m0;
  } else if (bits == 4) {
    const uint32_t m = (k0 ? 0x00000f0fu : 0u) | (k1 ? 0x0f0f0000u : 0u) | (k2 ? 0x0000f0f0u : 0u) |
                       (k3 ? 0xf0f00000u : 0u);
    for (int i = 0; i < words; ++i) v[i] &= m;
  }
}

// Scores, online-softmax update and P.V of one staged tile with ti.valid > 0
// tokens. `sc` is this wave's 128-word LDS slot for the group scales and
// offsets (null when no plane has them); qsum[c] is the sum of the lane's
// query head over dims 32c .. 32c + 31 (for INT2 K offsets).
template <int D, int KC, int VC>
__device__ __attribute__((always_inline)) inline void consume_tile(const Tile<D, KC, VC>& t, const TileInfo& ti, const h8* qv,
                                    const h8* qg, const u4* qb, const float* qsum, float scale_log2, float& m_run,
                                    float& l_run, f4* acc, uint32_t* sc, int lane) {
  constexpr int NC = D / 32, NB = D / 16;
  using T = Tile<D, KC, VC>;
  const int kq = lane >> 4;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  const bool partial = ti.valid < 16 || ti.lo > 0;  // wave-uniform
  const int vc = VC == C_ANY ? ti.vc : VC;

  uint32_t vw[T::VW];
#pragma unroll
  for (int i = 0; i < T::VW; ++i) vw[i] = t.v[i];
  if (partial) {
    constexpr int VWORDS = VC == C_ANY ? T::VW : D * bits_of(VC) / 128;
    mask_v_run(vw, VWORDS, VC == C_ANY ? bits_of(vc) : bits_of(VC), ti.lo - 4 * kq, ti.valid - 4 * kq);
  }

  // group scales (and INT2 offsets) of this lane's four tokens (4 x NC fp16
  // each for K and V); the words of tokens past the end are written as zero
  uint32_t ks[T::KS ? NC * 2 : 1], vs[T::VS ? NC * 2 : 1];
  uint32_t kz[T::KZ ? NC * 2 : 1], vz[T::VZ ? NC * 2 : 1];
  if constexpr (T::GS) {
    const int w = lane & 31;
    const int tok = (2 * w) / NC;
    const bool live = tok < ti.valid && tok >= ti.lo;
    // slot words 0..31 K scales, 32..63 V scales, 64..95 V offsets, 96..127 K offsets
    const uint32_t sk = T::KS ? t.sk[0] : 0u, sv = T::VS ? t.sv[0] : 0u;
    __builtin_amdgcn_wave_barrier();
    sc[lane] = live ? (lane < 32 ? sk : sv) : 0u;
    if constexpr (T::KZ || T::VZ) sc[64 + lane] = live ? (lane < 32 ? sv : sk) : 0u;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if constexpr (T::KS && KC != C_ANY) {
#pragma unroll
      for (int i = 0; i < NC * 2; i += 4) {
        const u4 x = *reinterpret_cast<const u4*>(sc + 2 * NC * kq + i);
        ks[i] = x[0]; ks[i + 1] = x[1]; ks[i + 2] = x[2]; ks[i + 3] = x[3];
      }
    }
    if constexpr (T::VS && VC != C_ANY) {
#pragma unroll
      for (int i = 0; i < NC * 2; i += 4) {
        const u4 x = *reinterpret_cast<const u4*>(sc + 32 + 2 * NC * kq + i);
        vs[i] = x[0]; vs[i + 1] = x[1]; vs[i + 2] = x[2]; vs[i + 3] = x[3];
      }
    }
    if constexpr (T::KZ && KC != C_ANY) {
      if (has_zero(ti.kc)) {
#pragma unroll
        for (int i = 0; i < NC * 2; i += 4) {
          const u4 x = *reinterpret_cast<const u4*>(sc + 96 + 2 * NC * kq + i);
          kz[i] = x[0]; kz[i + 1] = x[1]; kz[i + 2] = x[2]; kz[i + 3] = x[3];
        }
      }
    }
    if constexpr (T::VZ && VC != C_ANY) {
      if (has_zero(ti.vc)) {
#pragma unroll
        for (int i = 0; i < NC * 2; i += 4) {
          const u4 x = *reinterpret_cast<const u4*>(sc + 64 + 2 * NC * kq + i);
          vz[i] = x[0]; vz[i + 1] = x[1]; vz[i + 2] = x[2]; vz[i + 3] = x[3];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  float s[4];
  const bool kgrouped = KC == C_ANY ? is_int(ti.kc) : is_int(KC);
  if (KC == C_ANY || is_int(KC)) {
    // one accumulator per 32-dim group, scaled per (token, group)
    f4 scg[NC];
    if (KC == C_ANY && ti.kc == C_BF16) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u4 qh, ql;
        bf_split8(qv[c], qh, ql);
        const u4 kr = {t.k[4 * c], t.k[4 * c + 1], t.k[4 * c + 2], t.k[4 * c + 3]};
        scg[c] = mfma32_bf(kr, ql, mfma32_bf(kr, qh, zero));
      }
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        h8 kf = KC == C_ANY ? k_frag_any<D>(t.k, c, ti.kc) : k_frag<is_int(KC) ? KC : C_FP16, D>(t.k, c);
        scg[c] = mfma32(kf, (KC == C_ANY && kgrouped) ? qg[c] : qv[c], zero);
      }
    }
    if (kgrouped) {
      // the per-page kernel reads scales and offsets from the LDS slot where used (registers are short there)
      const _Float16* k16 = reinterpret_cast<const _Float16*>(KC == C_ANY ? sc + 2 * NC * kq : ks);
      const bool kzero = T::KZ && has_zero(KC == C_ANY ? ti.kc : KC);
      const _Float16* z16 = reinterpret_cast<const _Float16*>(KC == C_ANY ? sc + 96 + 2 * NC * kq : kz);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) x += (float)k16[j * NC + c] * scg[c][j];
        if (kzero) {
          // INT2: the offset of each group times the query's sum over it
#pragma unroll
          for (int c = 0; c < NC; ++c) x += (float)z16[j * NC + c] * qsum[c];
        }
        s[j] = x * scale_log2;
      }
    } else {
      const float f = scale_log2 * ti.sk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) x += scg[c][j];
        s[j] = x * f;
      }
    }
  } else if constexpr (KC == C_BF16) {
    // the codes against the query's bf16 high and low parts
    f4 acc_s = zero;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u4 qh, ql;
      if (qb) {
        qh = qb[c];
        ql = qb[NC + c];
      } else {
        bf_split8(qv[c], qh, ql);
      }
      const u4 kr = {t.k[4 * c], t.k[4 * c + 1], t.k[4 * c + 2], t.k[4 * c + 3]};
      acc_s = mfma32_bf(kr, ql, mfma32_bf(kr, qh, acc_s));
    }
    const float f = scale_log2 * ti.sk;
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = acc_s[j] * f;
  } else {
    f4 acc_s = zero;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc_s = mfma32(k_frag<KC, D>(t.k, c), qv[c], acc_s);
    const float f = scale_log2 * ti.sk;
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = acc_s[j] * f;
  }
  if (partial) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = (4 * kq + j < ti.valid && 4 * kq + j >= ti.lo) ? s[j] : NEG_INF;
  }

  // online softmax over this tile's 16 tokens (lanes col, col+16, col+32, col+48)
  const float mx = row4_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
  const float m_new = fmaxf(m_run, mx);
  if (__any(m_new > m_run)) {
    const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float aj = __shfl(alpha, 4 * kq + j);
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n][j] *= aj;
    }
    m_run = m_new;
  }
  const float mu = m_run == NEG_INF ? 0.f : m_run;
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(s[j] - mu);
  l_run += (p[0] + p[1]) + (p[2] + p[3]);

  // P.V. The weights go to the MFMA in fp16; where a V scale multiplies them
  // it is applied so that a weight of exactly 1 stays exact: INT group scales
  // are fp16 already, the fp32 FP8 page scale is split into an fp16 high and
  // low part (two MFMAs, 22 significant bits). Tail tokens have weight 0,
  // zero V codes and zero scales, so nothing non-finite reaches the MFMA.
  auto vfrag = [&](int n) {
    return VC == C_ANY ? v_frag_any<D>(vw, n, ti.vc) : v_frag<VC == C_ANY ? 0 : VC, D>(vw, n);
  };
  if (T::VZ && has_zero(vc)) {
    // INT2: V = z + s u. The offset and step terms are each rounded relative to
    // their own size, which can far exceed their sum's, so both weights go in
    // as fp16 high and low parts (22 significant bits): p s against the codes,
    // and p against the offsets of the lane's four tokens (group n / 2 of dims
    // 16n ..) as B, two MFMAs each per 16 dims.
    const _Float16* v16 = reinterpret_cast<const _Float16*>(VC == C_ANY ? sc + 32 + 2 * NC * kq : vs);
    const _Float16* z16 = reinterpret_cast<const _Float16*>(VC == C_ANY ? sc + 64 + 2 * NC * kq : vz);
    h4 ph, pl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ph[j] = (_Float16)p[j];
      pl[j] = (_Float16)(p[j] - (float)ph[j]);
    }
#pragma unroll
    for (int g = 0; g < NC; ++g) {
      h4 sh, sl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = p[j] * (float)v16[j * NC + g];
        sh[j] = (_Float16)x;
        sl[j] = (_Float16)(x - (float)sh[j]);
      }
      const h4 zf = {z16[0 * NC + g], z16[1 * NC + g], z16[2 * NC + g], z16[3 * NC + g]};
#pragma unroll
      for (int n = 2 * g; n < 2 * g + 2; ++n) {
        const h4 vf = vfrag(n);
        acc[n] = mfma16(sh, vf, acc[n]);
        acc[n] = mfma16(sl, vf, acc[n]);
        acc[n] = mfma16(ph, zf, acc[n]);
        acc[n] = mfma16(pl, zf, acc[n]);
      }
    }
  } else if (is_int(vc)) {
    const _Float16* v16 = reinterpret_cast<const _Float16*>(VC == C_ANY ? sc + 32 + 2 * NC * kq : vs);
    h4 pa[NC];
#pragma unroll
    for (int g = 0; g < NC; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) pa[g][j] = (_Float16)__builtin_fmaf(p[j], (float)v16[j * NC + g], 0.0f);
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = mfma16(pa[n / 2], vfrag(n), acc[n]);
  } else if (vc == C_BF16) {
    // the codes against the weights' bf16 high and low parts
    u2 ph, pl;
    bf_split4(p, ph, pl);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const u2 vr = {vw[2 * n], vw[2 * n + 1]};
      acc[n] = mfma16_bf(pl, vr, mfma16_bf(ph, vr, acc[n]));
    }
  } else if (vc == C_FP8) {
    h4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = p[j] * ti.sv;
      hi[j] = (_Float16)x;
      lo[j] = (_Float16)(x - (float)hi[j]);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const h4 vf = vfrag(n);
      acc[n] = mfma16(hi, vf, acc[n]);
      acc[n] = mfma16(lo, vf, acc[n]);
    }
  } else {
    const h4 pa = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = mfma16(pa, vfrag(n), acc[n]);
  }
}

// A tile of a kernel built for any codec, consumed by the code of the pair
// (K2, V2) its page holds: its raw words are that pair's run layout.
template <int D, int K2, int V2, int KC, int VC>
__device__ __attribute__((always_inline)) inline void consume_as(const Tile<D, KC, VC>& t, const TileInfo& ti, const h8* qv, const h8* qg,
                                  const float* qsum, float scale_log2, float& m_run, float& l_run, f4* acc,
                                  int lane) {
  Tile<D, K2, V2> u;
#pragma unroll
  for (int i = 0; i < Tile<D, K2, V2>::KW; ++i) u.k[i] = t.k[i];
#pragma unroll
  for (int i = 0; i < Tile<D, K2, V2>::VW; ++i) u.v[i] = t.v[i];
  consume_tile<D, K2, V2>(u, ti, qv, qg, nullptr, qsum, scale_log2, m_run, l_run, acc, nullptr, lane);
}

// Consume one tile. With codecs known only at run time, pages of the common
// one-scale pairs (FP8, FP16, BF16 for both planes) branch once to their own
// code: no group-scale exchange and no per-fragment codec dispatch; other
// pairs take the generic path (C_ANY; the C_FLT kernel has no others: the
// gather skipped and counted them).
template <int D, int KC, int VC>
__device__ __attribute__((always_inline)) inline void consume(const Tile<D, KC, VC>& t, const TileInfo& ti, const h8* qv, const h8* qg,
                               const u4* qb, const float* qsum, float scale_log2, float& m_run, float& l_run,
                               f4* acc, uint32_t* sc, int lane) {
  if constexpr ((KC == C_ANY && VC == C_ANY) || (KC == C_FLT && VC == C_FLT)) {
    if (ti.kc == C_FP8 && ti.vc == C_FP8)
      return consume_as<D, C_FP8, C_FP8>(t, ti, qv, qg, qsum, scale_log2, m_run, l_run, acc, lane);
    if (ti.kc == C_FP16 && ti.vc == C_FP16)
      return consume_as<D, C_FP16, C_FP16>(t, ti, qv, qg, qsum, scale_log2, m_run, l_run, acc, lane);
    // (BF16 pages of the any-codec kernel take its generic path, which feeds
    // BF16 planes to the bf16 MFMA: one copy of that code fewer)
    if (KC == C_FLT && ti.kc == C_BF16 && ti.vc == C_BF16)
      return consume_as<D, C_BF16, C_BF16>(t, ti, qv, qg, qsum, scale_log2, m_run, l_run, acc, lane);
  }
  if constexpr (KC == C_ANY) {
    // pages of codes shorter than 16 bytes per lane: the runs out of their chunks
    Tile<D, KC, VC> u = t;
    short_run<D>(u.k, ti.kc, lane);
    short_run<D>(u.v, ti.vc, lane);
    consume_tile<D, KC, VC>(u, ti, qv, qg, nullptr, qsum, scale_log2, m_run, l_run, acc, sc, lane);
  } else if constexpr (KC != C_FLT) {
    consume_tile<D, KC, VC>(t, ti, qv, qg, qb, qsum, scale_log2, m_run, l_run, acc, sc, lane);
  }
}

template <int D, int KC, int VC>
__global__ void __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<D, KC, VC>(), max_waves_per_eu<D, KC, VC>()))) decode_kernel(const DecodeArgs a) {
  constexpr int NC = D / 32, NB = D / 16;
  // the waves' states merge through LDS in one pass over all head dims
  // (33 KB per workgroup at D 128: four FP8 workgroups per compute unit still
  // fit; two passes over half the dims, 17 KB, measured 1-2% slower)
  constexpr int RED_BYTES = (WAVES * 16 * D + 2 * WAVES * 16) * 4;
  constexpr int DESC_BYTES = MAX_DESC * (int)sizeof(Desc);
  __shared__ __attribute__((aligned(16))) unsigned char smem[RED_BYTES > DESC_BYTES ? RED_BYTES : DESC_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t scale_slots[Tile<D, KC, VC>::GS ? WAVES * 128 : 4];
  Desc* desc = reinterpret_cast<Desc*>(smem);

  const int part = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps loop control scalar
  uint32_t* const sc = Tile<D, KC, VC>::GS ? scale_slots + 128 * wave : nullptr;
  const int col = lane & 15, kq = lane >> 4;
  const int G = a.group;
  const int P = a.page;

  // ---- row length and selection length: vector buffer loads. Scalar loads
  // complete out of order, so a scalar load of the row length would make the
  // first use of any kernel argument wait for it too; these are counted in
  // order and waited for only where used.
  const uint32_t len_raw = bload4(make_rsrc(reinterpret_cast<const uint8_t*>(a.seq_lens), (uint32_t)a.rows * 4u), 4u * b);
  uint32_t sel_raw = 0;
  if (a.sparse)
    sel_raw = bload4(make_rsrc(reinterpret_cast<const uint8_t*>(a.sel_lens), (uint32_t)a.rows * 4u), 4u * b);

  // ---- extent of this row and of this partition (wave-uniform values).
  // A row's 16-token tiles run through its pages (dense) or its selected
  // pages in list order (sparse), tpp per page; only tiles that can hold
  // attended tokens count. Partitions are either a fixed number of tiles
  // (tiles_per_part) or, with tiles_per_part = 0, the row's tiles split
  // evenly into nparts, so rows of different lengths give workgroups of
  // equal work. A sliding window keeps positions >= wlo; in dense mode the
  // partitions start at its first tile.
  const int tpp = P / 16;
  int L = 0, npg = 0, ntl = 0, wlo = 0, lo_tile = 0;
  bool bad_row = false;
  auto extent = [&]() {
    L = __builtin_amdgcn_readfirstlane((int)len_raw);
    bad_row = L < 0;
    L = L < 0 ? 0 : L;
    if (a.sparse) {
      const int n = __builtin_amdgcn_readfirstlane((int)sel_raw);
      bad_row = bad_row || n < 0 || n > a.max_sel;
      npg = min(max(n, 0), a.max_sel);
    } else {
      const int n = L / P + (L % P != 0);
      bad_row = bad_row || n > a.max_pages;
      npg = min(n, a.max_pages);
    }
    npg = __builtin_amdgcn_readfirstlane(npg);
    ntl = a.sparse ? npg * tpp : min(L / 16 + (L % 16 != 0), npg * tpp);
    if (a.window > 0) {
      wlo = __builtin_amdgcn_readfirstlane(max(L - a.window, 0));
      if (!a.sparse) lo_tile = min(wlo / 16, ntl);
    }
  };
  // Fixed partitions without a window do not depend on the row length: their
  // first chunk's table reads go out before it is known (they and the length
  // reads then cost one round together); the others wait for it first.
  const bool early = a.tiles_per_part > 0 && a.window <= 0;
  if (!early) extent();
  const int tpart = a.tiles_per_part > 0 ? a.tiles_per_part : max(1, (ntl - lo_tile + a.nparts - 1) / a.nparts);
  const int t0 = lo_tile + part * tpart;

  // ---- page descriptors of this partition, MAX_DESC at a time. Entries run
  // as far as the tables go; the row length may cut them shorter. Every read
  // of a chunk is issued before any result is checked, so the gather costs
  // two dependent rounds (three with a selection).
  const int s0 = t0 / tpp;
  const int s_lim = min((t0 + tpart + tpp - 1) / tpp, a.sparse ? a.max_sel : a.max_pages);
  struct Raw {
    int lp, pp, cod;
    uint64_t ko, vo;
    float sk, sv;
  };
  auto stage_issue = [&](int cbase, int chunk, Raw& r) {
    if (tid < chunk) {
      const int s = cbase + tid;
      // reads (indices clamped into their tables; results checked later)
      r.lp = a.sparse ? a.sel[(size_t)b * a.max_sel + s] : s;
      const bool lp_ok = (unsigned)r.lp < (unsigned)a.max_pages;
      r.pp = a.bt[(size_t)b * a.max_pages + (lp_ok ? r.lp : 0)];
      const bool pp_ok = lp_ok && (unsigned)r.pp < (unsigned)a.num_pages;
      const int pq = pp_ok ? r.pp : 0;
      r.cod = a.codec[pq];
      r.ko = a.koff[pq];
      r.vo = a.voff[pq];
      r.sk = 1.f;
      r.sv = 1.f;
      if (a.scale != nullptr) {
        r.sk = a.scale[((size_t)pq * a.hkv + h) * 2 + 0];
        r.sv = a.scale[((size_t)pq * a.hkv + h) * 2 + 1];
      }
    }
  };
  // s1: the end of the row's entries (a bad entry before it is an input error)
  auto stage_check = [&](int cbase, int chunk, int s1, const Raw& r) {
    if (tid < chunk) {
      const int s = cbase + tid;
      const bool lp_ok = (unsigned)r.lp < (unsigned)a.max_pages;
      const bool pp_ok = lp_ok && (unsigned)r.pp < (unsigned)a.num_pages;
      const int lp = r.lp, cod = r.cod;
      const uint64_t ko = r.ko, vo = r.vo;
      const int kc = cod & 15, vc = cod >> 4;
      bool ok = pp_ok && kc <= C_LAST && vc <= C_LAST;
      if (KC == C_FLT && !(kc == vc && kc <= C_FP8)) ok = false;  // a float page, one codec for both planes
      if (!per_page(KC) && kc != KC) ok = false;
      if (!per_page(VC) && vc != VC) ok = false;
      if ((kc == C_FP8 || vc == C_FP8) && a.scale == nullptr) ok = false;
      if ((ko | vo) & 15) ok = false;
      if (ok && (ko > a.pool_bytes || a.pool_bytes - ko < plane_bytes(kc, a.hkv, P, D))) ok = false;
      if (ok && (vo > a.pool_bytes || a.pool_bytes - vo < plane_bytes(vc, a.hkv, P, D))) ok = false;
      const bool live = s < s1;
      Desc d;
      d.k = 0; d.v = 0; d.sk = 1.f; d.sv = 1.f; d.valid = 0; d.codec = 0;
      if (ok && live) {
        const long long rem = (long long)L - (long long)lp * P;
        const long long before = (long long)wlo - (long long)lp * P;  // slots before the window
        const int lo = (int)(before < 0 ? 0 : (before > P ? P : before));
        d.valid = (int)(rem < 0 ? 0 : (rem > P ? P : rem));
        d.valid = d.valid > lo ? d.valid : 0;  // a page wholly before the window is skipped
        d.k = ko;
        d.v = vo;
        if (kc == C_FP8) d.sk = r.sk;
        if (vc == C_FP8) d.sv = r.sv;
        d.codec = cod | (lo << 8);
      } else if (live && h == 0) {
        count_error(a.err);
      }
      desc[tid] = d;
    }
  };
  int cbase = s0;
  int chunk = min(MAX_DESC, s_lim - cbase);
  int s1, t1;
  {
    Raw raw = {};
    if (chunk > 0) stage_issue(cbase, chunk, raw);
    if (early) extent();
    t1 = min(t0 + tpart, ntl);
    // table entries the partition touches inside the row: [s0, s1)
    s1 = t1 > t0 ? (t1 + tpp - 1) / tpp : s0;
    if (chunk > 0) stage_check(cbase, chunk, s1, raw);
  }

  // ---- q of this KV head's query group (B operand of the score MFMA), in
  // the dim order of the K runs: qv for one-scale codecs (and the per-page
  // dispatch variant), qg for group-scale codecs
  h8 qv[NC];
  h8 qg[KC == C_ANY ? NC : 1];
  {
    const _Float16* qrow = reinterpret_cast<const _Float16*>(a.q) + ((size_t)b * a.hq + (size_t)h * G + col) * D;
    constexpr bool PERM = KC == C_ANY || k_perm<KC>();
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int d0 = PERM ? (D / 4) * kq + 8 * c : 32 * c + 8 * kq;
      qv[c] = col < G ? *reinterpret_cast<const h8*>(qrow + d0) : h8{0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (KC == C_ANY)
        qg[c] = col < G ? *reinterpret_cast<const h8*>(qrow + 32 * c + 8 * kq) : h8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }


  // query sums over each 32-dim group, for the offsets of INT2 K pages: the
  // lane's eight dims of the grouped order, then the four rows of its column.
  // The per-page kernel, at the edge of its registers, keeps them in LDS
  // (read only for INT2 pages; the chunk loop's barrier orders the writes).
  float qsum_reg[KC == C_INT2 ? NC : 1];
  __shared__ float qsum_lds[KC == C_ANY ? WAVES * 16 * NC : 1];
  if constexpr (KC == C_INT2 || KC == C_ANY) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const h8 x = KC == C_ANY ? qg[c] : qv[c];
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) part += (float)x[j];
      const float qs = row4_sum(part);
      if constexpr (KC == C_INT2) qsum_reg[c] = qs;
      else if (lane < 16) qsum_lds[(wave * 16 + lane) * NC + c] = qs;
    }
  }
  const float* const qsum = KC == C_ANY ? qsum_lds + (wave * 16 + col) * NC : qsum_reg;

  // the BF16 kernel's query as bf16 high and low parts, once (the per-page
  // kernels split it for their BF16 pages as they come)
  u4 qb[KC == C_BF16 ? 2 * NC : 1];
  if constexpr (KC == C_BF16) {
#pragma unroll
    for (int c = 0; c < NC; ++c) bf_split8(qv[c], qb[c], qb[NC + c]);
  }

  float m_run = NEG_INF, l_run = 0.f;
  f4 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f4{0.f, 0.f, 0.f, 0.f};

  while (chunk > 0) {
    lds_barrier();
    // the partition's tiles among this chunk's: [klo, khi), counted from the
    // chunk's first tile
    const int kb = cbase * tpp;
    const int klo = max(t0 - kb, 0);
    const int khi = min(t1 - kb, chunk * tpp);

    // Ring of DEPTH tiles: while the oldest is consumed, the loads of the
    // next DEPTH-1 are in flight. Issues are unconditional (past the end the
    // wave issues its last tile again through a zero-size resource and never
    // consumes it), so the compiler's wait counts stay exact.
    const int ntiles = khi - klo;
    if (wave < ntiles) {
      constexpr int DEPTH = ring_depth<D, KC, VC>();
      const int nmine = (ntiles - wave + WAVES - 1) / WAVES;
      const int kfirst = klo + wave;
      const int klast = kfirst + (nmine - 1) * WAVES;
      Tile<D, KC, VC> t[DEPTH];
      TileInfo inf[DEPTH];
#pragma unroll
      for (int s = 0; s < DEPTH - 1; ++s)
        inf[s] = issue_tile<D, KC, VC>(t[s], desc, min(kfirst + s * WAVES, klast), tpp, a, h, lane,
                                       kfirst + s * WAVES > klast);
      for (int it = 0; it < nmine; it += DEPTH) {
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
          const int kn = kfirst + (it + s + DEPTH - 1) * WAVES;
          const int nx = (s + DEPTH - 1) % DEPTH;
          // past the end: same loads through a zero-size resource (no traffic)
          inf[nx] = issue_tile<D, KC, VC>(t[nx], desc, min(kn, klast), tpp, a, h, lane, kn > klast);
          if (it + s < nmine && inf[s].valid > 0)
            consume<D, KC, VC>(t[s], inf[s], qv, qg, KC == C_BF16 ? qb : nullptr, qsum, a.scale_log2, m_run, l_run,
                               acc, sc, lane);
        }
      }
    }
    if (cbase + chunk >= s1) break;  // the row ends inside this chunk
    // Before the next chunk, drain the ring's discarded loads (zero-size
    // reads, no traffic): with nothing in flight across the loop edge, the
    // wait counts at the top of the loop only cover q, not the tile
    // registers. After the last chunk nothing waits for them here.
    __builtin_amdgcn_s_waitcnt(VMCNT0);
    cbase += MAX_DESC;
    chunk = min(MAX_DESC, s_lim - cbase);
    if (chunk <= 0) break;
    lds_barrier();  // every wave is done with the previous chunk
    Raw raw = {};
    stage_issue(cbase, chunk, raw);
    stage_check(cbase, chunk, s1, raw);
  }

  // reported here, not where found, so that no wait on the row length sits
  // in front of the table reads
  if (bad_row && part == 0 && h == 0 && tid == 0) count_error(a.err);

  // ---- merge the four waves' (m, l, acc) through LDS
  l_run = row4_sum(l_run);
  float* red_acc = reinterpret_cast<float*>(smem);
  float* red_m = red_acc + WAVES * 16 * D;
  float* red_l = red_m + WAVES * 16;
  lds_barrier();  // the descriptors are no longer read
  if (lane < 16) {
    red_m[wave * 16 + lane] = m_run;
    red_l[wave * 16 + lane] = l_run;
  }
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int j = 0; j < 4; ++j) red_acc[(wave * 16 + 4 * kq + j) * D + 16 * n + col] = acc[n][j];
  lds_barrier();

  // at most 16 * D / THREADS outputs per thread (G <= 16), unrolled so that
  // the LDS reads of all of them go out together
#pragma unroll
  for (int it = 0; it < 16 * D / THREADS; ++it) {
    const int idx = tid + it * THREADS;
    if (idx >= G * D) break;
    const int g = idx / D, d = idx - g * D;
    // every wave's (m, l, acc) read at once (one LDS round, no branches); a
    // wave with nothing attended (m = -inf, l = 0, acc = 0) weighs 0
    float mw[WAVES], lw[WAVES], aw[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      mw[w] = red_m[w * 16 + g];
      lw[w] = red_l[w * 16 + g];
      aw[w] = red_acc[(w * 16 + g) * D + d];
    }
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mw[w]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float e = mw[w] != NEG_INF ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.f;
      Ls += e * lw[w];
      A += e * aw[w];
    }
    const size_t row = (size_t)b * a.hq + (size_t)h * G + g;
    if (a.final_out) {
      a.out[row * D + d] = Ls > 0.f ? A / Ls : 0.f;
      if (d == 0) a.lse[row] = Ls > 0.f ? M * LN2 + logf(Ls) : NEG_INF;
    } else {
      const size_t pi = row * a.nparts + part;
      a.part_acc[pi * D + d] = A;
      if (d == 0) {
        a.part_ml[2 * pi + 0] = Ls > 0.f ? M * LN2 : NEG_INF;
        a.part_ml[2 * pi + 1] = Ls;
      }
    }
  }
}

// ---------------------------------------------------------------- fold
// Fold for many parts where the wide fold below does not apply (head_dim not
// a multiple of 32, partials not 16-byte (acc) or 8-byte (m, l) aligned, more
// than 512 parts). Grid (row, 4-dim group), one wave each: spread over the
// whole chip, one round of loads, no LDS. Lane l keeps a running log-sum-exp over the parts
// p = l + 64k (every load of a batch in flight together); the 64 lanes then
// merge by a fixed butterfly (lane distance 32, 16, ..., 1), so results are
// run-to-run identical.
// A part is empty (and its acc never read) unless l > 0 and m is finite.
__device__ inline bool live_part(float m, float l) { return l > 0.f && __builtin_isfinite(m); }

__device__ inline void lse_merge(float& M, float& L, f4& A, float m2, float l2, f4 a2) {
  if (!live_part(m2, l2)) return;
  if (!(L > 0.f)) { M = m2; L = l2; A = a2; return; }
  const float mx = fmaxf(M, m2);
  const float c1 = __expf(M - mx), c2 = __expf(m2 - mx);
  L = L * c1 + l2 * c2;
  A = A * c1 + a2 * c2;
  M = mx;
}

template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Merge this lane's (M, L, A) with its partner's under the lane map `partner`.
template <class F>
__device__ inline void fold_step(float& M, float& L, f4& A, F partner) {
  const float m2 = partner(M), l2 = partner(L);
  const f4 a2 = {partner(A[0]), partner(A[1]), partner(A[2]), partner(A[3])};
  lse_merge(M, L, A, m2, l2, a2);
}

// `vec`: D % 4 == 0 and part_acc 16-byte aligned, so 4 dims load as one vector.
__global__ void __launch_bounds__(64) combine_kernel(int nparts, int D, int vec, const float* __restrict__ part_acc,
                                                     const float* __restrict__ part_ml, float* __restrict__ out,
                                                     float* __restrict__ lse) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const int d0 = 4 * blockIdx.y;
  const float* ml = part_ml + (size_t)row * nparts * 2;
  const float* acc = part_acc + (size_t)row * nparts * D + d0;
  float M = NEG_INF, L = 0.f;
  f4 A = {0.f, 0.f, 0.f, 0.f};
  constexpr int BATCH = 8;
  for (int p0 = lane; p0 < nparts; p0 += 64 * BATCH) {
    float m[BATCH], l[BATCH];
    f4 x[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = p0 + 64 * u;
      const bool in = p < nparts;
      m[u] = in ? ml[2 * (size_t)p] : NEG_INF;
      l[u] = in ? ml[2 * (size_t)p + 1] : 0.f;
      const float* ap = acc + (size_t)(in ? p : 0) * D;
      if (in && vec) {
        x[u] = *reinterpret_cast<const f4*>(ap);
      } else {
        x[u] = f4{in && d0 + 0 < D ? ap[0] : 0.f, in && d0 + 1 < D ? ap[1] : 0.f,
                  in && d0 + 2 < D ? ap[2] : 0.f, in && d0 + 3 < D ? ap[3] : 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) lse_merge(M, L, A, m[u], l[u], x[u]);
  }
  // butterfly: lane pairs inside quads (DPP quad permutes), across quads and
  // half-rows (DPP mirrors), then across 16-lane rows and 32-lane halves
  // (row swaps). Every step is an involution, so after six steps every lane
  // holds the merge of all 64.
  fold_step(M, L, A, [](float x) { return dpp_f<0xB1>(x); });   // quad_perm [1,0,3,2]
  fold_step(M, L, A, [](float x) { return dpp_f<0x4E>(x); });   // quad_perm [2,3,0,1]
  fold_step(M, L, A, [](float x) { return dpp_f<0x141>(x); });  // row_half_mirror
  fold_step(M, L, A, [](float x) { return dpp_f<0x140>(x); });  // row_mirror
  fold_step(M, L, A, [lane](float x) { float a, b; swap_rows<16>(x, a, b); return (lane & 16) ? a : b; });
  fold_step(M, L, A, [lane](float x) { float a, b; swap_rows<32>(x, a, b); return (lane & 32) ? a : b; });
  if (lane == 0) {
    const bool any = L > 0.f;
    float* o = out + (size_t)row * D + d0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (d0 + j < D) o[j] = any ? A[j] / L : 0.f;
    if (blockIdx.y == 0) lse[row] = any ? M + logf(L) : NEG_INF;
  }
}

// Fold for many parts (up to 32 KP per row) of rows whose head_dim is a
// multiple of 32: a workgroup of 256 threads per (row, 32 dims). Thread t
// takes dims 4 (t % 8) .. +3 of the slice for parts t / 8 + 32 k, so
// the eight threads of a part read its 128 contiguous bytes and every load
// instruction reads eight such spans, whole cache lines when part_acc is
// 128-byte aligned as the library's workspace is (a wave per 4 dims touches
// 64 lines per load and fetches each line eight times). All of a thread's loads are in
// flight together. The row's maximum M is taken first (exact in any order),
// then each live part enters with weight exp(m_p - M), with no chain of
// rescales; the part-slices' sums are added in LDS in ascending order, so
// results are run-to-run identical. part_ml is 8-byte aligned: (m, l) load
// as one pair. (512 threads, half the parts per thread, measured no faster
// on 512 parts.)
template <int KP>
__global__ void __launch_bounds__(256) combine_wide_kernel(int nparts, int D, const float* __restrict__ part_acc,
                                                          const float* __restrict__ part_ml,
                                                          float* __restrict__ out, float* __restrict__ lse) {
  constexpr int SL = 32, NW = 4;  // part-slices, waves
  __shared__ float wmax[NW];
  __shared__ float sl[SL][8];
  __shared__ f4 sa[SL][8];
  const int t = threadIdx.x, q = t & 7, sl_i = t >> 3;
  const int row = blockIdx.x, d0 = 32 * blockIdx.y + 4 * q;
  const float* ml = part_ml + (size_t)row * nparts * 2;
  const float* acc = part_acc + (size_t)row * nparts * D + d0;
  float m[KP], l[KP];
  f4 x[KP];
#pragma unroll
  for (int u = 0; u < KP; ++u) {
    const int p = sl_i + SL * u;
    const bool in = p < nparts;
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 v = in ? *reinterpret_cast<const f2*>(ml + 2 * (size_t)p) : f2{NEG_INF, 0.f};
    m[u] = v[0];
    l[u] = v[1];
    x[u] = in ? *reinterpret_cast<const f4*>(acc + (size_t)p * D) : f4{0.f, 0.f, 0.f, 0.f};
  }
  float mx = NEG_INF;
#pragma unroll
  for (int u = 0; u < KP; ++u)
    if (live_part(m[u], l[u])) mx = fmaxf(mx, m[u]);
  mx = fmaxf(mx, dpp_f<0xB1>(mx));   // quad_perm [1,0,3,2]
  mx = fmaxf(mx, dpp_f<0x4E>(mx));   // quad_perm [2,3,0,1]
  mx = fmaxf(mx, dpp_f<0x141>(mx));  // row_half_mirror
  mx = fmaxf(mx, dpp_f<0x140>(mx));  // row_mirror
  mx = row4_max(mx);
  if ((t & 63) == 0) wmax[t >> 6] = mx;
  __syncthreads();
  float M = wmax[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) M = fmaxf(M, wmax[k]);
  float L = 0.f;
  f4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KP; ++u) {
    if (live_part(m[u], l[u])) {  // an empty part's acc is never used
      const float w = __expf(m[u] - M);
      L = fmaf(w, l[u], L);
#pragma unroll
      for (int j = 0; j < 4; ++j) A[j] = fmaf(w, x[u][j], A[j]);
    }
  }
  sl[sl_i][q] = L;
  sa[sl_i][q] = A;
  __syncthreads();
  if (t < 32) {  // thread (q, j): dim 4 q + j of the slice
    const int qq = t & 7, j = t >> 3;
    float Ls = 0.f, As = 0.f;
#pragma unroll 8
    for (int k = 0; k < SL; ++k) {
      Ls += sl[k][qq];
      As += sa[k][qq][j];
    }
    const bool any = Ls > 0.f;
    out[(size_t)row * D + 32 * blockIdx.y + 4 * qq + j] = any ? As / Ls : 0.f;
    if (blockIdx.y == 0 && t == 0) lse[row] = any ? M + logf(Ls) : NEG_INF;
  }
}

// Fold for few parts per row: one thread per (row, dim), the loads of BATCH
// parts issued before they are used (up to 32 parts in one round), parts
// summed in ascending order. With every part in one batch the row's maximum
// comes first (as in the wide fold); more parts take a running log-sum-exp.
constexpr int FOLD_SMALL_MAX = 64;

template <int BATCH>
__global__ void __launch_bounds__(256) combine_small_kernel(int rows, int nparts, int D, int ml2,
                                                            const float* __restrict__ part_acc,
                                                            const float* __restrict__ part_ml,
                                                            float* __restrict__ out, float* __restrict__ lse) {
  // grid (row groups of 4, dim groups of 64): thread (row, dim) without a division
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int d = (int)blockIdx.y * 64 + (int)(threadIdx.x & 63);
  if (row >= rows || d >= D) return;
  const float* ml = part_ml + row * nparts * 2;
  const float* acc = part_acc + row * nparts * D + d;
  float M = NEG_INF, L = 0.f, A = 0.f;
  if (nparts <= BATCH) {
    // every part in one round of loads: the maximum first, then each live
    // part with weight exp(m_p - M) in ascending order (no rescale chain)
    float m[BATCH], l[BATCH], x[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const bool in = u < nparts;
      if (ml2) {  // part_ml 8-byte aligned: (m, l) as one pair
        typedef float f2 __attribute__((ext_vector_type(2)));
        const f2 v = in ? *reinterpret_cast<const f2*>(ml + 2 * u) : f2{NEG_INF, 0.f};
        m[u] = v[0];
        l[u] = v[1];
      } else {
        m[u] = in ? ml[2 * u] : NEG_INF;
        l[u] = in ? ml[2 * u + 1] : 0.f;
      }
      x[u] = in ? acc[(long long)u * D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      if (live_part(m[u], l[u])) M = fmaxf(M, m[u]);
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      if (live_part(m[u], l[u])) {
        const float w = __expf(m[u] - M);
        L = fmaf(w, l[u], L);
        A = fmaf(w, x[u], A);
      }
    }
  } else {
    for (int p0 = 0; p0 < nparts; p0 += BATCH) {
      float m[BATCH], l[BATCH], x[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int p = p0 + u;
        m[u] = p < nparts ? ml[2 * p] : NEG_INF;
        l[u] = p < nparts ? ml[2 * p + 1] : 0.f;
        x[u] = p < nparts ? acc[(long long)p * D] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (live_part(m[u], l[u])) {
          // running log-sum-exp over the parts seen so far
          if (m[u] > M) {
            const float c = M == NEG_INF ? 0.f : __expf(M - m[u]);
            L *= c;
            A *= c;
            M = m[u];
          }
          const float w = __expf(m[u] - M);
          L += w * l[u];
          A += w * x[u];
        }
      }
    }
  }
  const bool any = M != NEG_INF && L > 0.f;
  out[row * D + d] = any ? A / L : 0.f;
  if (d == 0) lse[row] = any ? M + logf(L) : NEG_INF;
}

template <int D, int KC, int VC>
int launch_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.nparts, a.hkv, a.rows);
  hipLaunchKernelGGL((decode_kernel<D, KC, VC>), grid, dim3(THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int D>
int launch_d(const DecodeArgs& a, int kc, int vc, hipStream_t s) {
#define PKV_PAIR(K, V) \
  if (kc == K && vc == V) return launch_t<D, K, V>(a, s);
  PKV_PAIR(C_FP16, C_FP16)
  PKV_PAIR(C_BF16, C_BF16)
  PKV_PAIR(C_FP8, C_FP8)
  PKV_PAIR(C_INT8, C_INT4)
  PKV_PAIR(C_INT8, C_INT8)
  PKV_PAIR(C_INT4, C_INT4)
  PKV_PAIR(C_INT2, C_INT2)
  PKV_PAIR(C_BIT1, C_BIT1)
#undef PKV_PAIR
  if (kc == C_FLT && vc == C_FLT) return launch_t<D, C_FLT, C_FLT>(a, s);
  return launch_t<D, C_ANY, C_ANY>(a, s);
}

// Built-in scratch of the allocation-free decode entry point: the split-K
// partials of one call. Every GPU the library runs on holds its own copy
// until the process ends. Host code never passes this name to a kernel (on
// the host it is only a stand-in for the symbol); it uses the device address
// noalloc_scratch() returns.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

}  // namespace

int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return -4;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // once per device, with that device current: the address of this
    // device's copy of the array
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -4;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return 0;
}

int launch_decode(const DecodeArgs& a, int head_dim, int k_codec, int v_codec, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int kc = k_codec == -2 ? C_FLT : (k_codec < 0 ? C_ANY : k_codec);
  const int vc = v_codec == -2 ? C_FLT : (v_codec < 0 ? C_ANY : v_codec);
  if (head_dim == 128) return launch_d<128>(a, kc, vc, s);
  if (head_dim == 64) return launch_d<64>(a, kc, vc, s);
  return -2;
}

int launch_combine(int rows, int nparts, int head_dim, const float* part_acc, const float* part_ml,
                   float* out, float* lse, void* stream) {
  if (rows == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // one thread per (row, dim) walks the parts eight at a time: right when
  // that is one round of loads, or when there are threads enough to fill the
  // chip; few rows with many parts go to one wave per (row, 4 dims)
  const bool wide_ok = head_dim % 32 == 0 && reinterpret_cast<uintptr_t>(part_acc) % 16 == 0 &&
                       reinterpret_cast<uintptr_t>(part_ml) % 8 == 0 && nparts <= 512;
  // (17 to 64 parts go to the wide fold where it applies: 336 rows x 21
  // parts at head_dim 64 took 3.9 us there against 5.2 us here; up to 16
  // parts this one is faster, 256 rows x 12 parts 3.6 against 3.9 us)
  const bool small = (nparts <= 8 || (nparts <= FOLD_SMALL_MAX && (long long)rows * head_dim >= 16384)) &&
                     !(wide_ok && nparts > 16);
  if (small) {
    const dim3 grid((unsigned)((rows + 3) / 4), (unsigned)((head_dim + 63) / 64));
    const int ml2 = reinterpret_cast<uintptr_t>(part_ml) % 8 == 0;
    if (nparts <= 8)
      hipLaunchKernelGGL(combine_small_kernel<8>, grid, dim3(256), 0, s, rows, nparts, head_dim, ml2, part_acc,
                         part_ml, out, lse);
    else if (nparts <= 16)
      hipLaunchKernelGGL(combine_small_kernel<16>, grid, dim3(256), 0, s, rows, nparts, head_dim, ml2, part_acc,
                         part_ml, out, lse);
    else
      hipLaunchKernelGGL(combine_small_kernel<32>, grid, dim3(256), 0, s, rows, nparts, head_dim, ml2, part_acc,
                         part_ml, out, lse);
  } else if (wide_ok) {
    // many parts, whole 128-byte lines per load: a workgroup per (row, 32 dims)
    const dim3 grid(rows, head_dim / 32);
    if (nparts <= 128)
      hipLaunchKernelGGL(combine_wide_kernel<4>, grid, dim3(256), 0, s, nparts, head_dim, part_acc, part_ml, out, lse);
    else if (nparts <= 256)
      hipLaunchKernelGGL(combine_wide_kernel<8>, grid, dim3(256), 0, s, nparts, head_dim, part_acc, part_ml, out, lse);
    else
      hipLaunchKernelGGL(combine_wide_kernel<16>, grid, dim3(256), 0, s, nparts, head_dim, part_acc, part_ml, out, lse);
  } else {
    const int vec = (head_dim % 4 == 0) && (reinterpret_cast<uintptr_t>(part_acc) % 16 == 0);
    hipLaunchKernelGGL(combine_kernel, dim3(rows, (head_dim + 3) / 4), dim3(64), 0, s, nparts, head_dim, vec,
                       part_acc, part_ml, out, lse);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
