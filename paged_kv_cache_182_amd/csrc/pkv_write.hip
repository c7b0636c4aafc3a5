// Write side of the paged cache, gfx950: token append into 16-bit pages and
// re-encoding (demotion) of full 16-bit pages to FP8 / INT8 / INT4 / 16-bit.
//
// Recent pages stay FP16 while they fill; full older pages are re-encoded
// into a compact codec (ARGUS "Adaptive activation" and "v0.5"). FP8 pages
// hold e4m3 codes with one fp32 scale per (page, KV head, plane) (FreeToken
// PR #499 update, item 1); INT8/INT4 pages hold one fp16 scale per token and
// group of 32 dims (GGML Q8/Q4 pages, ARGUS "Direct paged attention").
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
// INT4 packs eight elements per 32-bit word, element r of word w in nibble
// slot (r%2)*4 + r/2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

enum : int { W_FP16 = 0, W_BF16 = 1, W_FP8 = 2, W_INT8 = 3, W_INT4 = 4 };

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ inline int wbits(int c) { return c <= W_BF16 ? 16 : (c == W_INT4 ? 4 : 8); }
__device__ inline bool w16(int c) { return c == W_FP16 || c == W_BF16; }
__device__ inline bool wint(int c) { return c == W_INT8 || c == W_INT4; }

__device__ inline uint64_t wplane_bytes(int c, int hkv, int page, int d) {
  const uint64_t codes = (uint64_t)hkv * page * d * wbits(c) / 8;
  return codes + (wint(c) ? (uint64_t)hkv * page * (d / 32) * 2 : 0);
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

// fp32 -> OCP e4m3 code, nearest even; |y| <= 448, finite.
__device__ inline uint32_t f_to_e4m3(float y) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (bits >> 31) << 7;
  const float a = __builtin_fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {                 // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8; 8 is the smallest normal
  } else {
    int E = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;   // -6 .. 8
    float r = __builtin_rintf(__builtin_ldexpf(a, 3 - E));                 // 8 .. 16
    if (r >= 16.0f) { r = 8.0f; ++E; }
    code = (uint32_t)((E + 7) << 3) + (uint32_t)r - 8u;
  }
  return sign | code;
}

__device__ inline void count_err(int32_t* err) {
  if (err) atomicAdd(err, 1);
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
    const int cb = a.codec[pp];
    codec = plane ? (cb >> 4) : (cb & 15);
    ok = w16(cb & 15) && w16(cb >> 4);
    off = plane ? a.voff[pp] : a.koff[pp];
    ok = ok && (off & 15) == 0 && off <= a.pool_bytes && a.pool_bytes - off >= wplane_bytes(codec, a.hkv, P, D);
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
constexpr int ENC_THREADS = 256;
constexpr int ENC_TILES = ENC_THREADS / 64;   // tiles staged at once

// Grid (pair i, KV head, plane).
template <int D>
__global__ void __launch_bounds__(ENC_THREADS) encode_kernel(EncodeArgs a) {
  __shared__ float xs[ENC_TILES][16][D + 1];          // staged tiles, [token][dim]
  __shared__ float sc[ENC_TILES][16][D / 32];         // INT group scales (fp32 of the fp16 value)
  __shared__ float red[ENC_THREADS / 64];
  const int i = blockIdx.x, h = blockIdx.y, plane = blockIdx.z, tid = threadIdx.x;
  const int P = a.page, hkv = a.hkv;
  const int lane = tid & 63, slot = tid >> 6;

  // ---- pair checks (every thread computes the same answer)
  const int src = a.src[i], dst = a.dst[i];
  const int dcodec = plane ? (a.dst_codec >> 4) : (a.dst_codec & 15);
  bool ok = (unsigned)src < (unsigned)a.num_pages && (unsigned)dst < (unsigned)a.num_pages && src != dst;
  int scodec = 0;
  uint64_t so = 0, dof = 0;
  if (ok) {
    const int cb = a.codec[src];
    ok = w16(cb & 15) && w16(cb >> 4);
    scodec = plane ? (cb >> 4) : (cb & 15);
    so = plane ? a.voff[src] : a.koff[src];
    dof = plane ? a.voff[dst] : a.koff[dst];
    const uint64_t sb = wplane_bytes(scodec, hkv, P, D), db = wplane_bytes(dcodec, hkv, P, D);
    ok = ok && ((so | dof) & 15) == 0 && so <= a.pool_bytes && a.pool_bytes - so >= sb &&
         dof <= a.pool_bytes && a.pool_bytes - dof >= db;
    // the destination planes must not overlap either source plane
    const uint64_t sk = a.koff[src], sv = a.voff[src];
    const uint64_t skb = wplane_bytes(cb & 15, hkv, P, D), svb = wplane_bytes(cb >> 4, hkv, P, D);
    ok = ok && (dof + db <= sk || sk + skb <= dof) && (dof + db <= sv || sv + svb <= dof);
  }
  if (!ok) {
    if (h == 0 && plane == 0 && tid == 0) count_err(a.err);
    return;
  }
  const uint8_t* sp = a.pool + so + (size_t)h * P * D * 2;
  uint8_t* dp = a.pool + dof + (size_t)h * P * D * wbits(dcodec) / 8;

  // ---- FP8: the block's absmax first (one streaming pass over the head's codes)
  float s8 = 1.f;
  if (dcodec == W_FP8) {
    float m = 0.f;
    const uint32_t n16 = (uint32_t)(P * D * 2 / 16);
    for (uint32_t c = tid; c < n16; c += ENC_THREADS) {
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
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    s8 = m == 0.f ? 1.f : __fdiv_rn(m, 448.0f);
    if (tid == 0 && a.scale) a.scale[((size_t)dst * hkv + h) * 2 + plane] = s8;
  } else if (tid == 0 && a.scale) {
    a.scale[((size_t)dst * hkv + h) * 2 + plane] = 1.f;
  }
  if (h == 0 && plane == 0 && tid == 0) a.codec_out[dst] = (uint8_t)a.dst_codec;

  const bool is_v = plane == 1;
  constexpr int E = D / 4;                               // run elements per lane
  constexpr int Rs = D / 2;                              // source run bytes (16-bit)
  const int dbits = wbits(dcodec);
  const int Rd = D * dbits / 32;                         // destination run bytes
  const bool dgrouped = wint(dcodec) && !is_v;
  const int qmax = dcodec == W_INT8 ? 127 : 7;
  const int ntiles = P / 16;
  constexpr int G = D / 32;

  for (int t0 = 0; t0 < ntiles; t0 += ENC_TILES) {
    const int tile = t0 + slot;
    const bool live = tile < ntiles;
    __syncthreads();
    // stage: lane L of this slot reads its source run (16-bit layout, ungrouped K)
    if (live) {
      const uint8_t* ts = sp + (size_t)tile * 16 * D * 2;
#pragma unroll
      for (int c = 0; c < Rs / 16; ++c) {
        const u4 w = *reinterpret_cast<const u4*>(ts + run_byte(lane, 16 * c, Rs));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int e = 8 * c + k;
          int tt, d;
          run_elem(lane, e, D, is_v, false, tt, d);
          const uint16_t code = (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xFFFF));
          xs[slot][tt][d] = h16_to_f(code, scodec);
        }
      }
    }
    __syncthreads();
    // INT group scales: one (token, group) per thread of the slot
    if (live && wint(dcodec)) {
      for (int q = lane; q < 16 * G; q += 64) {
        const int tt = q / G, g = q % G;
        float m = 0.f;
        for (int j = 0; j < 32; ++j) m = fmaxf(m, __builtin_fabsf(xs[slot][tt][32 * g + j]));
        const _Float16 s16 = m == 0.f ? (_Float16)1.0f : (_Float16)__fdiv_rn(m, (float)qmax);
        sc[slot][tt][g] = (float)s16;
        const size_t so16 = (size_t)hkv * P * D * dbits / 8 + ((size_t)h * P + 16 * tile + tt) * G * 2 + 2 * g;
        *reinterpret_cast<_Float16*>(a.pool + dof + so16) = s16;
      }
    }
    __syncthreads();
    if (!live) continue;
    // destination run of lane L: E elements, Rd bytes, written 16 (or 8) bytes at a time
    uint8_t* td = dp + (size_t)tile * 16 * D * dbits / 8;
    uint32_t word[D / 8];                               // the run: up to D/2 bytes
#pragma unroll
    for (int k = 0; k < D / 8; ++k) word[k] = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      int tt, d;
      run_elem(lane, e, D, is_v, dgrouped, tt, d);
      const float x = xs[slot][tt][d];
      uint32_t code;
      if (dcodec == W_FP16) {
        code = __builtin_bit_cast(uint16_t, (_Float16)x);
      } else if (dcodec == W_BF16) {
        code = f_to_bf16(x);
      } else if (dcodec == W_FP8) {
        const float y = fminf(fmaxf(__fdiv_rn(x, s8), -448.0f), 448.0f);
        code = f_to_e4m3(y);
      } else {
        const float q = __builtin_rintf(__fdiv_rn(x, sc[slot][tt][d / 32]));
        code = (uint32_t)(int)fminf(fmaxf(q, (float)-qmax), (float)qmax);
      }
      if (dbits == 16) {
        word[e >> 1] |= (code & 0xFFFFu) << (16 * (e & 1));
      } else if (dbits == 8) {
        word[e >> 2] |= (code & 0xFFu) << (8 * (e & 3));
      } else {
        const int r = e & 7, nslot = (r & 1) * 4 + (r >> 1);
        word[e >> 3] |= (code & 0xFu) << (4 * nslot);
      }
    }
    if (Rd >= 16) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        if (16 * c < Rd)
        *reinterpret_cast<u4*>(td + run_byte(lane, 16 * c, Rd)) =
            u4{word[4 * c], word[4 * c + 1], word[4 * c + 2], word[4 * c + 3]};
    } else {   // INT4, D = 64: 8-byte runs
      *reinterpret_cast<uint2*>(td + run_byte(lane, 0, Rd)) = uint2{word[0], word[1]};
    }
  }
}

}  // namespace

int launch_append(const AppendArgs& a, void* stream) {
  if (a.rows == 0) return 0;
  hipLaunchKernelGGL(append_kernel, dim3(a.rows, a.hkv, 2), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_encode(const EncodeArgs& a, void* stream) {
  if (a.n == 0) return 0;
  const dim3 grid(a.n, a.hkv, 2);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a.head_dim == 64)
    hipLaunchKernelGGL(encode_kernel<64>, grid, dim3(ENC_THREADS), 0, s, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL(encode_kernel<128>, grid, dim3(ENC_THREADS), 0, s, a);
  else
    return -2;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
