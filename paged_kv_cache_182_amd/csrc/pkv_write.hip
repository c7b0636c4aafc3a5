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
// Codes of one destination run (lane L of a tile): D/4 elements from the
// staged tile x[token][dim], written with 16-byte (8 for INT4 at D = 64)
// stores at the run's chunk positions.
template <int D, int DC, bool IS_V>
__device__ __attribute__((always_inline)) inline void emit_run(const float (*x)[D + 1], const float (*sc)[D / 32], float s8, uint8_t* td,
                                int lane) {
  constexpr int BITS = DC <= W_BF16 ? 16 : (DC == W_INT4 ? 4 : 8);
  constexpr int E = D / 4, RD = D * BITS / 32;
  constexpr bool GROUPED = (DC == W_INT8 || DC == W_INT4) && !IS_V;
  constexpr float QMAX = DC == W_INT8 ? 127.0f : 7.0f;
  uint32_t word[RD / 4];
#pragma unroll
  for (int k = 0; k < RD / 4; ++k) word[k] = 0;
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
    } else {
      const float q = __builtin_rintf(__fdiv_rn(v, sc[tt][d / 32]));
      code = (uint32_t)(int)fminf(fmaxf(q, -QMAX), QMAX);
    }
    if constexpr (BITS == 16) {
      word[e >> 1] |= (code & 0xFFFFu) << (16 * (e & 1));
    } else if constexpr (BITS == 8) {
      word[e >> 2] |= (code & 0xFFu) << (8 * (e & 3));
    } else {
      const int r = e & 7, nslot = (r & 1) * 4 + (r >> 1);
      word[e >> 3] |= (code & 0xFu) << (4 * nslot);
    }
  }
  if constexpr (RD >= 16) {
#pragma unroll
    for (int c = 0; c < RD / 16; ++c)
      *reinterpret_cast<u4*>(td + run_byte(lane, 16 * c, RD)) =
          u4{word[4 * c], word[4 * c + 1], word[4 * c + 2], word[4 * c + 3]};
  } else {
    *reinterpret_cast<uint2*>(td + run_byte(lane, 0, RD)) = uint2{word[0], word[1]};
  }
}

template <int D, bool IS_V>
__device__ __attribute__((always_inline)) inline void emit_any(int dc, const float (*x)[D + 1], const float (*sc)[D / 32], float s8, uint8_t* td,
                                int lane) {
  switch (dc) {
    case W_FP16: emit_run<D, W_FP16, IS_V>(x, sc, s8, td, lane); break;
    case W_BF16: emit_run<D, W_BF16, IS_V>(x, sc, s8, td, lane); break;
    case W_FP8: emit_run<D, W_FP8, IS_V>(x, sc, s8, td, lane); break;
    case W_INT8: emit_run<D, W_INT8, IS_V>(x, sc, s8, td, lane); break;
    default: emit_run<D, W_INT4, IS_V>(x, sc, s8, td, lane); break;
  }
}

// Grid (pair i, KV head, plane); TILES tiles of 16 tokens staged at once, one
// 64-lane slot each (TILES = min(4, P/16), so no slot idles on small pages).
template <int D, int TILES>
__global__ void __launch_bounds__(64 * TILES) encode_kernel(EncodeArgs a) {
  constexpr int THREADS = 64 * TILES;
  __shared__ float xs[TILES][16][D + 1];              // staged tiles, [token][dim]
  __shared__ float scs[TILES][16][D / 32];            // INT group scales (fp32 of the fp16 value)
  __shared__ float red[TILES];
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
    // the destination plane must not overlap either source plane
    const uint64_t sk = a.koff[src], sv = a.voff[src];
    const uint64_t skb = wplane_bytes(cb & 15, hkv, P, D), svb = wplane_bytes(cb >> 4, hkv, P, D);
    ok = ok && (dof + db <= sk || sk + skb <= dof) && (dof + db <= sv || sv + svb <= dof);
  }
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
    // INT group scales: one (token, group) per lane of the slot
    if (live && wint(dcodec)) {
      for (int q = lane; q < 16 * G; q += 64) {
        const int tt = q / G, g = q % G;
        float m = 0.f;
#pragma unroll 8
        for (int j = 0; j < 32; ++j) m = fmaxf(m, __builtin_fabsf(xs[slot][tt][32 * g + j]));
        // fp16 scale kept inside its positive finite range [2^-24, 65504]
        _Float16 s16 = (_Float16)__fdiv_rn(m, qmax);
        s16 = s16 == (_Float16)0.0f ? __builtin_bit_cast(_Float16, (uint16_t)0x0001) : s16;
        s16 = s16 > (_Float16)65504.0f ? (_Float16)65504.0f : s16;
        s16 = m == 0.f ? (_Float16)1.0f : s16;
        scs[slot][tt][g] = (float)s16;
        const size_t so16 = (size_t)hkv * P * D * dbits / 8 + ((size_t)h * P + 16 * tile + tt) * G * 2 + 2 * g;
        *reinterpret_cast<_Float16*>(a.pool + dof + so16) = s16;
      }
    }
    __syncthreads();
    if (!live) continue;
    uint8_t* td = dp + (size_t)tile * 16 * D * dbits / 8;
    if (is_v)
      emit_any<D, true>(dcodec, xs[slot], scs[slot], s8, td, lane);
    else
      emit_any<D, false>(dcodec, xs[slot], scs[slot], s8, td, lane);
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
  const int tiles = a.page >= 64 ? 4 : a.page / 16;     // page is a multiple of 16
  if (a.head_dim == 64) {
    if (tiles >= 4) hipLaunchKernelGGL((encode_kernel<64, 4>), grid, dim3(256), 0, s, a);
    else if (tiles == 3) hipLaunchKernelGGL((encode_kernel<64, 3>), grid, dim3(192), 0, s, a);
    else if (tiles == 2) hipLaunchKernelGGL((encode_kernel<64, 2>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((encode_kernel<64, 1>), grid, dim3(64), 0, s, a);
  } else if (a.head_dim == 128) {
    if (tiles >= 4) hipLaunchKernelGGL((encode_kernel<128, 4>), grid, dim3(256), 0, s, a);
    else if (tiles == 3) hipLaunchKernelGGL((encode_kernel<128, 3>), grid, dim3(192), 0, s, a);
    else if (tiles == 2) hipLaunchKernelGGL((encode_kernel<128, 2>), grid, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((encode_kernel<128, 1>), grid, dim3(64), 0, s, a);
  } else {
    return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace pkv
