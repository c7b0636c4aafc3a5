// Internal interface between the C ABI shim (pkv_api.cpp) and the kernels
// (pkv_kernels.hip). Not installed; no part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Waves per SIMD the decode kernel for (head_dim, K codec, V codec) is built
// for. head_dim 128: four for FP8 (the tile ring fits 128 VGPRs), three for
// the other fixed pairs; head_dim 64: six for the one-scale codecs (80
// VGPRs), four for the pairs with group scales; the per-page dispatch kernel
// (codec -1, and every declared pair without a kernel of its own), which
// holds the largest tile of every codec and the code of several: three at 64,
// two at 128; its float-only variant (codec -2): four at 64, two at 128.
// Sizes the library-chosen partition count
// (workgroups resident at once = compute units x this).
// Whether a declared (K, V) codec pair has a decode kernel of its own: the
// pairs launch_decode instantiates (FP16, BF16, FP8, INT8, INT4, INT2 and
// BIT1 with themselves, INT8-K with INT4-V); every other pair runs the
// per-page kernel.
constexpr bool decode_pair_kernel(int k_codec, int v_codec) {
  return (k_codec == v_codec && k_codec >= 0 && k_codec <= 6) || (k_codec == 3 && v_codec == 4);
}
constexpr int decode_waves_per_simd(int head_dim, int k_codec, int v_codec) {
  if (k_codec == -2 && v_codec == -2) return head_dim == 64 ? 4 : 2;  // float pages only
  if (!decode_pair_kernel(k_codec, v_codec)) return head_dim == 64 ? 3 : 2;
  const bool one_scale = k_codec <= 2 && v_codec <= 2;
  // BF16 at head_dim 64 keeps its query's bf16 parts in registers: five
  // waves; INT8 with itself (95 VGPRs) five, the other group-scale pairs four
  if (head_dim == 64) return one_scale ? (k_codec == 1 ? 5 : 6) : (k_codec == 3 && v_codec == 3 ? 5 : 4);
  return (k_codec == 2 && v_codec == 2) ? 4 : 3;
}

// Pairs launch_prefill instantiates (FP16, BF16 and FP8 with themselves,
// INT8-K with INT4-V); every other pair runs the per-page kernel.
constexpr bool prefill_pair_kernel(int k_codec, int v_codec) {
  return (k_codec == v_codec && k_codec >= 0 && k_codec <= 2) || (k_codec == 3 && v_codec == 4);
}
// Waves per SIMD of the prefill kernel for (head_dim, K codec, V codec): the
// occupancy asked of the compiler (as its minimum) and the one the
// library-chosen prefill partition count is sized for. At head_dim 64 four
// for FP16 and FP8 (128 VGPRs), three for BF16 (125: its query's bf16
// parts), two for INT8/INT4 (at three it spills); at 128 two for the 16-bit
// and FP8 pairs, one for INT8/INT4; one for the per-page kernel.
constexpr int prefill_waves_per_simd(int head_dim, int k_codec, int v_codec) {
  if (!prefill_pair_kernel(k_codec, v_codec)) return 1;
  if (head_dim == 64) return k_codec == 0 || k_codec == 2 ? 4 : (k_codec == 1 ? 3 : 2);
  return k_codec <= 2 ? 2 : 1;
}

// Everything one decode launch needs, resolved on the host.
struct DecodeArgs {
  const uint16_t* q;        // fp16 [B][Hq][D]
  const uint8_t* pool;      // byte arena
  const uint64_t* koff;     // [num_pages]
  const uint64_t* voff;     // [num_pages]
  const uint8_t* codec;     // [num_pages]
  const float* scale;       // [num_pages][Hkv][2] or nullptr
  const int32_t* bt;        // [B][max_pages]
  const int32_t* seq_lens;  // [B]
  const int32_t* sel;       // [B][max_sel] or nullptr
  const int32_t* sel_lens;  // [B] or nullptr
  float* out;               // [B][Hq][D]
  float* lse;               // [B][Hq]
  float* part_acc;          // [B*Hq][nparts][D]   (nparts > 1)
  float* part_ml;           // [B*Hq][nparts][2]   (nparts > 1)
  int32_t* err;             // device counter or nullptr
  int32_t rows, hq, hkv, group, page, num_pages, max_pages, max_sel;
  int32_t tiles_per_part;   // 16-token tiles per partition; 0: each row's tiles split evenly into nparts
  int32_t tile_shift;       // log2(page / 16) when that is a power of two, else -1
  int32_t nparts;
  int32_t sparse;
  int32_t final_out;        // 1: write out/lse (single partition); 0: write partials
  int32_t window;           // sliding window in tokens (each row attends positions >= L - window); 0: none
  float scale_log2;         // softmax_scale * log2(e)
  uint64_t pool_bytes;      // size of the arena; planes must lie inside it
};

// One token per row into its 16-bit page (pkv_append_kv).
struct AppendArgs {
  const uint16_t* k_new;    // fp16 [rows][Hkv][D]
  const uint16_t* v_new;
  uint8_t* pool;
  const uint64_t* koff;
  const uint64_t* voff;
  const uint8_t* codec;
  const int32_t* bt;        // [rows][max_pages]
  const int32_t* seq_lens;  // [rows], lengths before the append
  int32_t* err;
  int32_t rows, hkv, head_dim, page, num_pages, max_pages;
  uint64_t pool_bytes;
};

// Re-encode n 16-bit pages (pkv_encode_pages).
struct EncodeArgs {
  const int32_t* src;       // [n] physical page ids read
  const int32_t* dst;       // [n] physical page ids written
  uint8_t* pool;
  const uint64_t* koff;
  const uint64_t* voff;
  const uint8_t* codec;     // read: source codecs
  uint8_t* codec_out;       // written: page_codec[dst] = dst_codec
  float* scale;             // [num_pages][Hkv][2] or nullptr
  int32_t* err;
  int32_t n, dst_codec, hkv, head_dim, page, num_pages;
  uint64_t pool_bytes;
};

// Chunked-prefill attention (pkv_prefill_attention).
struct PrefillArgs {
  const uint16_t* q;        // fp16 [B][T][Hq][D]
  const uint8_t* pool;
  const uint64_t* koff;
  const uint64_t* voff;
  const uint8_t* codec;
  const float* scale;       // [num_pages][Hkv][2] or nullptr
  const int32_t* bt;        // [B][max_pages]
  const int32_t* seq_lens;  // [B]
  float* out;               // [B][T][Hq][D]   (final_out)
  float* lse;               // [B][T][Hq]      (final_out)
  float* part_acc;          // [B*T*Hq][nparts][D]
  float* part_ml;           // [B*T*Hq][nparts][2]
  int32_t* err;
  int32_t rows, tokens, hq, hkv, group, page, num_pages, max_pages;
  int32_t kv_begin;         // first key position attended (>= 0)
  int32_t kv_end;           // one past the last key position (already capped at max_pages * page)
  int32_t window;           // sliding window: a query sees its last `window` positions (<= 0: no window)
  int32_t part_base;        // kv_begin rounded down to a page boundary: partitions start here
  int32_t part_tokens;      // a multiple of page
  int32_t nparts, col_groups, final_out;
  int32_t k_codec, v_codec; // declared codecs, -1 for any
  float scale_log2;
  uint64_t pool_bytes;
};

int launch_prefill(const PrefillArgs& a, int head_dim, void* stream);
// acc <- log-sum-exp fold of (acc, (out, lse)), rows of head_dim values.
int launch_fold_into(int rows, int head_dim, float* acc_out, float* acc_lse, const float* out,
                     const float* lse, void* stream);

// Block top-k page selection (pkv_select_pages).
struct SelectArgs {
  const uint16_t* q_idx;    // fp16 [B][idx_dim]
  const uint16_t* slab;     // fp16 [B][max_blocks][idx_dim]
  const int32_t* seq_lens;  // [B]
  float* scores;            // [B][max_blocks] (written for the row's blocks)
  int32_t* sel;             // [B][max_sel]
  int32_t* sel_lens;        // [B]
  int32_t* dropped;         // device counter or nullptr
  int32_t* err;             // device counter or nullptr
  int32_t rows, page, max_pages, max_sel;
  int32_t block_tokens, block_topk, sink_pages, recent_pages, idx_dim, max_blocks;
  int32_t cus;  // compute units of the device (sizes the score grid)
};

int launch_select(const SelectArgs& a, void* stream);

int launch_append(const AppendArgs& a, void* stream);
int launch_encode(const EncodeArgs& a, void* stream);

// Launches the decode kernel for (head_dim, k codec, v codec); codec -1 means
// per-page dispatch. Returns 0 on success, -2 if no kernel exists for the
// combination, -4 if the launch failed.
int launch_decode(const DecodeArgs& a, int head_dim, int k_codec, int v_codec, void* stream);

// Size of the built-in scratch of pkv_decode_attention_noalloc (bytes).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;

// Device address of the current device's built-in scratch (looked up once per
// device, then cached). Returns 0, or -4 if the device or the symbol cannot
// be queried.
int noalloc_scratch(void** ptr);

// Launches the log-sum-exp fold over `rows` rows of `nparts` partials.
int launch_combine(int rows, int nparts, int head_dim, const float* part_acc,
                   const float* part_ml, float* out, float* lse, void* stream);

}  // namespace pkv
