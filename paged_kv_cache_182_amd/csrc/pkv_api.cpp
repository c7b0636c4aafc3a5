// C ABI of libpkv: argument validation, partition sizing and launches.
// The declarations and their documentation are in include/pkv.h.

#include "../../include/pkv.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "pkv_internal.h"

namespace {

constexpr int kMinPartitionTokens = 256;
constexpr int kMinTilesPerPartition = 8; // decode: two 16-token tiles per wave of a workgroup

// Compute units of the current HIP device, read once per device and cached
// (the only state the library keeps). Where no device can be queried (a
// host without a GPU sizing partitions) the count of gfx950 parts, 256
// (MI350X / MI355X: 8 XCDs x 32), is used.
constexpr int kDefaultComputeUnits = 256;
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return kDefaultComputeUnits;
  }
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return kDefaultComputeUnits;
  }
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_codec(int32_t c) {
  return c == PKV_CODEC_MIXED || c == PKV_CODEC_MIXED_FLOAT || (c >= PKV_FP16 && c <= PKV_BIT1_G32);
}

// Whether one plane of a page (largest at 16 bits per code) stays below 4 GiB:
// the kernels address a plane with 32-bit offsets.
bool plane_fits32(const pkv_params* p) {
  const uint64_t d = p->head_dim > 0 ? (uint64_t)p->head_dim : 0u;
  return (uint64_t)p->num_kv_heads * (uint64_t)p->page_size * d * 2u < (1ull << 32);
}

// Checks the plain-value part of the params. Returns PKV_OK or an error.
int check_params(const pkv_params* p) {
  if (!p) return PKV_ERR_INVALID_ARG;
  if (p->num_rows < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (p->page_size <= 0 || p->page_size % 16 != 0) return PKV_ERR_INVALID_ARG;
  if (p->num_pages < 0 || p->max_pages_per_row < 1 || p->max_sel_pages < 0) return PKV_ERR_INVALID_ARG;
  if (p->partition_tokens < 0 || p->partition_tokens % 16 != 0) return PKV_ERR_INVALID_ARG;
  if (!isfinite(p->softmax_scale)) return PKV_ERR_INVALID_ARG;
  if (p->window_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (p->page_size > (1 << 20)) return PKV_ERR_UNSUPPORTED;  // in-page slot counts are 24-bit on the device
  if (!plane_fits32(p)) return PKV_ERR_UNSUPPORTED;
  if (!valid_codec(p->k_codec) || !valid_codec(p->v_codec)) return PKV_ERR_INVALID_ARG;
  if ((p->k_codec == PKV_CODEC_MIXED_FLOAT) != (p->v_codec == PKV_CODEC_MIXED_FLOAT)) return PKV_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (p->num_q_heads / p->num_kv_heads > 16) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Pages (dense) or selection entries (sparse) a row can reach at most.
int64_t row_capacity(const pkv_params* p) {
  return p->max_sel_pages > 0 ? p->max_sel_pages : p->max_pages_per_row;
}

// 16-token tiles a row can reach at most: with a sliding window of W tokens
// (dense mode), the tiles that hold its W positions.
int64_t row_tiles(const pkv_params* p) {
  int64_t t = row_capacity(p) * (p->page_size / 16);
  if (p->window_tokens > 0 && p->max_sel_pages == 0) {
    const int64_t w = ((int64_t)p->window_tokens + 15) / 16 + 1;
    if (w < t) t = w;
  }
  return t;
}

// Partitions per row. A positive partition_tokens fixes their length; 0 lets
// the library split each row's tiles evenly into as many partitions as fill
// one round of resident decode workgroups (compute units x waves per SIMD;
// four waves per workgroup), with at least two tiles per wave in a partition
// (one per wave measured slower for one-row launches: more partials to fold).
int64_t partitions(const pkv_params* p) {
  const int64_t tiles = row_tiles(p);
  if (p->partition_tokens > 0) {
    const int64_t tpart = p->partition_tokens / 16;
    return (tiles + tpart - 1) / tpart;
  }
  const int64_t units = (int64_t)(p->num_rows > 0 ? p->num_rows : 1) * p->num_kv_heads;
  const int64_t resident =
      (int64_t)compute_units() * pkv::decode_waves_per_simd(p->head_dim, p->k_codec, p->v_codec);
  int64_t parts = resident / units;
  const int64_t most = (tiles + kMinTilesPerPartition - 1) / kMinTilesPerPartition;
  if (parts > most) parts = most;
  return parts < 1 ? 1 : parts;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch failed";
    case PKV_ERR_SCRATCH: return "request exceeds the built-in scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

int pkv_num_partitions(const pkv_params* p) {
  const int st = check_params(p);
  if (st != PKV_OK) return st;
  const int64_t n = partitions(p);
  return n > 0x7fffffff ? PKV_ERR_UNSUPPORTED : (int)n;
}

size_t pkv_workspace_bytes(const pkv_params* p) {
  if (check_params(p) != PKV_OK) return 0;
  const int64_t n = partitions(p);
  if (n <= 1) return 0;
  return (size_t)p->num_rows * p->num_q_heads * n * (p->head_dim + 2) * sizeof(float);
}

namespace {

// Validates the pointers and fills the launch description (not the outputs).
int prepare(const pkv_params* p, const void* q, const uint8_t* page_pool,
            const uint64_t* page_k_off, const uint64_t* page_v_off, const uint8_t* page_codec,
            const float* page_scale, const int32_t* block_table, const int32_t* seq_lens,
            const int32_t* page_sel, const int32_t* sel_lens, int32_t* err_count,
            pkv::DecodeArgs* a) {
  if (!q || !page_pool || !page_k_off || !page_v_off || !page_codec || !block_table || !seq_lens)
    return PKV_ERR_INVALID_ARG;
  const bool sparse = p->max_sel_pages > 0;
  if (sparse != (page_sel != nullptr) || sparse != (sel_lens != nullptr)) return PKV_ERR_INVALID_ARG;
  if ((p->k_codec == PKV_FP8_E4M3 || p->v_codec == PKV_FP8_E4M3) && !page_scale)
    return PKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(page_pool, 256) || !aligned(page_k_off, 8) ||
      !aligned(page_v_off, 8) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      (page_scale && !aligned(page_scale, 4)) || (page_sel && !aligned(page_sel, 4)) ||
      (sel_lens && !aligned(sel_lens, 4)) || (err_count && !aligned(err_count, 4)))
    return PKV_ERR_INVALID_ARG;
  const int64_t nparts = partitions(p);
  if (nparts > 65535 || (int64_t)p->num_rows > 65535 || p->num_kv_heads > 65535)
    return PKV_ERR_UNSUPPORTED;  // grid dimension limits
  if (row_capacity(p) * p->page_size > 0x7fffffff) return PKV_ERR_UNSUPPORTED;  // token positions are int32

  a->q = static_cast<const uint16_t*>(q);
  a->pool = page_pool;
  a->koff = page_k_off;
  a->voff = page_v_off;
  a->codec = page_codec;
  a->scale = page_scale;
  a->bt = block_table;
  a->seq_lens = seq_lens;
  a->sel = page_sel;
  a->sel_lens = sel_lens;
  a->out = nullptr;
  a->lse = nullptr;
  a->part_acc = nullptr;
  a->part_ml = nullptr;
  a->err = err_count;
  a->rows = p->num_rows;
  a->hq = p->num_q_heads;
  a->hkv = p->num_kv_heads;
  a->group = p->num_q_heads / p->num_kv_heads;
  a->page = p->page_size;
  a->num_pages = p->num_pages;
  a->max_pages = p->max_pages_per_row;
  a->max_sel = p->max_sel_pages;
  a->tiles_per_part = p->partition_tokens / 16;  // 0: even split of each row
  const int tpp = p->page_size / 16;
  a->tile_shift = (tpp & (tpp - 1)) == 0 ? __builtin_ctz((unsigned)tpp) : -1;
  a->nparts = (int32_t)nparts;
  a->sparse = sparse ? 1 : 0;
  a->final_out = 0;
  a->window = p->window_tokens;
  a->scale_log2 = p->softmax_scale * 1.44269504088896340736f;
  a->pool_bytes = p->pool_bytes;
  return PKV_OK;
}

int launch_status(int st) { return st == 0 ? PKV_OK : (st == -2 ? PKV_ERR_UNSUPPORTED : PKV_ERR_HIP); }

}  // namespace

int pkv_decode_attention(const pkv_params* p, const void* q, const uint8_t* page_pool,
                         const uint64_t* page_k_off, const uint64_t* page_v_off,
                         const uint8_t* page_codec, const float* page_scale,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* page_sel, const int32_t* sel_lens, float* out,
                         float* lse, void* workspace, size_t workspace_bytes,
                         int32_t* err_count, void* stream) {
  int st = check_params(p);
  if (st != PKV_OK) return st;
  if (p->num_rows == 0) return PKV_OK;
  if (!out || !lse || !aligned(out, 4) || !aligned(lse, 4)) return PKV_ERR_INVALID_ARG;
  pkv::DecodeArgs a;
  st = prepare(p, q, page_pool, page_k_off, page_v_off, page_codec, page_scale, block_table,
               seq_lens, page_sel, sel_lens, err_count, &a);
  if (st != PKV_OK) return st;
  if (a.nparts > 1) {
    const size_t need = pkv_workspace_bytes(p);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return PKV_ERR_WORKSPACE;
    a.part_acc = static_cast<float*>(workspace);
    a.part_ml = a.part_acc + (size_t)p->num_rows * p->num_q_heads * a.nparts * p->head_dim;
  } else {
    a.out = out;
    a.lse = lse;
    a.final_out = 1;
  }
  st = launch_status(pkv::launch_decode(a, p->head_dim, p->k_codec, p->v_codec, stream));
  if (st != PKV_OK || a.nparts == 1) return st;
  return launch_status(pkv::launch_combine(p->num_rows * p->num_q_heads, a.nparts, p->head_dim,
                                           a.part_acc, a.part_ml, out, lse, stream));
}

int pkv_decode_attention_noalloc(const pkv_params* p, const void* q, const uint8_t* page_pool,
                                 const uint64_t* page_k_off, const uint64_t* page_v_off,
                                 const uint8_t* page_codec, const float* page_scale,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* page_sel, const int32_t* sel_lens, float* out,
                                 float* lse, int32_t* err_count, void* stream) {
  int st = check_params(p);
  if (st != PKV_OK) return st;
  if (p->num_rows == 0) return PKV_OK;
  // the partials this call needs must fit the built-in scratch (checked
  // before anything else touches the device)
  if (pkv_workspace_bytes(p) > pkv::kNoAllocScratchBytes) return PKV_ERR_SCRATCH;
  if (!out || !lse || !aligned(out, 4) || !aligned(lse, 4)) return PKV_ERR_INVALID_ARG;
  pkv::DecodeArgs a;
  st = prepare(p, q, page_pool, page_k_off, page_v_off, page_codec, page_scale, block_table,
               seq_lens, page_sel, sel_lens, err_count, &a);
  if (st != PKV_OK) return st;
  if (a.nparts > 1) {
    void* ws = nullptr;
    if (pkv::noalloc_scratch(&ws) != 0) return PKV_ERR_HIP;
    a.part_acc = static_cast<float*>(ws);
    a.part_ml = a.part_acc + (size_t)p->num_rows * p->num_q_heads * a.nparts * p->head_dim;
  } else {
    a.out = out;
    a.lse = lse;
    a.final_out = 1;
  }
  st = launch_status(pkv::launch_decode(a, p->head_dim, p->k_codec, p->v_codec, stream));
  if (st != PKV_OK || a.nparts == 1) return st;
  return launch_status(pkv::launch_combine(p->num_rows * p->num_q_heads, a.nparts, p->head_dim,
                                           a.part_acc, a.part_ml, out, lse, stream));
}

size_t pkv_noalloc_scratch_bytes(void) { return pkv::kNoAllocScratchBytes; }

int pkv_decode_partials(const pkv_params* p, const void* q, const uint8_t* page_pool,
                        const uint64_t* page_k_off, const uint64_t* page_v_off,
                        const uint8_t* page_codec, const float* page_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* page_sel, const int32_t* sel_lens, float* part_acc,
                        float* part_ml, int32_t* err_count, void* stream) {
  int st = check_params(p);
  if (st != PKV_OK) return st;
  if (p->num_rows == 0) return PKV_OK;
  if (!part_acc || !part_ml || !aligned(part_acc, 16) || !aligned(part_ml, 16))
    return PKV_ERR_INVALID_ARG;
  pkv::DecodeArgs a;
  st = prepare(p, q, page_pool, page_k_off, page_v_off, page_codec, page_scale, block_table,
               seq_lens, page_sel, sel_lens, err_count, &a);
  if (st != PKV_OK) return st;
  a.part_acc = part_acc;
  a.part_ml = part_ml;
  return launch_status(pkv::launch_decode(a, p->head_dim, p->k_codec, p->v_codec, stream));
}

int pkv_lse_combine(int32_t rows, int32_t num_parts, int32_t head_dim, const float* part_acc,
                    const float* part_ml, float* out, float* lse, void* stream) {
  if (rows < 0 || num_parts < 1 || head_dim < 1 || head_dim > 512) return PKV_ERR_INVALID_ARG;
  if (rows == 0) return PKV_OK;
  if (!part_acc || !part_ml || !out || !lse) return PKV_ERR_INVALID_ARG;
  if (!aligned(part_acc, 4) || !aligned(part_ml, 4) || !aligned(out, 4) || !aligned(lse, 4))
    return PKV_ERR_INVALID_ARG;
  if (rows > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  return pkv::launch_combine(rows, num_parts, head_dim, part_acc, part_ml, out, lse, stream) == 0
             ? PKV_OK
             : PKV_ERR_HIP;
}

}  // extern "C"

// ------------------------------------------------------------ write side
namespace {

// Plain-value checks shared by the write-side calls (q heads and codecs of
// the read path are not used).
int check_write_params(const pkv_params* p) {
  if (!p) return PKV_ERR_INVALID_ARG;
  if (p->num_rows < 0 || p->num_kv_heads <= 0 || p->num_pages < 0) return PKV_ERR_INVALID_ARG;
  if (p->page_size <= 0 || p->page_size % 16 != 0 || p->max_pages_per_row < 1) return PKV_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (p->num_rows > 65535 || p->num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  if (p->page_size > (1 << 20) || !plane_fits32(p)) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_append_kv(const pkv_params* p, const void* k_new, const void* v_new, uint8_t* page_pool,
                  const uint64_t* page_k_off, const uint64_t* page_v_off, const uint8_t* page_codec,
                  const int32_t* block_table, const int32_t* seq_lens, int32_t* err_count, void* stream) {
  const int st = check_write_params(p);
  if (st != PKV_OK) return st;
  if (p->num_rows == 0) return PKV_OK;
  if (!k_new || !v_new || !page_pool || !page_k_off || !page_v_off || !page_codec || !block_table || !seq_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(page_pool, 256) || !aligned(page_k_off, 8) ||
      !aligned(page_v_off, 8) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      (err_count && !aligned(err_count, 4)))
    return PKV_ERR_INVALID_ARG;
  pkv::AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.pool = page_pool;
  a.koff = page_k_off;
  a.voff = page_v_off;
  a.codec = page_codec;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.err = err_count;
  a.rows = p->num_rows;
  a.hkv = p->num_kv_heads;
  a.head_dim = p->head_dim;
  a.page = p->page_size;
  a.num_pages = p->num_pages;
  a.max_pages = p->max_pages_per_row;
  a.pool_bytes = p->pool_bytes;
  return pkv::launch_append(a, stream) == 0 ? PKV_OK : PKV_ERR_HIP;
}

int pkv_encode_pages(const pkv_params* p, int32_t n, const int32_t* src_pages, const int32_t* dst_pages,
                     int32_t dst_codec, uint8_t* page_pool, const uint64_t* page_k_off,
                     const uint64_t* page_v_off, uint8_t* page_codec, float* page_scale, int32_t* err_count,
                     void* stream) {
  const int st = check_write_params(p);
  if (st != PKV_OK) return st;
  const int kc = dst_codec & 15, vc = (dst_codec >> 4) & 15;
  if (n < 0 || dst_codec < 0 || dst_codec > 0xFF || kc > PKV_BIT1_G32 || vc > PKV_BIT1_G32)
    return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (n > 0x7fffffff / 2) return PKV_ERR_UNSUPPORTED;
  if (!src_pages || !dst_pages || !page_pool || !page_k_off || !page_v_off || !page_codec)
    return PKV_ERR_INVALID_ARG;
  if ((kc == PKV_FP8_E4M3 || vc == PKV_FP8_E4M3) && !page_scale) return PKV_ERR_INVALID_ARG;
  if (!aligned(src_pages, 4) || !aligned(dst_pages, 4) || !aligned(page_pool, 256) ||
      !aligned(page_k_off, 8) || !aligned(page_v_off, 8) || (page_scale && !aligned(page_scale, 4)) ||
      (err_count && !aligned(err_count, 4)))
    return PKV_ERR_INVALID_ARG;
  pkv::EncodeArgs a{};
  a.src = src_pages;
  a.dst = dst_pages;
  a.pool = page_pool;
  a.koff = page_k_off;
  a.voff = page_v_off;
  a.codec = page_codec;
  a.codec_out = page_codec;
  a.scale = page_scale;
  a.err = err_count;
  a.n = n;
  a.dst_codec = dst_codec;
  a.hkv = p->num_kv_heads;
  a.head_dim = p->head_dim;
  a.page = p->page_size;
  a.num_pages = p->num_pages;
  a.pool_bytes = p->pool_bytes;
  const int r = pkv::launch_encode(a, stream);
  return r == 0 ? PKV_OK : (r == -2 ? PKV_ERR_UNSUPPORTED : PKV_ERR_HIP);
}

}  // extern "C"

// ------------------------------------------------------------ chunked prefill
namespace {

constexpr int kPrefillCols = 128;  // query columns (token, head-of-group pairs) per workgroup

struct PrefillPlan {
  int64_t base, end;        // partitions cover [base, end): base = kv_begin rounded down to a page
  int64_t part_tokens;
  int64_t nparts;
  int64_t col_groups;
};

// Validates the prefill-specific values and sizes the partitions.
int plan_prefill(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end, PrefillPlan* pl) {
  int st = check_params(p);
  if (st != PKV_OK) return st;
  if (p->max_sel_pages != 0) return PKV_ERR_INVALID_ARG;  // the prefill attends the dense cache
  if (p->window_tokens != 0) return PKV_ERR_INVALID_ARG;  // its sliding window is an argument of its own
  if (p->partition_tokens % p->page_size != 0) return PKV_ERR_INVALID_ARG;  // prefill partitions are whole pages
  if (q_tokens < 0 || kv_begin < 0 || (kv_end >= 0 && kv_end < kv_begin)) return PKV_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)p->max_pages_per_row * p->page_size;
  pl->base = (int64_t)kv_begin / p->page_size * p->page_size;
  pl->end = kv_end < 0 ? cap : (kv_end < cap ? kv_end : cap);
  const int64_t span = pl->end > pl->base ? pl->end - pl->base : 0;
  const int64_t cols = (int64_t)q_tokens * (p->num_q_heads / p->num_kv_heads);
  pl->col_groups = cols > 0 ? (cols + kPrefillCols - 1) / kPrefillCols : 1;
  if (p->partition_tokens > 0) {
    pl->part_tokens = p->partition_tokens;
  } else {
    // as many partitions as fill one round of resident workgroups (a partial
    // last round leaves most of the chip idle while it runs)
    const int64_t units = (int64_t)(p->num_rows > 0 ? p->num_rows : 1) * p->num_kv_heads * pl->col_groups;
    const int64_t resident =
        (int64_t)compute_units() * pkv::prefill_waves_per_simd(p->head_dim, p->k_codec, p->v_codec);
    int64_t parts = resident / units;
    if (parts < 1) parts = 1;
    int64_t pt = (span + parts - 1) / parts;
    if (pt < kMinPartitionTokens) pt = kMinPartitionTokens;
    pt = (pt + p->page_size - 1) / p->page_size * p->page_size;
    pl->part_tokens = pt;
  }
  pl->nparts = span > 0 ? (span + pl->part_tokens - 1) / pl->part_tokens : 1;
  if (pl->nparts < 1) pl->nparts = 1;
  if (pl->end > 0x7fffffff) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_prefill_num_partitions(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end) {
  PrefillPlan pl;
  const int st = plan_prefill(p, q_tokens, kv_begin, kv_end, &pl);
  if (st != PKV_OK) return st;
  return pl.nparts > 0x7fffffff ? PKV_ERR_UNSUPPORTED : (int)pl.nparts;
}

size_t pkv_prefill_workspace_bytes(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end) {
  PrefillPlan pl;
  if (plan_prefill(p, q_tokens, kv_begin, kv_end, &pl) != PKV_OK || pl.nparts <= 1) return 0;
  return (size_t)p->num_rows * q_tokens * p->num_q_heads * pl.nparts * (p->head_dim + 2) * sizeof(float);
}

int pkv_prefill_attention(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end,
                          int32_t window_tokens, const void* q, const uint8_t* page_pool, const uint64_t* page_k_off,
                          const uint64_t* page_v_off, const uint8_t* page_codec, const float* page_scale,
                          const int32_t* block_table, const int32_t* seq_lens, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, int32_t* err_count, void* stream) {
  PrefillPlan pl;
  int st = plan_prefill(p, q_tokens, kv_begin, kv_end, &pl);
  if (st != PKV_OK) return st;
  if (p->num_rows == 0 || q_tokens == 0) return PKV_OK;
  if (!q || !page_pool || !page_k_off || !page_v_off || !page_codec || !block_table || !seq_lens || !out || !lse)
    return PKV_ERR_INVALID_ARG;
  if ((p->k_codec == PKV_FP8_E4M3 || p->v_codec == PKV_FP8_E4M3) && !page_scale) return PKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(page_pool, 256) || !aligned(page_k_off, 8) || !aligned(page_v_off, 8) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(out, 4) || !aligned(lse, 4) ||
      (page_scale && !aligned(page_scale, 4)) || (err_count && !aligned(err_count, 4)))
    return PKV_ERR_INVALID_ARG;
  const int64_t gx = (pl.nparts + 7) / 8 * 8 * pl.col_groups;
  if (gx > 0x7fffffff || p->num_rows > 65535 || p->num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)p->num_rows * q_tokens * p->num_q_heads;
  if (rows > 0x7fffffff) return PKV_ERR_UNSUPPORTED;

  pkv::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.pool = page_pool;
  a.koff = page_k_off;
  a.voff = page_v_off;
  a.codec = page_codec;
  a.scale = page_scale;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.err = err_count;
  a.rows = p->num_rows;
  a.tokens = q_tokens;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.page = p->page_size;
  a.num_pages = p->num_pages;
  a.max_pages = p->max_pages_per_row;
  a.kv_begin = kv_begin;
  a.kv_end = (int32_t)pl.end;
  a.window = window_tokens > 0 ? window_tokens : 0;
  a.part_base = (int32_t)pl.base;
  a.part_tokens = (int32_t)pl.part_tokens;
  a.nparts = (int32_t)pl.nparts;
  a.col_groups = (int32_t)pl.col_groups;
  a.k_codec = p->k_codec;
  a.v_codec = p->v_codec;
  a.scale_log2 = p->softmax_scale * 1.44269504088896340736f;
  a.pool_bytes = p->pool_bytes;
  if (pl.nparts > 1) {
    const size_t need = pkv_prefill_workspace_bytes(p, q_tokens, kv_begin, kv_end);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return PKV_ERR_WORKSPACE;
    a.part_acc = static_cast<float*>(workspace);
    a.part_ml = a.part_acc + (size_t)rows * pl.nparts * p->head_dim;
    a.final_out = 0;
  } else {
    a.out = out;
    a.lse = lse;
    a.final_out = 1;
  }
  st = launch_status(pkv::launch_prefill(a, p->head_dim, stream));
  if (st != PKV_OK || pl.nparts == 1) return st;
  return launch_status(
      pkv::launch_combine((int)rows, a.nparts, p->head_dim, a.part_acc, a.part_ml, out, lse, stream));
}

int pkv_lse_fold_into(int32_t rows, int32_t head_dim, float* acc_out, float* acc_lse, const float* out,
                      const float* lse, void* stream) {
  if (rows < 0 || head_dim < 1 || head_dim > 512) return PKV_ERR_INVALID_ARG;
  if (rows == 0) return PKV_OK;
  if (!acc_out || !acc_lse || !out || !lse) return PKV_ERR_INVALID_ARG;
  if (!aligned(acc_out, 4) || !aligned(acc_lse, 4) || !aligned(out, 4) || !aligned(lse, 4))
    return PKV_ERR_INVALID_ARG;
  return pkv::launch_fold_into(rows, head_dim, acc_out, acc_lse, out, lse, stream) == 0 ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"

// ------------------------------------------------------------ page selection
namespace {

constexpr int32_t kSelectMaxPages = 262144;  // one LDS bit per page of a row

int64_t gcd64(int64_t x, int64_t y) {
  while (y) {
    const int64_t t = x % y;
    x = y;
    y = t;
  }
  return x;
}

}  // namespace

extern "C" {

int pkv_select_capacity(int32_t page_size, int32_t block_tokens, int32_t block_topk, int32_t sink_pages,
                        int32_t recent_pages) {
  if (page_size <= 0 || block_tokens <= 0 || block_topk < 0 || sink_pages < 0 || recent_pages < 0)
    return PKV_ERR_INVALID_ARG;
  const int64_t g = gcd64(block_tokens, page_size);
  const int64_t per_block = (page_size - g + block_tokens - 1) / page_size + 1;
  const int64_t cap = per_block * block_topk + sink_pages + recent_pages;
  return cap > 0x7fffffff ? PKV_ERR_UNSUPPORTED : (int)cap;
}

int pkv_select_pages(const pkv_params* p, int32_t block_tokens, int32_t block_topk, int32_t sink_pages,
                     int32_t recent_pages, int32_t idx_dim, int32_t max_blocks, const void* q_idx, const void* slab,
                     const int32_t* seq_lens, float* block_scores, int32_t* page_sel, int32_t* sel_lens,
                     int32_t* dropped, int32_t* err_count, void* stream) {
  if (!p || p->num_rows < 0 || p->page_size <= 0 || p->page_size % 16 != 0 || p->max_pages_per_row < 1 ||
      p->max_sel_pages < 1)
    return PKV_ERR_INVALID_ARG;
  if (block_tokens <= 0 || block_topk < 0 || sink_pages < 0 || recent_pages < 0 || idx_dim <= 0 ||
      idx_dim % 8 != 0 || max_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (idx_dim > 4096 || p->max_pages_per_row > kSelectMaxPages || p->num_rows > 65535) return PKV_ERR_UNSUPPORTED;
  // a row of the slab is read through one 32-bit buffer range (with a chunk of 64 blocks to spare)
  if (((int64_t)max_blocks + 64) * idx_dim * 2 > (int64_t(1) << 32) - (int64_t(1) << 16)) return PKV_ERR_UNSUPPORTED;
  if (p->num_rows == 0) return PKV_OK;
  if (!q_idx || !seq_lens || !page_sel || !sel_lens || (max_blocks > 0 && (!slab || !block_scores)))
    return PKV_ERR_INVALID_ARG;
  if (!aligned(q_idx, 2) || !aligned(seq_lens, 4) || !aligned(page_sel, 4) || !aligned(sel_lens, 4) ||
      (slab && !aligned(slab, 16)) || (block_scores && !aligned(block_scores, 4)) ||
      (dropped && !aligned(dropped, 4)) || (err_count && !aligned(err_count, 4)))
    return PKV_ERR_INVALID_ARG;
  pkv::SelectArgs a{};
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.slab = static_cast<const uint16_t*>(slab);
  a.seq_lens = seq_lens;
  a.scores = block_scores;
  a.sel = page_sel;
  a.sel_lens = sel_lens;
  a.dropped = dropped;
  a.err = err_count;
  a.rows = p->num_rows;
  a.page = p->page_size;
  a.max_pages = p->max_pages_per_row;
  a.max_sel = p->max_sel_pages;
  a.block_tokens = block_tokens;
  a.block_topk = block_topk;
  a.sink_pages = sink_pages;
  a.recent_pages = recent_pages;
  a.idx_dim = idx_dim;
  a.max_blocks = max_blocks;
  a.cus = compute_units();
  return pkv::launch_select(a, stream) == 0 ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
