/*
 * pkv.h -- C ABI of libpkv: single-query (decode) attention read straight
 * from a paged KV cache whose pages use mixed codecs, on AMD MI355X (gfx950).
 *
 * What is computed. For every row b (an independent query: a sequence, or a
 * (layer, sequence) pair) and query head hq, with KV head h = hq / G where
 * G = num_q_heads / num_kv_heads (grouped-query attention; ARGUS page "Why
 * decode is slow"):
 *
 *     s_t  = softmax_scale * sum_i q[b][hq][i] * K_t[h][i]
 *     out  = sum_t exp(s_t - m) V_t[h] / sum_t exp(s_t - m),  m = max_t s_t
 *     lse  = m + ln(sum_t exp(s_t - m))                         (natural log)
 *
 * over the attended tokens t: in dense mode tokens 0 .. seq_lens[b]-1, found
 * through the row's block table (logical page -> physical page; FreeToken PR
 * #499 "Design"); in sparse mode only the tokens t < seq_lens[b] of the
 * logical pages listed in page_sel (PR #499 "What" and "Why this works");
 * with a sliding window of W tokens, only those at positions >= L_b - W.
 * The kernel walks the pages with an exact online softmax (ARGUS "Direct
 * paged attention"); long rows are split into partitions of
 * partition_tokens whose (acc, max, sum) partials are folded by log-sum-exp
 * into the output (PR #499 discussion, in-place host K/V design). An empty
 * token set gives out = 0 and lse = -inf.
 *
 * Codecs (per physical page, separately for K and V; ARGUS page intro and
 * "v0.5": FP16/BF16 and Q8/Q4 group pages; PR #499 update: FP8 e4m3 codes +
 * fp32 scales):
 *   PKV_FP16      IEEE binary16.
 *   PKV_BF16      bfloat16. Decode and the chunked prefill feed the codes
 *                 to the bf16 matrix instructions as they are, against the
 *                 query and the softmax weights split into bf16 high and low
 *                 parts: bf16's whole range is exact.
 *   PKV_FP8_E4M3  OCP E4M3FN codes times page_scale[page][h][K|V] (fp32).
 *   PKV_INT8_G32  int8 codes times one fp16 scale per (token, 32 dims).
 *   PKV_INT4_G32  int4 codes times one fp16 scale per (token, 32 dims).
 *   PKV_INT2_G32  the INT2 tier of ARGUS's cascade (page intro), as the
 *                 unsigned-affine 2-bit kind of its "Pluggable tiers": codes
 *                 u in 0..3 denoting z + s*u, with an fp16 offset z and an
 *                 fp16 step s per (token, 32 dims).
 *   PKV_BIT1_G32  the 1-bit tier: sign codes (bit 1 = negative) times one
 *                 fp16 scale per (token, 32 dims).
 *
 * In-page layout (this library's definition). page_k_off[p] / page_v_off[p]
 * are byte offsets from page_pool to the K and V planes of physical page p;
 * both must be multiples of 16. A plane holds the codes of every KV head,
 * head after head (page_size * head_dim codes each), then, for the group-scale
 * codecs (INT8, INT4, INT2, BIT1), fp16 scales[Hkv][page_size][head_dim/32],
 * and for INT2 then fp16 offsets[Hkv][page_size][head_dim/32]. One head's
 * codes are page_size/16 tiles of 16 tokens, tile after tile; a tile
 * (16*D*bits/8 bytes) is the register image of the 64 lanes of the wave that
 * consumes it. Lane L (0..63) owns a run of D/4 consecutive elements,
 * R = D*bits/32 bytes: with R >= 16 the runs are interleaved in 16-byte chunks
 * (chunk c of lane L at byte c*1024 + 16*L of the tile), else run L sits at
 * byte R*L. Element e of lane L's run holds, with tt the token within the
 * tile:
 *   K, FP16/BF16/FP8:  tt = L%16, dim = (D/4)*(L/16) + e;
 *   K, group scales:   tt = L%16, dim = 32*(e/8) + 8*(L/16) + e%8;
 *   V, every codec:    tt = 4*(L/16) + e%4, dim = 16*(e/4) + L%16.
 * Elements are little-endian. Codes of fewer than 8 bits fill the run in
 * little-endian units of min(32, run bits) bits holding m codes each; code r
 * of a unit sits at slot (r%2)*(m/2) + r/2 (even codes in the low half):
 * INT4 eight per 32-bit word (nibble slot (r%2)*4 + r/2), INT2 sixteen, BIT1
 * thirty-two, or sixteen in a 16-bit unit at head_dim 64.
 *
 * Threading and ownership. The caller owns every buffer (device memory
 * unless stated otherwise). Calls enqueue work on `stream` (a hipStream_t;
 * NULL is the default stream) and return without synchronizing; buffers must
 * stay valid until that work completes. The library allocates nothing and
 * keeps no state beyond a per-device cache of the compute-unit count, so
 * calls are re-entrant; calls that share an output or a workspace race
 * unless ordered on one stream.
 *
 * Errors. Return values report host-visible problems only. Problems that are
 * visible only on the device (a page id outside [0, num_pages), an unknown
 * codec nibble, a codec other than the one the launch declares, a misaligned
 * plane offset, a plane reaching past pool_bytes, a negative length, ceil(seq_len / page_size) above
 * max_pages_per_row, a selection entry outside [0, max_pages_per_row), a
 * sel_len outside [0, max_sel_pages]) skip the offending page or clamp the
 * row and add one to *err_count per offending entry, so nothing is consumed
 * silently (PR #499 "Design": drop counter against silent corruption).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: partitions are ranges of 16-token tiles (partition_tokens a multiple of
 *    16; 0 splits each row evenly), PKV_CODEC_MIXED_FLOAT.
 * 3: pkv_decode_attention_noalloc, pkv_noalloc_scratch_bytes, PKV_ERR_SCRATCH.
 * 4: pkv_params.window_tokens (sliding-window decode); PKV_INT2_G32, PKV_BIT1_G32. */
#define PKV_ABI_VERSION 4

/* Page codecs; page_codec[p] = K codec | (V codec << 4). */
enum {
  PKV_FP16 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3 = 2,
  PKV_INT8_G32 = 3,
  PKV_INT4_G32 = 4,
  PKV_INT2_G32 = 5,          /* unsigned affine 2-bit: offset + step * u per (token, 32 dims) */
  PKV_BIT1_G32 = 6,          /* 1-bit: sign times a scale per (token, 32 dims) */
  PKV_CODEC_MIXED = -1,      /* pkv_params.k_codec / v_codec: any codec per page and plane */
  PKV_CODEC_MIXED_FLOAT = -2 /* both k_codec and v_codec: each page holds K and V in one of
                                FP16, BF16, FP8 (the same for both planes), chosen per page.
                                Runs a smaller decode kernel than PKV_CODEC_MIXED; a page in
                                another codec is a device-visible error. The prefill treats
                                it as PKV_CODEC_MIXED. */
};

/* Status codes. */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null/misaligned pointer, inconsistent sizes    */
  PKV_ERR_UNSUPPORTED = -2, /* valid request with no kernel (fail closed: the
                               caller falls back; ARGUS "Why decode is slow")  */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required      */
  PKV_ERR_HIP = -4,         /* a HIP launch failed                             */
  PKV_ERR_SCRATCH = -5      /* pkv_decode_attention_noalloc: the partials of the
                               call exceed the library's built-in scratch      */
};

/* Geometry and launch description of one call. Plain values, host memory. */
typedef struct pkv_params {
  int32_t num_rows;          /* B: independent queries (rows) in this call, >= 0        */
  int32_t num_q_heads;       /* Hq                                                      */
  int32_t num_kv_heads;      /* Hkv; Hq % Hkv == 0, G = Hq / Hkv <= 16                   */
  int32_t head_dim;          /* D: 64 or 128                                            */
  int32_t page_size;         /* P tokens per page: a positive multiple of 16; P above
                                2^20, or a 16-bit plane of 4 GiB or more
                                (Hkv * P * D * 2 bytes), is PKV_ERR_UNSUPPORTED: the
                                kernels address a plane with 32-bit offsets      */
  int32_t num_pages;         /* physical pages described by the page tables            */
  int32_t max_pages_per_row; /* row stride of block_table (entries), >= 1               */
  int32_t max_sel_pages;     /* 0: dense mode; > 0: sparse mode, row stride of page_sel */
  int32_t partition_tokens;  /* split-K partition length in tokens, a positive multiple
                                of 16 (decode; prefill: of page_size). A row's 16-token
                                tiles run through its pages (dense) or its selected
                                pages in list order (sparse); partition i covers tiles
                                [i*T/16, (i+1)*T/16), so partitions may split a page.
                                0: the library splits each row's tiles evenly into
                                pkv_num_partitions(p) partitions (decode), or picks a
                                whole-page length (prefill)                              */
  int32_t k_codec;           /* codec of every K plane in this call, or PKV_CODEC_MIXED(_FLOAT) */
  int32_t v_codec;           /* codec of every V plane in this call, or PKV_CODEC_MIXED(_FLOAT) */
  float softmax_scale;       /* tau, finite (1/sqrt(head_dim) in the usual case)        */
  uint64_t pool_bytes;       /* size of page_pool in bytes: a plane that does not fit
                                inside it is a device-visible error                      */
  int32_t window_tokens;     /* decode: sliding window W >= 0 (ARGUS v0.5: direct attention
                                with sliding-window masks): row b attends only positions
                                >= seq_lens[b] - W, its last W; 0: none. Dense mode: the
                                partitions cover the window's tiles only. Must be 0 for
                                pkv_prefill_attention (which takes its window as an
                                argument); ignored by the write side                     */
} pkv_params;

/* PKV_ABI_VERSION of the loaded library. */
int pkv_abi_version(void);

/* Static description of a status code; never NULL. */
const char* pkv_status_string(int status);

/* Partitions each row is split into for these params (>= 1), or a negative
 * status if the params are invalid. Sizes the workspace and the partials.
 * With partition_tokens = 0: as many as fill one round of resident
 * workgroups (the current device's compute units -- 256 on MI355X -- x the
 * kernel's waves per SIMD, four waves per workgroup, rows x KV heads
 * workgroups per partition index), at most one per
 * 8 tiles of the longest row and at least 1; row b's partition i then covers
 * tiles [i c, (i + 1) c), c = max(1, ceil(ceil(L_b / 16) / n)) (dense) or
 * ceil(sel_lens[b] P / 16 / n) (sparse). With a sliding window (dense mode)
 * a row's tiles are counted from tile floor((L_b - W) / 16), the first one
 * the window reaches, and there are at most ceil(W / 16) + 1 of them. */
int pkv_num_partitions(const pkv_params* p);

/* Bytes of device workspace pkv_decode_attention needs for these params:
 * rows*Hq*partitions*(D + 2)*4 when partitions > 1, else 0. Returns 0 for
 * invalid params as well (the decode call then reports the error). */
size_t pkv_workspace_bytes(const pkv_params* p);

/* Decode attention (all steps: table gather, codec decode, scores, online
 * softmax, P.V, partition partials and their log-sum-exp fold).
 *
 *   q            fp16 [B][Hq][D], 16-byte aligned.
 *   page_pool    byte arena holding every plane, 256-byte aligned.
 *   page_k_off,
 *   page_v_off   uint64 [num_pages] byte offsets of the K / V plane of each page.
 *   page_codec   uint8 [num_pages], K codec in the low nibble, V in the high one.
 *   page_scale   fp32 [num_pages][Hkv][2] (K, V) FP8 scales; read only for FP8
 *                planes. May be NULL when neither codec is declared FP8; an
 *                FP8 page met with NULL scales is then a device-visible error.
 *   block_table  int32 [B][max_pages_per_row] physical page of each logical page.
 *   seq_lens     int32 [B] tokens per row.
 *   page_sel     sparse mode: int32 [B][max_sel_pages] logical pages to attend,
 *                any order, no duplicates; NULL in dense mode.
 *   sel_lens     sparse mode: int32 [B] valid entries of each page_sel row.
 *   out          fp32 [B][Hq][D] (written).
 *   lse          fp32 [B][Hq] natural-log log-sum-exp (written).
 *   workspace    device scratch of pkv_workspace_bytes(p) bytes, 16-byte aligned,
 *                NULL allowed when that is 0. Contents need no initialization.
 *   err_count    device int32 counter incremented per device-visible problem,
 *                or NULL. A bad page is counted once by every partition whose
 *                tiles reach it (partitions finer than a page share pages).
 *   stream       hipStream_t to enqueue on (NULL: default stream).
 */
int pkv_decode_attention(const pkv_params* p, const void* q, const uint8_t* page_pool,
                         const uint64_t* page_k_off, const uint64_t* page_v_off,
                         const uint8_t* page_codec, const float* page_scale,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* page_sel, const int32_t* sel_lens, float* out,
                         float* lse, void* workspace, size_t workspace_bytes,
                         int32_t* err_count, void* stream);

/* pkv_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The same work, kernels and results as pkv_decode_attention,
 * bit for bit; the split-K partials go to a scratch array built into the
 * library instead of a caller workspace, so there are no workspace
 * arguments. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).
 *
 * The scratch holds pkv_noalloc_scratch_bytes() bytes (8 MiB) per GPU, from
 * the library's load until the process ends; a call whose
 * pkv_workspace_bytes(p) exceeds it returns PKV_ERR_SCRATCH before touching
 * the device (8 MiB holds, e.g., 16 query heads x 512 partitions of
 * head_dim 128 at 4.3 MB). Every call on one GPU uses that GPU's one array:
 * calls that overlap in time on one GPU (different streams, or different
 * host threads without ordering) race on it and must be serialized by the
 * caller, e.g. by issuing them on one stream. Nothing in the scratch needs to
 * start at zero (every partial a call reads it has written). The first call
 * on a device looks up that device's copy of the array (once per device).
 * Arguments as for pkv_decode_attention. */
int pkv_decode_attention_noalloc(const pkv_params* p, const void* q, const uint8_t* page_pool,
                                 const uint64_t* page_k_off, const uint64_t* page_v_off,
                                 const uint8_t* page_codec, const float* page_scale,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* page_sel, const int32_t* sel_lens, float* out,
                                 float* lse, int32_t* err_count, void* stream);

/* Bytes of the built-in scratch of pkv_decode_attention_noalloc (per GPU). */
size_t pkv_noalloc_scratch_bytes(void);

/* The same work as pkv_decode_attention up to, but not including, the fold:
 * writes the unnormalised partial result of every partition instead of out and
 * lse (the form pkv_lse_combine folds; also the form a caller that splits a row
 * across windows or devices exchanges; PR #499 discussion, in-place host K/V
 * design). Arguments as for pkv_decode_attention, with
 *
 *   part_acc  fp32 [B][Hq][n][D]  sum over the partition of exp(s - m) v,
 *   part_ml   fp32 [B][Hq][n][2]  (m natural-log max, l sum of exp(s - m)),
 *
 * n = pkv_num_partitions(p), both 16-byte aligned. An empty partition writes
 * (0, -inf, 0). No workspace is used.
 */
int pkv_decode_partials(const pkv_params* p, const void* q, const uint8_t* page_pool,
                        const uint64_t* page_k_off, const uint64_t* page_v_off,
                        const uint8_t* page_codec, const float* page_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* page_sel, const int32_t* sel_lens, float* part_acc,
                        float* part_ml, int32_t* err_count, void* stream);

/* Log-sum-exp fold of partial results (PR #499 discussion: windows folded by
 * their log-sum-exp into an fp32 accumulator). For each of `rows` rows:
 *
 *   M = max_p m_p;  w_p = exp(m_p - M);  L = sum_p w_p l_p;
 *   out = sum_p w_p acc_p / L;  lse = M + ln L,
 *
 * summing the parts in a fixed order (run-to-run identical results). A part
 * is empty unless l_p > 0 and m_p is finite (an empty partition writes
 * (0, -inf, 0)); an empty part's acc is never read, and a row whose parts
 * are all empty gets out = 0 and lse = -inf.
 *
 *   part_acc  fp32 [rows][num_parts][head_dim], unnormalised sum exp(s - m_p) v.
 *   part_ml   fp32 [rows][num_parts][2] = (m_p natural-log max, l_p sum).
 *   out       fp32 [rows][head_dim];  lse  fp32 [rows].
 * rows >= 0, num_parts >= 1, 1 <= head_dim <= 512; pointers 4-byte aligned.
 */
int pkv_lse_combine(int32_t rows, int32_t num_parts, int32_t head_dim, const float* part_acc,
                    const float* part_ml, float* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Write side: the steps right before this read path, producing exactly the
 * page format it reads. Recent pages stay 16-bit while they fill; full older
 * pages are re-encoded into a compact codec (ARGUS "Adaptive activation" and
 * "v0.5": tiered pages, FP16 for the recent window). FP8 pages hold e4m3
 * codes plus fp32 scales (FreeToken PR #499 update, item 1); INT8/INT4 pages
 * hold one fp16 scale per token and group of 32 (GGML Q8/Q4 pages).
 * Both calls use num_rows (append only), num_kv_heads, head_dim (64 or 128),
 * page_size, num_pages, max_pages_per_row (append only) and pool_bytes of p;
 * the other fields are ignored. Asynchronous on `stream`, like the rest.
 * ------------------------------------------------------------------------- */

/* Stores one new token per row in its 16-bit page.
 *
 *   k_new, v_new  fp16 [num_rows][Hkv][D], 2-byte aligned.
 *   seq_lens      [num_rows] lengths BEFORE the append: row b's token goes to
 *                 slot seq_lens[b] % P of logical page seq_lens[b] / P, i.e.
 *                 physical page block_table[b][seq_lens[b] / P]. The caller
 *                 advances seq_lens afterwards.
 *   Other tables as in pkv_decode_attention; the page's K and V planes must
 *   be FP16 or BF16 (a BF16 plane stores the value rounded to nearest even).
 *
 * Writes 2*Hkv*D codes per row and nothing else. A row whose length is
 * negative or beyond max_pages_per_row, whose page id is out of range, whose
 * page is not 16-bit in both planes or either of whose planes is misaligned
 * or lies outside the pool is counted once in *err_count (if given) and
 * skipped: neither plane is written. Host-visible errors as in
 * pkv_decode_attention. */
int pkv_append_kv(const pkv_params* p, const void* k_new, const void* v_new, uint8_t* page_pool,
                  const uint64_t* page_k_off, const uint64_t* page_v_off, const uint8_t* page_codec,
                  const int32_t* block_table, const int32_t* seq_lens, int32_t* err_count, void* stream);

/* Re-encodes n full 16-bit pages into another codec (demotion).
 *
 *   src_pages, dst_pages  [n] physical page ids: page src_pages[i] (FP16 or
 *                 BF16 in both planes) is read, every slot of it, and page
 *                 dst_pages[i] is written. The destination planes live at
 *                 page_k_off / page_v_off[dst] (16-byte aligned, inside the
 *                 pool, sized for dst_codec) and must overlap neither the
 *                 source planes nor each other. No destination may appear
 *                 twice, or as a source of another pair, in one call (not
 *                 checked).
 *   dst_codec     K codec in the low nibble, V codec in the high nibble:
 *                 FP16, BF16, FP8 e4m3, INT8, INT4, INT2 or BIT1. Encoding,
 *                 decided in fp32:
 *                   FP8: s = fp32(absmax / 448) per (page, KV head, plane),
 *                        1 if the block is all zero; code = e4m3 nearest to
 *                        fp32(x / s), ties to even.
 *                   INT8/INT4: s = fp16(fp32(absmax) / qmax) per (token, 32
 *                        dims), qmax 127 / 7, kept inside fp16's finite range
 *                        [2^-24, 65504], 1 if the group is all zero;
 *                        code = clip(rint(fp32(x) / fp32(s)), -qmax, qmax).
 *                   INT2: per (token, 32 dims) z = fp16(min) (saturated to
 *                        +-65504), s = fp16(fp32(max - z) / 3) kept inside
 *                        [2^-24, 65504], 1 when max - z <= 0;
 *                        u = clip(rint(fp32(x - z) / s), 0, 3).
 *                   BIT1: per (token, 32 dims) s = fp16(fp32(sum |x| / 32)),
 *                        the sum taken in float64 (exact for 16-bit sources),
 *                        capped at 65504; bit = x < 0.
 *                   BF16/FP16: the value, rounded to nearest even.
 *                 Source values are expected finite (infinities saturate
 *                 the INT codes); the codes of a block or group holding a
 *                 NaN are unspecified.
 *   page_codec    page_codec[dst] is set to dst_codec.
 *   page_scale    [num_pages][Hkv][2]; page_scale[dst][h] is set to the FP8
 *                 scales (1 for a plane in another codec). May be NULL only
 *                 if neither plane is FP8.
 *
 * A pair with an id out of range, equal ids, a source that is not 16-bit,
 * a plane outside the pool, a misaligned plane or overlapping planes -- in
 * either plane -- is counted once in *err_count (if given) and skipped
 * whole: no byte of either destination plane, no scale and no page_codec
 * entry of it is written. Host-visible errors as in
 * pkv_decode_attention; PKV_ERR_INVALID_ARG also for a bad codec nibble or a
 * missing page_scale. */
int pkv_encode_pages(const pkv_params* p, int32_t n, const int32_t* src_pages, const int32_t* dst_pages,
                     int32_t dst_codec, uint8_t* page_pool, const uint64_t* page_k_off,
                     const uint64_t* page_v_off, uint8_t* page_codec, float* page_scale, int32_t* err_count,
                     void* stream);

/* ---------------------------------------------------------------------------
 * Chunked prefill: a chunk of new query tokens per row attends the cache,
 * window by window, with the windows folded by their log-sum-exp into an
 * fp32 accumulator (FreeToken PR #499 discussion, in-place host K/V design;
 * ARGUS "Why decode is slow" for grouped-query attention).
 *
 * The chunk's T = q_tokens tokens have already been appended, so they are
 * the last T of row b's L = seq_lens[b] tokens: query t sits at position
 * pos = L - T + t and attends, causally, the keys
 *
 *     j in [max(kv_begin, pos + 1 - W), min(kv_end, pos + 1))
 *
 * (kv_end < 0: no bound; W = window_tokens, the sliding window: each query
 * sees at most its last W positions, its own included; W <= 0: none; ARGUS
 * v0.5: direct attention with sliding-window masks)
 * with the scores, softmax, out and lse of pkv_decode_attention (natural-log
 * lse; an empty key set, e.g. pos < 0 when T > L, gives out = 0 and
 * lse = -inf). With T = 1, the whole range and no sliding window this is the
 * decode result (with a sliding window, T = 1 is sliding-window decode). The
 * key range is split into partitions of partition_tokens (0: chosen by the
 * library: as many as fill one round of resident workgroups, whole pages of
 * at least 256 tokens) starting at kv_begin rounded down to a page boundary; their
 * partials are folded as by pkv_lse_combine. With a sliding window, passing
 * kv_begin = (the smallest first-query position) - W + 1 lets the partitions
 * cover only the keys in play.
 *
 * FP8 page scales must be finite here. The V page scale s enters the
 * softmax in the log domain (log2|s| added to the page's scores, 1/|s| on the
 * weights' sum, its sign on the weights): |s| below 2^-40 is taken as 2^-40
 * (a V value moves by less than 4.1e-10) and |s| above 2^40 is outside the
 * supported domain (the encoder's scales lie in [2^-33, 147]).
 *
 * Dense mode only: max_sel_pages must be 0. Codecs (all seven; BF16 as
 * described with the codecs), the page tables, the device-visible error
 * counting and the threading rules are those of pkv_decode_attention (each
 * bad page is counted once per partition and row).
 */

/* Partitions of the key range for this call (>= 1), or a negative status. */
int pkv_prefill_num_partitions(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end);

/* Device workspace bytes pkv_prefill_attention needs:
 * rows*q_tokens*Hq*partitions*(D + 2)*4 when partitions > 1, else 0 (also 0
 * for invalid arguments; the call then reports the error). */
size_t pkv_prefill_workspace_bytes(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end);

/*   q          fp16 [B][q_tokens][Hq][D], 16-byte aligned.
 *   out        fp32 [B][q_tokens][Hq][D] (written).
 *   lse        fp32 [B][q_tokens][Hq] (written).
 *   workspace  pkv_prefill_workspace_bytes() bytes, 16-byte aligned (NULL when 0).
 * Other arguments as for pkv_decode_attention. Returns PKV_ERR_INVALID_ARG for
 * q_tokens < 0, kv_begin < 0, 0 <= kv_end < kv_begin or max_sel_pages != 0. */
int pkv_prefill_attention(const pkv_params* p, int32_t q_tokens, int32_t kv_begin, int32_t kv_end,
                          int32_t window_tokens, const void* q, const uint8_t* page_pool, const uint64_t* page_k_off,
                          const uint64_t* page_v_off, const uint8_t* page_codec, const float* page_scale,
                          const int32_t* block_table, const int32_t* seq_lens, float* out, float* lse,
                          void* workspace, size_t workspace_bytes, int32_t* err_count, void* stream);

/* Folds one window's result into a running accumulator, in place (PR #499
 * discussion: windows folded by log-sum-exp into an fp32 accumulator). Per
 * row r, with M = max(acc_lse[r], lse[r]), w_a = exp(acc_lse[r] - M) and
 * w_b = exp(lse[r] - M):
 *
 *   acc_out[r] = (w_a acc_out[r] + w_b out[r]) / (w_a + w_b)
 *   acc_lse[r] = M + ln(w_a + w_b)
 *
 * A side with lse = -inf contributes nothing (its out values are not read
 * into the result); both -inf gives acc_out = 0, acc_lse = -inf. Start an
 * accumulator with acc_lse = -inf. acc_out, out fp32 [rows][head_dim];
 * acc_lse, lse fp32 [rows]; 4-byte aligned; 1 <= head_dim <= 512. */
int pkv_lse_fold_into(int32_t rows, int32_t head_dim, float* acc_out, float* acc_lse, const float* out,
                      const float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Page selection for the sparse path: an indexer's block top-k over a
 * compressed slab, and the selected pages compacted into the fixed-capacity
 * page_sel / sel_lens arrays that pkv_decode_attention reads in sparse mode
 * (FreeToken PR #499 "Why this works": top-k block selection over a
 * compressed slab, on the GPU, fixed shape; "Design": compaction with a drop
 * counter, capacity 2 * block_topk + 8).
 *
 * Row b's L = seq_lens[b] tokens are cut into blocks of block_tokens; block j
 * covers [j*BT, min((j+1)*BT, L)). Its score is the dot product of the row's
 * indexer query q_idx[b] with the block's summary slab[b][j], both fp16,
 * accumulated in fp32 in index order (one rounding per term; reproducible bit
 * for bit). The block_topk best scores are taken (ties to the lower block,
 * NaN below every number; all blocks when block_topk >= their number). The
 * selection is every page a chosen block touches, plus the row's first
 * sink_pages and last recent_pages pages, in ascending order; the first
 * max_sel_pages are written to page_sel[b], sel_lens[b] gets their number,
 * and *dropped grows by the pages that did not fit.
 */

/* Pages a selection can need at most: with g = gcd(BT, P), a block touches at
 * most (P - g + BT - 1) / P + 1 pages, so this is that times block_topk plus
 * sink_pages + recent_pages (for BT <= P and sink + recent = 8, at most the
 * pages' 2 * block_topk + 8). Negative status for invalid arguments. */
int pkv_select_capacity(int32_t page_size, int32_t block_tokens, int32_t block_topk, int32_t sink_pages,
                        int32_t recent_pages);

/* Uses p->num_rows (B), p->page_size (P), p->max_pages_per_row (rows longer
 * than max_pages_per_row * P are clamped and counted in *err_count; at most
 * 262,144) and p->max_sel_pages (the capacity of a page_sel row, >= 1).
 *   q_idx         fp16 [B][idx_dim], idx_dim a positive multiple of 8 (<= 4096).
 *   slab          fp16 [B][max_blocks][idx_dim], 16-byte aligned; a row with
 *                 more than max_blocks blocks is cut to max_blocks and counted
 *                 in *err_count. A row of the slab, (max_blocks + 64) * idx_dim
 *                 * 2 bytes, must stay below 4 GiB - 64 KiB (PKV_ERR_UNSUPPORTED
 *                 otherwise).
 *   block_scores  fp32 [B][max_blocks]: written with the scores of the row's
 *                 blocks (the scratch the selection reads).
 *   page_sel      int32 [B][max_sel_pages], sel_lens int32 [B] (written).
 *   dropped, err_count  device int32 counters, or NULL.
 */
int pkv_select_pages(const pkv_params* p, int32_t block_tokens, int32_t block_topk, int32_t sink_pages,
                     int32_t recent_pages, int32_t idx_dim, int32_t max_blocks, const void* q_idx, const void* slab,
                     const int32_t* seq_lens, float* block_scores, int32_t* page_sel, int32_t* sel_lens,
                     int32_t* dropped, int32_t* err_count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
