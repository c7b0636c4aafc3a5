"""CPU float64 oracle for mixed-codec paged decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The
library's product path (``paged_kv_cache_182_amd``) never imports it, and this
package shares no code with that path: codec decoding, the in-page layout
reader, attention and the log-sum-exp fold are all written here from their
definitions.

What it computes (sources are the three pages' own sections):

* Codec values (``codecs``): FP16/BF16 pages; FP8 e4m3 codes times an fp32
  scale (FreeToken PR #499 update, item 1); INT8/INT4 with one scale per group
  of 32 along head_dim (GGML Q8/Q4 pages in ARGUS "v0.5" and "Direct paged
  attention"); the INT2 and 1-bit tiers of ARGUS's cascade (intro), INT2 as
  the unsigned-affine 2-bit kind of "Pluggable tiers" (offset + step * u per
  group of 32) and 1-bit as sign times a group scale.
* Attention (``attention``): for each query head, softmax over every attended
  token of the scaled q.k score, applied to V -- the exact result that ARGUS's
  page-at-a-time online-softmax recurrence reaches ("Why decode is slow",
  "Direct paged attention"). Tokens come from the block table in logical order
  (FreeToken PR #499 "Design": logical -> physical translation), or only from
  the selected pages in sparse mode (PR #499 "Why this works").
* Fold (``attention.fold``): partial results combined through their
  log-sum-exp into one result (PR #499 discussion, in-place host K/V design:
  windows folded by log-sum-exp into an fp32 accumulator).
* Byte accounting (``accounting``): bytes of codes + scales, pinned to the
  memory figures ARGUS prints for its engine at 32K ("Direct paged attention").
* Write side (``encode``): a new token appended into its 16-bit page, and
  full 16-bit pages re-encoded (demoted) to FP8 / INT8 / INT4 (ARGUS "v0.5"
  and "Adaptive activation"; FreeToken PR #499 update, item 1).
* Chunked prefill (``prefill``): a chunk of new query tokens per row attends
  the cache causally, window by window, and the windows' results are folded
  by their log-sum-exp into an accumulator (PR #499 discussion, in-place host
  K/V design).
* Page selection (``select``): an indexer's block top-k over a compressed
  slab, and the selected pages compacted into a fixed-capacity list with a
  drop counter (PR #499 "Why this works" and "Design").

Pins live in ``tests/test_oracle_*.py``; see each function for what pins it.
"""
from .codecs import (decode_bf16, decode_bit1, decode_fp16, decode_fp8_e4m3, decode_int4,  # noqa: F401
                     decode_int8, decode_uint2)
from .attention import decode_attention, fold, gather_kv, partials  # noqa: F401
from .accounting import kv_bytes_per_token  # noqa: F401
from .encode import append_token, encode_page  # noqa: F401
from .prefill import fold_into, prefill_attention  # noqa: F401
from .select import select_pages  # noqa: F401
