"""The five decode workloads and scaled-down variants of them.

Shapes follow the workloads the pages discuss: Qwen2.5-0.5B-like geometry
(14 query / 2 KV heads, head_dim 64, 1024-token pages; ARGUS "What is proven
today"), ARGUS's FP16 -> FP8 tiering of older pages ("Adaptive activation"),
GGML Q8/Q4-style group codecs ("v0.5"), FreeToken's sparse selected-page
decode with FP8 pages (PR #499 "What", "Why this works") and the 1M-token
window folded by log-sum-exp (PR #499 discussion, in-place host K/V design).

``scale`` < 1 shrinks context lengths (and rows) so the CPU oracle finishes in
seconds while the shape of the workload (codecs, ragged tails, placement,
selection) stays the same.
"""
from __future__ import annotations

import numpy as np

from .layout import BIT1, FP8, FP16, INT2, INT4, INT8
from .workload import Workload, build_workload, streams

NAMES = {
    1: "tiny_fp16_4k",
    2: "mixed_fp16_fp8_24layer_16k",
    3: "batched_int8k_int4v_32k",
    4: "sparse_fp8_selected_262k",
    5: "splitk_fp8_1m",
}


def config(cid: int, small: bool = False) -> Workload:
    """Build workload ``cid`` (1..5). ``small`` gives the reduced test variant."""
    seed = 1000 + cid
    rng = streams(seed)
    if cid == 1:
        return build_workload(NAMES[1], rows=1, hq=14, hkv=2, dim=64, page=1024,
                              seq_lens=[4096], codec_of=lambda r, lp: (FP16, FP16),
                              seed=seed, rng=rng, partition_tokens=1024,
                              info={"config": 1, "layers": 1, "batch": 1})
    if cid == 2:
        layers, page = (24, 1024) if not small else (3, 64)
        pages = 16
        fp16_from = pages - 4                       # newest 4 logical pages stay FP16
        return build_workload(
            NAMES[2] + ("_small" if small else ""), rows=layers, hq=14, hkv=2, dim=64,
            page=page, seq_lens=[pages * page] * layers,
            codec_of=lambda r, lp: (FP16, FP16) if lp >= fp16_from else (FP8, FP8),
            seed=seed, rng=rng, outlier_frac=0.01, outlier_mult=8.0,
            partition_tokens=0 if not small else page, info={"config": 2, "layers": layers, "batch": 1})
    if cid == 3:
        rows, lo, hi, width = (8, 24576, 32768, 2048) if not small else (3, 300, 700, 48)
        lens = rng["lengths"].integers(lo, hi, endpoint=True, size=rows)
        return build_workload(
            NAMES[3] + ("_small" if small else ""), rows=rows, hq=32, hkv=8, dim=128,
            page=16, seq_lens=lens, codec_of=lambda r, lp: (INT8, INT4), seed=seed,
            rng=rng, max_pages=width, partition_tokens=0 if not small else 128,
            info={"config": 3, "layers": 1, "batch": rows})
    if cid == 4:
        layers, batch, ctx, nsel = (12, 4, 262144, 128) if not small else (2, 2, 4096, 16)
        rows = layers * batch
        lp_count = ctx // 16
        sel = np.empty((rows, nsel), dtype=np.int32)
        for r in range(rows):
            pick = rng["selection"].choice(lp_count - 1, size=nsel - 1, replace=False)
            sel[r] = np.sort(np.append(pick, lp_count - 1))
        return build_workload(
            NAMES[4] + ("_small" if small else ""), rows=rows, hq=16, hkv=2, dim=128,
            page=16, seq_lens=[ctx] * rows, codec_of=lambda r, lp: (FP8, FP8),
            seed=seed, rng=rng, selection=sel, logical_pages=lp_count,
            partition_tokens=256 if not small else 64,
            info={"config": 4, "layers": layers, "batch": batch})
    if cid == 5:
        ctx, page, part = (1 << 20, 64, 2048) if not small else (1 << 14, 64, 512)
        return build_workload(
            NAMES[5] + ("_small" if small else ""), rows=1, hq=16, hkv=2, dim=128,
            page=page, seq_lens=[ctx], codec_of=lambda r, lp: (FP8, FP8), seed=seed,
            rng=rng, q_scale=3.6, partition_tokens=part,
            info={"config": 5, "layers": 1, "batch": 1})
    raise ValueError(cid)


def effective_kv_bytes_formula(w: Workload) -> int:
    """Codes + scales of the attended tokens, per the in-page layout."""
    from .layout import CODEC_BITS
    d, hkv, p = w.head_dim, w.num_kv_heads, w.page_size
    total = 0
    for r, pages in enumerate(w.attended_pages()):
        for lp, valid in pages:
            pp = int(w.block_table[r, lp])
            c = int(w.page_codec[pp])
            for codec in (c & 15, c >> 4):
                per_tok = d * CODEC_BITS[codec] // 8
                if codec in (INT8, INT4, BIT1):
                    per_tok += (d // 32) * 2
                elif codec == INT2:
                    per_tok += 2 * (d // 32) * 2          # scales and offsets
                total += hkv * valid * per_tok
                if codec == FP8:
                    total += hkv * 4        # one fp32 scale per (page, head, plane)
    return total
