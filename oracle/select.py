"""GPU page selection, from its definition: block top-k by an indexer score
over a compressed slab, then fixed-capacity compaction of the pages those
blocks touch, with a drop counter.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Definition followed (FreeToken PR #499 "Why this works": every sparse step
first runs an indexer that takes a top-k of blocks over a compressed slab on
the GPU, then reads only the selected pages; PR #499 "Design": the selected
pages are compacted into a fixed-shape array whose capacity is
2 * block_topk + 8, with a counter of entries that did not fit):

* Blocks. Row b's tokens 0 .. L-1 are cut into blocks of ``block_tokens``;
  block j covers [j*BT, min((j+1)*BT, L)). There are ceil(L / BT) blocks.
* Score. The slab holds one summary vector per block (fp16, ``idx_dim``
  values); the row's indexer query is q_idx (fp16). score_j is their dot
  product accumulated in float32 in index order, one rounding per step:
  acc = fp32(acc + q_i * s_i) for i = 0 .. idx_dim-1, from acc = 0 (each
  product of two fp16 values is exact in float32). A NaN score ranks below
  every number.
* Top-k. The block_topk highest scores; among equal scores the lower block
  index wins. All blocks when block_topk >= the number of blocks.
* Pages. A selected block contributes every logical page it touches, pages
  floor(j*BT / P) .. floor((min((j+1)*BT, L) - 1) / P). The first
  ``sink_pages`` and the last ``recent_pages`` pages of the row are always
  included (clipped to the row's ceil(L / P) pages).
* Compaction. The distinct pages in ascending order; the first max_sel of
  them are written, the rest are dropped and counted.

Pinned in tests/test_oracle_select.py.
"""
from __future__ import annotations

import math

import numpy as np


def block_scores(q_idx: np.ndarray, slab: np.ndarray, nblocks: int) -> np.ndarray:
    """float32 [nblocks]: sequential float32 dot products of q_idx (fp16
    [idx_dim]) with slab[j] (fp16 [.., idx_dim]) for j < nblocks."""
    q = np.asarray(q_idx, dtype=np.float16).astype(np.float32)
    s = np.asarray(slab[:nblocks], dtype=np.float16).astype(np.float32)
    acc = np.zeros(nblocks, dtype=np.float32)
    for i in range(q.shape[0]):
        acc = (acc + q[i] * s[:, i]).astype(np.float32)     # product exact, one rounding per add
    return acc


def top_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best blocks (NaN lowest, ties to the lower index),
    ascending."""
    n = scores.shape[0]
    if k >= n:
        return np.arange(n)
    key = np.where(np.isnan(scores), -np.inf, scores.astype(np.float64))
    # NaN below -inf: sort on (is_nan, -score, index)
    order = np.lexsort((np.arange(n), -key, np.isnan(scores)))
    return np.sort(order[:k])


def select_pages(q_idx, slab, L: int, page_size: int, block_tokens: int, block_topk: int,
                 sink_pages: int, recent_pages: int, max_sel: int):
    """One row. Returns (pages int32 [n <= max_sel] ascending, dropped count,
    block scores float32)."""
    L = int(L)
    if L <= 0:
        return np.zeros(0, dtype=np.int32), 0, np.zeros(0, dtype=np.float32)
    nblocks = -(-L // block_tokens)
    npages = -(-L // page_size)
    scores = block_scores(q_idx, slab, nblocks)
    chosen = top_blocks(scores, block_topk) if block_topk > 0 else np.zeros(0, dtype=np.int64)
    pages = set()
    for j in chosen:
        lo = int(j) * block_tokens
        hi = min((int(j) + 1) * block_tokens, L)
        pages.update(range(lo // page_size, (hi - 1) // page_size + 1))
    pages.update(range(min(sink_pages, npages)))
    pages.update(range(max(npages - recent_pages, 0), npages))
    allp = np.array(sorted(pages), dtype=np.int32)
    kept = allp[:max_sel]
    return kept, int(allp.size - kept.size), scores


def capacity(page_size: int, block_tokens: int, block_topk: int, sink_pages: int, recent_pages: int) -> int:
    """Pages a selection can need at most. Block starts are multiples of BT,
    so their offsets inside a page are multiples of g = gcd(BT, P); the
    furthest, P - g, makes a block touch (P - g + BT - 1) // P + 1 pages. With
    BT <= P that is at most 2, so with sink + recent = 8 the capacity is at
    most the pages' 2 * block_topk + 8."""
    g = math.gcd(block_tokens, page_size)
    per_block = (page_size - g + block_tokens - 1) // page_size + 1
    return per_block * block_topk + sink_pages + recent_pages
