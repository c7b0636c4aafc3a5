"""Pins for oracle/select.py (block top-k page selection and compaction), no
GPU.

Checked against things other than the oracle: exact integer dot products
where every partial sum is representable (closed form), the float32 rounding
bound against math.fsum elsewhere, the defining properties of a top-k with
ties to the lower index (every selected score >= every other, the lowest
indices among ties) and numpy's argpartition on distinct scores, pages found
by mapping every token of a block to its page (brute force), and the pages'
capacity 2 * block_topk + 8.
"""
import math

import numpy as np
import pytest

from oracle.select import block_scores, capacity, select_pages, top_blocks


def test_scores_exact_on_small_integers():
    rng = np.random.default_rng(1)
    q = rng.integers(-8, 9, 64).astype(np.float16)
    s = rng.integers(-8, 9, (50, 64)).astype(np.float16)
    got = block_scores(q, s, 50)
    want = s.astype(np.int64) @ q.astype(np.int64)
    assert np.array_equal(got, want.astype(np.float32))


def test_scores_within_float32_bound():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(128).astype(np.float16)
    s = (rng.standard_normal((200, 128)) * 3).astype(np.float16)
    got = block_scores(q, s, 200).astype(np.float64)
    for j in range(200):
        terms = [float(q[i]) * float(s[j, i]) for i in range(128)]
        exact = math.fsum(terms)
        bound = 128 * 2.0 ** -24 * math.fsum(abs(t) for t in terms)
        assert abs(got[j] - exact) <= bound
    assert block_scores(q, s, 7).shape == (7,)


def top_k_properties(scores, k, sel):
    n = scores.shape[0]
    assert sel.size == min(k, n) and np.all(np.diff(sel) > 0)
    rest = np.setdiff1d(np.arange(n), sel)
    fin = lambda a: a[~np.isnan(scores[a])]
    if rest.size and sel.size:
        lo_sel = np.nanmin(scores[sel]) if fin(sel).size else -np.inf
        hi_rest = np.nanmax(scores[rest]) if fin(rest).size else -np.inf
        # no unselected number beats a selected number; NaN only if numbers ran out
        assert hi_rest <= lo_sel
        if np.isnan(scores[sel]).any():
            assert fin(rest).size == 0
        # ties at the threshold go to the lower indices
        t = lo_sel
        tied_rest = rest[scores[rest] == t]
        tied_sel = sel[scores[sel] == t]
        if tied_rest.size and tied_sel.size:
            assert tied_sel.max() < tied_rest.min()


@pytest.mark.parametrize("seed", range(6))
def test_top_blocks_properties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    scores = rng.integers(-5, 6, n).astype(np.float32)       # many ties
    if seed % 2:
        scores[rng.random(n) < 0.1] = np.nan
    for k in (0, 1, 7, n // 2, n, n + 5):
        sel = top_blocks(scores, k)
        top_k_properties(scores, k, sel)


def test_top_blocks_equals_argpartition_on_distinct_scores():
    rng = np.random.default_rng(9)
    scores = rng.permutation(1000).astype(np.float32) * 0.5
    for k in (1, 10, 333, 999):
        want = np.sort(np.argpartition(-scores, k - 1)[:k])
        assert np.array_equal(top_blocks(scores, k), want)


def pages_by_tokens(blocks, L, P, BT):
    pages = set()
    for j in blocks:
        for t in range(j * BT, min((j + 1) * BT, L)):
            pages.add(t // P)
    return pages


@pytest.mark.parametrize("P,BT", [(16, 16), (16, 8), (16, 24), (32, 48), (64, 64), (16, 1), (16, 40)])
def test_pages_of_blocks_brute_force(P, BT):
    rng = np.random.default_rng(P + BT)
    L = int(rng.integers(1, 2000))
    nb = -(-L // BT)
    D = 32
    q = rng.standard_normal(D).astype(np.float16)
    slab = rng.standard_normal((nb + 3, D)).astype(np.float16)
    k = int(rng.integers(0, nb + 2))
    pages, dropped, scores = select_pages(q, slab, L, P, BT, k, 2, 3, 10 ** 6)
    chosen = top_blocks(block_scores(q, slab, nb), k) if k else []
    want = pages_by_tokens(chosen, L, P, BT)
    npages = -(-L // P)
    want |= set(range(min(2, npages))) | set(range(max(npages - 3, 0), npages))
    assert list(pages) == sorted(want) and dropped == 0
    assert len(pages) <= capacity(P, BT, k, 2, 3)


def test_capacity_is_exact_and_within_the_pages_bound():
    # brute force over block positions: the bound is the worst case exactly
    for P, BT in ((16, 24), (16, 40), (32, 5), (16, 16), (16, 8), (16, 12), (64, 100), (16, 1)):
        worst = max(len(pages_by_tokens([j], 10 ** 6, P, BT)) for j in range(300))
        assert worst == capacity(P, BT, 1, 0, 0), (P, BT)
    # block_tokens <= page_size, sink + recent = 8: within the pages' 2 * block_topk + 8,
    # and equal to it when blocks straddle page boundaries
    for BT in (2, 8, 12, 16, 5):
        assert capacity(16, BT, 32, 4, 4) <= 2 * 32 + 8
    assert capacity(16, 12, 32, 4, 4) == 2 * 32 + 8


def test_drops_are_counted_and_the_lowest_pages_kept():
    rng = np.random.default_rng(4)
    L, P, BT, D = 1000, 16, 16, 32
    q = rng.standard_normal(D).astype(np.float16)
    slab = rng.standard_normal((63, D)).astype(np.float16)
    full, d0, _ = select_pages(q, slab, L, P, BT, 20, 1, 1, 100)
    assert d0 == 0 and 20 <= len(full) <= 22
    part, d1, _ = select_pages(q, slab, L, P, BT, 20, 1, 1, 10)
    assert np.array_equal(part, full[:10]) and d1 == len(full) - 10


def test_edge_cases():
    q = np.ones(8, np.float16)
    slab = np.ones((4, 8), np.float16)
    p, d, s = select_pages(q, slab, 0, 16, 16, 5, 1, 1, 10)
    assert p.size == 0 and d == 0
    p, d, _ = select_pages(q, slab, 40, 16, 16, 0, 0, 0, 10)      # nothing asked for
    assert p.size == 0
    p, d, _ = select_pages(q, slab, 40, 16, 16, 0, 5, 5, 10)      # forced pages clipped to 3 pages
    assert list(p) == [0, 1, 2]
    p, d, _ = select_pages(q, slab, 40, 16, 16, 99, 0, 0, 10)     # k beyond the blocks
    assert list(p) == [0, 1, 2]
