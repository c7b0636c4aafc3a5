"""GPU page selection vs the oracle (oracle/select.py): block scores bit for
bit, the selected pages and their count exactly, drops exactly; and the
selection feeding the sparse decode path end to end."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_182_amd as pkv
import synth
from oracle.select import select_pages as ref_select
from synth.device import to_device
from synth.layout import FP8
from gpu_util import compare, params_for

pytestmark = pytest.mark.gpu


def run_select(lens, P, BT, k, sink, recent, idx_dim, max_sel, max_pages, q, slab, expect_err=0):
    rows = len(lens)
    p = pkv.make_params(rows=rows, num_q_heads=1, num_kv_heads=1, head_dim=128, page_size=P, num_pages=1,
                        max_pages_per_row=max_pages, pool_bytes=0, max_sel_pages=max_sel)
    dropped = torch.zeros(1, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    sel, n, sc = pkv.select_pages(p, torch.from_numpy(q).cuda(), torch.from_numpy(slab).cuda(),
                                  torch.tensor(lens, dtype=torch.int32, device="cuda"), block_tokens=BT,
                                  block_topk=k, sink_pages=sink, recent_pages=recent, dropped=dropped,
                                  err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == expect_err
    return sel.cpu().numpy(), n.cpu().numpy(), sc.cpu().numpy(), int(dropped.item())


def check(lens, P, BT, k, sink, recent, idx_dim, max_sel, seed, ties=False, nan=False, nan_frac=0.05):
    rng = np.random.default_rng(seed)
    max_pages = max(-(-max(lens) // P), 1)
    max_blocks = max(-(-max(lens) // BT), 1)
    rows = len(lens)
    if ties:
        q = rng.integers(-2, 3, (rows, idx_dim)).astype(np.float16)
        slab = rng.integers(-2, 3, (rows, max_blocks, idx_dim)).astype(np.float16)
    else:
        q = rng.standard_normal((rows, idx_dim)).astype(np.float16)
        slab = (rng.standard_normal((rows, max_blocks, idx_dim)) * 2).astype(np.float16)
    if nan:
        slab[rng.random((rows, max_blocks)) < nan_frac, 3] = np.nan
    sel, n, sc, dropped = run_select(lens, P, BT, k, sink, recent, idx_dim, max_sel, max_pages, q, slab)
    total_drop = 0
    for r, L in enumerate(lens):
        pages, drop, scores = ref_select(q[r], slab[r], L, P, BT, k, sink, recent, max_sel)
        nb = scores.shape[0]
        assert np.array_equal(sc[r, :nb].view(np.uint32), scores.view(np.uint32)), f"scores row {r}"
        assert n[r] == len(pages) and np.array_equal(sel[r, :n[r]], pages), f"pages row {r}"
        total_drop += drop
    assert dropped == total_drop
    return sel, n


@pytest.mark.parametrize("P,BT", [(16, 16), (16, 8), (16, 24), (32, 48), (64, 64), (16, 5)])
def test_selection_matches_oracle(P, BT):
    print(f"case P={P} BT={BT}", flush=True)
    lens = [1, 15, 17, 300, 2049, 0, 5000]
    for k in (0, 1, 7, 40, 10 ** 6):
        check(lens, P, BT, k, 1, 2, 64, 400, seed=P + BT + k)


@pytest.mark.parametrize("idx_dim", [8, 64, 128, 136])
def test_ties_and_nan_scores(idx_dim):
    lens = [4000, 333, 16384]
    check(lens, 16, 16, 50, 0, 1, idx_dim, 200, seed=idx_dim, ties=True)
    check(lens, 16, 16, 50, 0, 1, idx_dim, 200, seed=idx_dim + 1, ties=True, nan=True)
    check(lens, 16, 16, 3000, 0, 0, idx_dim, 2000, seed=idx_dim + 2, nan=True)


def test_drops_counted():
    lens = [5000, 6000, 100]
    check(lens, 16, 24, 64, 4, 4, 64, 20, seed=3)           # capacity far below the need
    cap = pkv.select_capacity(16, 24, 64, 4, 4)
    _, n = check(lens, 16, 24, 64, 4, 4, 64, cap, seed=3)  # the library's capacity: nothing dropped
    assert n.max() <= cap


def test_large_rows_radix_select():
    """16,384 blocks per row (a 262,144-token context of 16-token pages), the
    sparse workload's selection shape: 127 blocks + the last page."""
    lens = [262144, 262144 - 5, 131072]
    check(lens, 16, 16, 127, 0, 1, 64, pkv.select_capacity(16, 16, 127, 0, 1), seed=11)
    check(lens, 16, 16, 127, 0, 1, 64, 128, seed=12, ties=True)


def test_select_search_paths():
    """Each way the k-th best key is found: per-wave candidates with one wave
    searching them (16,384 blocks, k 127), the same with 32 keys per thread
    (20,000 blocks), the search over every key when the candidates overflow
    (k 300 on 16,384 blocks: at least 300 from each of 16 waves), keys re-read
    from memory per step (40,000 blocks), and a row whose k-th key is a NaN
    score (the lowest key)."""
    print("case 16,384 / 20,000 / 40,000 blocks", flush=True)
    cap = pkv.select_capacity(16, 16, 127, 0, 1)
    check([262144, 20000 * 16 - 3, 40000 * 16], 16, 16, 127, 0, 1, 64, cap, seed=31)
    check([262144, 20000 * 16, 40000 * 16 - 9], 16, 16, 127, 0, 1, 64, cap, seed=32, ties=True)
    print("case candidate overflow", flush=True)
    check([262144, 262144 - 100], 16, 16, 300, 0, 1, 64, pkv.select_capacity(16, 16, 300, 0, 1), seed=33)
    print("case k-th key a NaN", flush=True)
    check([16 * 1000, 16 * 5000], 16, 16, 700, 0, 0, 64, 1000, seed=34, nan=True, nan_frac=0.5)


@pytest.mark.parametrize("idx_dim", [64, 128])
def test_many_rows_ragged_short_and_empty(idx_dim):
    """34 rows of up to 16,384 blocks (2,176 scoring workgroups), ragged,
    short and empty: workgroups past a row's last block have nothing to do,
    and the last chunk of a row is partial."""
    lens = [262144 - 37 * r for r in range(30)] + [0, 4097, 131072 + 3, 256 * 16 * 3]
    check(lens, 16, 16, 127, 0, 1, idx_dim, pkv.select_capacity(16, 16, 127, 0, 1), seed=13 + idx_dim)


def test_selection_feeds_sparse_decode():
    """GPU selection -> pkv_decode_attention in sparse mode == the oracle's
    decode over the same selected pages."""
    P, BT, k = 16, 16, 20
    w = synth.build_workload("sel_e2e", rows=3, hq=16, hkv=2, dim=128, page=P, seq_lens=[900, 1500, 333],
                             codec_of=lambda r, lp: (FP8, FP8), seed=21)
    rng = np.random.default_rng(5)
    max_blocks = w.max_pages
    q_idx = rng.standard_normal((3, 64)).astype(np.float16)
    slab = rng.standard_normal((3, max_blocks, 64)).astype(np.float16)
    cap = pkv.select_capacity(P, BT, k, 0, 1)
    sel, n, _, dropped = run_select([900, 1500, 333], P, BT, k, 0, 1, 64, cap, w.max_pages, q_idx, slab)
    assert dropped == 0
    ws = synth.Workload(**{**w.__dict__, "page_sel": np.ascontiguousarray(sel.astype(np.int32)),
                           "sel_lens": n.astype(np.int32)})
    dw = to_device(ws)
    p = params_for(ws)
    out, lse = pkv.decode_attention(p, *dw.args())
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.decode_attention(ws)
    compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
            "select -> sparse decode")
