"""Chunked-prefill attention and the window fold on the GPU vs the float64
oracle (oracle/prefill.py).

Tolerances as for decode: max-abs 1e-3 on out and 1e-4 on lse; queries with
an empty key set must give out = 0 and lse = -inf exactly. The kernel forms
the same fp16 MFMA operands and applies the scales in fp32 as the decode
kernel does, so the decode bar applies unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_182_amd as pkv
import synth
from synth.device import to_device
from synth.layout import BF16, BIT1, FP8, FP16, INT2, INT4, INT8
from gpu_util import compare, params_for, poison_tails, rewrite_bf16, run

pytestmark = pytest.mark.gpu

# Two GPU results over different splittings of the keys: P.V weights are
# rounded to fp16 relative to each split's own running max (relative error
# up to 2^-11 per weight), so their outputs may differ by a few fp16 ulps of
# the weighted values (|v| up to ~4 here, 2^-11 * 4 = 2e-3 at worst; random
# signs average most of it out); lse is summed in fp32 and moves by
# fp32 rounding only.
SPLIT_OUT_TOL = 5e-4
SPLIT_LSE_TOL = 2e-5

PAIRS = [(FP16, FP16), (BF16, BF16), (FP8, FP8), (INT8, INT4), (INT4, INT8), (FP8, FP16), (FP16, INT8),
         (INT2, INT2), (BIT1, BIT1), (INT2, BIT1), (BIT1, INT2), (FP8, INT2), (INT2, FP16)]


def small(seq_lens, kc, vc, hq, hkv, dim, page, seed=7, **kw):
    return synth.build_workload(f"pf_{kc}{vc}", rows=len(seq_lens), hq=hq, hkv=hkv, dim=dim, page=page,
                                seq_lens=seq_lens, codec_of=kw.pop("codec_of", lambda r, lp: (kc, vc)),
                                seed=seed, **kw)


def run_prefill(w, q, kv_begin=0, kv_end=-1, partition_tokens=0, dw=None, expect_err=0, window=0, **pk):
    dw = dw or to_device(w)
    p = params_for(w, partition_tokens, **pk)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    out, lse = pkv.prefill_attention(p, qd, dw.pool, dw.page_k_off, dw.page_v_off, dw.page_codec, dw.page_scale,
                                     dw.block_table, dw.seq_lens, kv_begin=kv_begin, kv_end=kv_end, window=window,
                                     err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == expect_err
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(w, T, kv_begin=0, kv_end=-1, partition_tokens=0, seed=3, what="", q_scale=1.0, window=0, **pk):
    q = synth.prefill_queries(seed, w.rows, T, w.num_q_heads, w.head_dim, q_scale)
    out, lse = run_prefill(w, q, kv_begin, kv_end, partition_tokens, window=window, **pk)
    ref_o, ref_l = oracle.prefill_attention(w, q, kv_begin, None if kv_end < 0 else kv_end, window=window)
    return compare(out, lse, ref_o, ref_l, what or f"{w.name} T={T} kv=[{kv_begin},{kv_end}) pt={partition_tokens}")


@pytest.mark.parametrize("kc,vc", PAIRS)
@pytest.mark.parametrize("dim", [64, 128])
def test_codec_pairs_ragged(kc, vc, dim):
    print(f"case codecs=({kc},{vc}) dim={dim}", flush=True)
    w = poison_tails(small([1, 15, 17, 300, 513], kc, vc, hq=8, hkv=2, dim=dim, page=32))
    check(w, 7, partition_tokens=64)
    check(w, 40, partition_tokens=0)


@pytest.mark.parametrize("T", [1, 2, 16, 33, 64])
def test_chunk_lengths(T):
    print(f"case T={T}", flush=True)
    w = poison_tails(small([70, 200, 1000], FP8, FP8, hq=16, hkv=2, dim=128, page=64))
    check(w, T, partition_tokens=128)
    check(w, T, partition_tokens=0)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 1), (14, 2), (32, 8), (16, 1)])
def test_group_sizes_and_column_groups(hq, hkv):
    """T*G from 5 to 640 columns: one or several groups of 128 columns."""
    print(f"case hq={hq} hkv={hkv}", flush=True)
    w = poison_tails(small([77, 250], INT8, INT4, hq=hq, hkv=hkv, dim=128, page=16))
    check(w, 40, partition_tokens=64)


@pytest.mark.parametrize("kv_begin,kv_end", [(0, 100), (5, 77), (64, 256), (100, 101), (130, -1), (600, -1),
                                             (50, 50), (17, 1000)])
def test_key_windows(kv_begin, kv_end):
    print(f"case window=[{kv_begin},{kv_end})", flush=True)
    w = poison_tails(small([150, 300, 260], FP16, INT8, hq=8, hkv=2, dim=64, page=32))
    check(w, 24, kv_begin, kv_end, partition_tokens=64)
    check(w, 24, kv_begin, kv_end, partition_tokens=0)


def test_chunk_longer_than_row_and_empty_rows():
    """T > L: the first T - L queries sit before the row (empty, out 0 and
    lse -inf); an empty row gives empty results throughout."""
    w = small([0, 5, 40], FP16, FP16, hq=4, hkv=2, dim=64, page=16)
    check(w, 12, partition_tokens=16)
    check(w, 12)


def test_mixed_codecs_per_page():
    pairs = [(FP16, FP16), (FP8, FP8), (INT8, INT4), (BF16, FP8), (INT4, INT8), (INT2, INT2), (BIT1, INT2),
             (INT2, BIT1)]
    rng = np.random.default_rng(4)
    pick = {}

    def codec_of(r, lp):
        if (r, lp) not in pick:
            pick[(r, lp)] = pairs[int(rng.integers(len(pairs)))]
        return pick[(r, lp)]

    w = poison_tails(small([400, 129, 64], 0, 0, hq=8, hkv=2, dim=128, page=16, codec_of=codec_of))
    check(w, 20, partition_tokens=64)
    check(w, 20, partition_tokens=0, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED)


@pytest.mark.parametrize("cuts", [[0, 128, 256, 1024], [0, 100, 101, 400, 1024], [0, 1024]])
def test_window_fold_on_device(cuts):
    """Windows attended one call each and folded by pkv_lse_fold_into equal
    one call over the whole range (and the oracle)."""
    w = small([700, 1000], FP8, INT8, hq=8, hkv=2, dim=128, page=64, seed=9)
    T = 48
    q = synth.prefill_queries(2, w.rows, T, w.num_q_heads, w.head_dim)
    dw = to_device(w)
    full_o, full_l = run_prefill(w, q, dw=dw)
    acc_o = torch.zeros((w.rows, T, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    acc_l = torch.full((w.rows, T, w.num_q_heads), float("-inf"), dtype=torch.float32, device="cuda")
    for i in range(len(cuts) - 1):
        o, l = run_prefill(w, q, cuts[i], cuts[i + 1], dw=dw)
        pkv.lse_fold_into(acc_o, acc_l, torch.from_numpy(o.astype(np.float32)).cuda(),
                          torch.from_numpy(l.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    ao, al = acc_o.cpu().numpy().astype(np.float64), acc_l.cpu().numpy().astype(np.float64)
    fin = np.isfinite(full_l)
    assert np.array_equal(np.isfinite(al), fin)
    eo, el = np.max(np.abs(ao - full_o)), np.max(np.abs(al[fin] - full_l[fin]))
    print(f"windowed vs one call: out {eo:.3e} lse {el:.3e}", flush=True)
    assert eo <= SPLIT_OUT_TOL and el <= SPLIT_LSE_TOL
    ref_o, ref_l = oracle.prefill_attention(w, q)
    compare(ao, al, ref_o, ref_l, "windowed fold")


def test_fold_into_matches_oracle():
    rng = np.random.default_rng(8)
    rows, D = 300, 128
    ao, bo = rng.standard_normal((rows, D)).astype(np.float32), rng.standard_normal((rows, D)).astype(np.float32)
    al, bl = (rng.standard_normal(rows) * 4).astype(np.float32), (rng.standard_normal(rows) * 4).astype(np.float32)
    al[:20] = -np.inf
    bl[10:30] = -np.inf                    # rows 10..19 empty on both sides
    bo[20:30] = np.nan                     # an empty side's values are never read into the result
    ref_o, ref_l = oracle.fold_into(ao, al, bo, bl)
    t = [torch.from_numpy(x.copy()).cuda() for x in (ao, al, bo, bl)]
    pkv.lse_fold_into(*t)
    torch.cuda.synchronize()
    go, gl = t[0].cpu().numpy().astype(np.float64), t[1].cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(gl), fin) and np.all(go[~fin] == 0)
    assert np.max(np.abs(go - ref_o)) <= 1e-5 and np.max(np.abs(gl[fin] - ref_l[fin])) <= 1e-5


def test_bad_pages_are_counted_and_skipped():
    w = small([96, 64], FP8, FP8, hq=8, hkv=2, dim=128, page=32)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_pages + 5             # page id out of range
    w2 = synth.Workload(**{**w.__dict__, "block_table": bt})
    T = 10
    q = synth.prefill_queries(1, w.rows, T, 8, 128)
    out, lse = run_prefill(w2, q, partition_tokens=32, expect_err=1)   # one page, one partition: one count
    ref_o, ref_l = oracle.prefill_attention(w, q)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    # row 1 is untouched by the bad entry
    compare(out[1:], lse[1:], ref_o[1:], ref_l[1:], "rows without a bad page")


def test_repeat_runs_bit_identical():
    w = small([1000, 333], INT8, INT4, hq=16, hkv=2, dim=128, page=16)
    q = synth.prefill_queries(5, w.rows, 37, 16, 128)
    dw = to_device(w)
    a = run_prefill(w, q, dw=dw)
    b = run_prefill(w, q, dw=dw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_partition_sizes_agree():
    w = small([3000], FP8, FP8, hq=16, hkv=2, dim=128, page=64)
    q = synth.prefill_queries(6, 1, 64, 16, 128, 3.6)
    dw = to_device(w)
    ref = run_prefill(w, q, dw=dw, partition_tokens=64)
    for pt in (128, 1024, 4096):
        o, l = run_prefill(w, q, dw=dw, partition_tokens=pt)
        eo, el = np.max(np.abs(o - ref[0])), np.max(np.abs(l - ref[1]))
        print(f"partition {pt} vs 64: out {eo:.3e} lse {el:.3e}", flush=True)
        assert eo <= SPLIT_OUT_TOL and el <= SPLIT_LSE_TOL
    ref_o, ref_l = oracle.prefill_attention(w, q)
    compare(ref[0], ref[1], ref_o, ref_l, "3000 tokens, 64 queries")


@pytest.mark.parametrize("window", [1, 7, 16, 100, 333, 4096])
def test_sliding_window(window):
    """Sliding-window attention (each query sees its last W positions); T = 1
    is sliding-window decode."""
    print(f"case window={window}", flush=True)
    w = poison_tails(small([1, 40, 300, 1000], FP8, INT8, hq=16, hkv=2, dim=128, page=16))
    check(w, 24, window=window, partition_tokens=64)
    check(w, 1, window=window, partition_tokens=0)
    check(w, 37, 100, 900, window=window, partition_tokens=0)


def test_sliding_window_mixed_codecs_and_groups():
    pairs = [(FP16, FP16), (FP8, FP8), (INT8, INT4), (BF16, FP8)]
    w = poison_tails(small([700, 129], 0, 0, hq=14, hkv=2, dim=64, page=32,
                           codec_of=lambda r, lp: pairs[(r + lp) % len(pairs)]))
    check(w, 50, window=64, partition_tokens=64, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED)


@pytest.mark.parametrize("kc,vc", [(FP8, FP8), (INT8, INT4)])
def test_partitions_over_256_pages(kc, vc):
    """partition_tokens = 8192 at 16-token pages: 512 pages per partition,
    staged into LDS in two rounds of 256 descriptors; rows end inside the
    first round, on its boundary and inside the second; a key window starting
    inside a partition's second round."""
    print(f"case prefill >256 pages per partition ({kc},{vc})", flush=True)
    w = poison_tails(small([9000, 4096, 12001], kc, vc, hq=8, hkv=2, dim=128, page=16, seed=13))
    check(w, 5, partition_tokens=8192)
    check(w, 33, 4200, -1, partition_tokens=8192)


@pytest.mark.parametrize("window", [1, 100, 4096])
def test_sliding_window_decode_equals_prefill_t1(window):
    """The decode path's sliding window and the prefill path's window at
    T = 1 are two kernels for the same result."""
    print(f"case decode vs prefill window={window}", flush=True)
    w = poison_tails(small([40, 300, 5000], FP8, INT8, hq=16, hkv=2, dim=128, page=16))
    q = synth.prefill_queries(4, w.rows, 1, w.num_q_heads, w.head_dim)
    po, pl = run_prefill(w, q, window=window)
    w.q = np.ascontiguousarray(q[:, 0])
    w.window_tokens = window
    p = params_for(w, 0)
    p.window_tokens = window
    out, lse = pkv.decode_attention(p, *to_device(w).args())
    torch.cuda.synchronize()
    do, dl = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(do - po[:, 0])) <= SPLIT_OUT_TOL and np.max(np.abs(dl - pl[:, 0])) <= SPLIT_LSE_TOL
    compare(do, dl, *oracle.decode_attention(w), f"decode window {window}")


def row_vmax(w):
    """Largest |V| of each row's pages (an upper bound of what any of its
    queries attends), per (row, query head)."""
    from oracle.attention import gather_kv
    G = w.num_q_heads // w.num_kv_heads
    m = np.zeros((w.rows, w.num_q_heads))
    for r in range(w.rows):
        for hk in range(w.num_kv_heads):
            _, v = gather_kv(w, r, hk)
            if v.size:
                m[r, hk * G:(hk + 1) * G] = np.max(np.abs(v))
    return m


def test_bf16_beyond_fp16_range():
    """BF16 codes go to the bf16 MFMA as they are: values past fp16's 65504
    and below its 2^-24 stay exact, and nothing is counted. Rows: N(0,1) with
    5% outliers x 1e5 (queries x 1e-4, scores of order one); K and V near
    1e-30; K near 1e6 against queries near 1e-6 (fp16 subnormals); values
    x 3e4. Bound on out: the weights keep 16 significant bits and every
    product is exact, so the error is below 2^-16 of the largest |V| a query
    attends plus fp32 rounding: 3e-5 x the row's largest |V|, and 1e-3
    absolute on top for rows of values near one. LSE: 1e-4 as everywhere.
    The BF16 kernel and the per-page kernel."""
    print("case prefill bf16 full range", flush=True)
    w = small([700, 333, 1024, 17], BF16, BF16, hq=8, hkv=2, dim=128, page=64, seed=21)
    rng = np.random.default_rng(8)

    def make(r, lp, is_v):
        x = rng.standard_normal((w.num_kv_heads, w.page_size, w.head_dim)).astype(np.float32)
        if r == 0:
            big = rng.random(x.shape) < 0.05
            return np.where(big, x * 1e5, x)
        if r == 1:
            return x * 1e-30
        if r == 2:
            return x * 1e6 if not is_v else x
        return x * 3e4
    rewrite_bf16(w, make)
    T = 8
    q = synth.prefill_queries(5, w.rows, T, w.num_q_heads, w.head_dim, 1.0).astype(np.float32)
    q = (q * np.array([1e-4, 1.0, 1e-6, 1e-4], dtype=np.float32)[:, None, None, None]).astype(np.float16)
    assert np.count_nonzero(q[2]) > q[2].size // 2
    ref_o, ref_l = oracle.prefill_attention(w, q)
    fin = np.isfinite(ref_l)
    tol = (3e-5 * row_vmax(w)[:, None, :, None] + np.where(np.arange(w.rows) == 1, 0.0, 1e-3)[:, None, None, None])
    dw = to_device(w)
    for pk in ({}, {"k_codec": pkv.CODEC_MIXED, "v_codec": pkv.CODEC_MIXED}):
        o, l = run_prefill(w, q, dw=dw, **pk)
        err = np.abs(o - ref_o)
        print(f"prefill bf16 range {pk}: out err / tol max {float(np.max(err / tol)):.3f}, "
              f"lse max-abs {float(np.max(np.abs(l[fin] - ref_l[fin]))):.3e}", flush=True)
        assert np.array_equal(np.isfinite(l), fin)
        assert np.all(np.isfinite(o)) and np.all(err <= tol), f"kernel {pk}"
        assert float(np.max(np.abs(l[fin] - ref_l[fin]))) <= 1e-4
        # row 1 (values near 1e-30) is not flushed: its outputs match to 1e-4 relative
        assert np.max(np.abs(o[1] - ref_o[1])) <= 1e-4 * np.max(np.abs(ref_o[1]))


def test_bf16_planes_beside_other_codecs():
    """The per-page kernel with BF16 on one plane only: K BF16 / V FP8 and
    K INT8 / V BF16 pages, values past fp16's range on the BF16 planes (a
    pair of tiles across two such pages splits its P.V between the bf16 and
    the fp16 MFMA)."""
    print("case prefill bf16 mixed pairs", flush=True)
    w = small([900, 400], 0, 0, hq=16, hkv=2, dim=128, page=16, seed=5,
              codec_of=lambda r, lp: (BF16, FP8) if (r + lp) % 2 else (INT8, BF16))
    rng = np.random.default_rng(9)
    rewrite_bf16(w, lambda r, lp, is_v: rng.standard_normal((2, 16, 128)).astype(np.float32) * (1e5 if is_v else 2e5))
    q = (synth.prefill_queries(6, w.rows, 12, w.num_q_heads, w.head_dim, 1.0).astype(np.float32) * 1e-5
         ).astype(np.float16)
    ref_o, ref_l = oracle.prefill_attention(w, q)
    fin = np.isfinite(ref_l)
    o, l = run_prefill(w, q, partition_tokens=128, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED)
    tol = 3e-5 * row_vmax(w)[:, None, :, None] + 1e-3
    assert np.array_equal(np.isfinite(l), fin)
    assert np.all(np.isfinite(o)) and np.all(np.abs(o - ref_o) <= tol)
    assert float(np.max(np.abs(l[fin] - ref_l[fin]))) <= 1e-4


@pytest.mark.parametrize("dim", [64, 128])
def test_tier_cascade_rows(dim):
    """A row whose pages sit in every tier of the cascade, newest FP16 to
    oldest 1-bit, under the per-page codec kernel at whole-page and
    library-chosen partitions."""
    print(f"case tier cascade dim={dim}", flush=True)
    tiers = [BIT1, INT2, INT4, INT8, FP8, FP16]          # logical page 0 is the oldest

    def codec_of(r, lp):
        c = tiers[min(lp * len(tiers) // 12, len(tiers) - 1)]
        return (c, c)
    w = poison_tails(small([12 * 64 - 5, 700, 64], 0, 0, hq=16, hkv=2, dim=dim, page=64, codec_of=codec_of,
                           seed=19, q_scale=2.0))
    for pt in (128, 0):
        check(w, 24, partition_tokens=pt, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED,
              what=f"tier cascade dim={dim} pt={pt}")


@pytest.mark.parametrize("codec", [INT2, BIT1])
@pytest.mark.parametrize("dim", [64, 128])
def test_subbyte_v_codes_exact(codec, dim):
    """One key per row and a zero query: each query's out is that key's V
    exactly. Every 2-bit code (INT2: offset + step * u) or both signs (BIT1),
    with fp16 steps and offsets whose sums are exact in fp32."""
    print(f"case sub-byte V codes {codec} dim={dim}", flush=True)
    from oracle.layout import code_bits
    rows = 4
    w = small([1] * rows, FP16, codec, hq=2, hkv=1, dim=dim, page=16, seed=5)
    arr = w.pool.as_array()
    bpos, shift = code_bits(16, dim, codec, True)
    rng = np.random.default_rng(9)
    G = dim // 32
    for r in range(rows):
        pp = int(w.block_table[r, 0])
        off = int(w.page_v_off[pp])
        head_bytes = 16 * dim * (2 if codec == INT2 else 1) // 8
        arr[off:off + head_bytes] = 0
        codes = rng.integers(0, 4 if codec == INT2 else 2, size=dim)
        np.bitwise_or.at(arr, off + bpos[0], (codes << shift[0]).astype(np.uint8))
        sc = off + head_bytes
        steps = np.float16(rng.choice([0.25, 0.5, 1.5, 3.0], size=G))
        arr[sc:sc + 2 * G] = np.frombuffer(steps.tobytes(), np.uint8)
        if codec == INT2:
            zo = sc + 16 * G * 2
            offs = np.float16(rng.choice([-2.0, -0.75, 0.125, 1.0], size=G))
            arr[zo:zo + 2 * G] = np.frombuffer(offs.tobytes(), np.uint8)
    q = np.zeros((rows, 1, w.num_q_heads, dim), dtype=np.float16)
    out, _ = run_prefill(w, q)
    ref, _ = oracle.prefill_attention(w, q)
    assert np.array_equal(out, ref.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("dim", [64, 128])
def test_int2_large_values(dim):
    """INT2 K and V pages of N(0, 16^2) values: a group's offset and step
    terms (about 40 and up to 80) far exceed the weighted values they sum to,
    so each must reach the MFMA with 22-bit weights (fp16 high and low parts)
    to stay within the 1e-3 bar; the per-page kernel and the declared pair."""
    print(f"case INT2 large values dim={dim}", flush=True)
    w = poison_tails(small([300, 513, 64], INT2, INT2, hq=8, hkv=2, dim=dim, page=32, seed=23,
                           outlier_frac=1.0, outlier_mult=16.0))
    check(w, 24, partition_tokens=64)
    check(w, 24, partition_tokens=0, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED)


@pytest.mark.parametrize("dim", [64, 128])
def test_fp8_v_scales_sign_zero_and_tiny(dim):
    """FP8 V page scales enter the softmax in the log domain: 16-token pages
    (every pair of tiles spans two pages) with scales of both signs, a zero
    scale (its codes decode to zero whatever they hold) and one of 2^-50
    (taken as 2^-40: its values move by less than 4.1e-10), through the
    prefill and, the same pages, the decode kernel, against the oracle."""
    print(f"case fp8 v scales dim={dim}", flush=True)
    w = small([700, 64, 1500, 33], FP8, FP8, hq=16, hkv=2, dim=dim, page=16)
    rng = np.random.default_rng(dim)
    sc = w.page_scale.copy()
    sc[:, :, 1] *= rng.choice([-1.0, 1.0], size=sc.shape[:2]) * rng.uniform(0.5, 2.0, size=sc.shape[:2])
    sc[w.block_table[0, 3], :, 1] = 0.0
    sc[w.block_table[2, 10], :, 1] = 2.0 ** -50
    w.page_scale[...] = sc.astype(w.page_scale.dtype)
    check(w, 24, partition_tokens=0, q_scale=2.0)
    check(w, 5, partition_tokens=64)
    # the same pages declared per page: the per-page (any codec) kernels
    mixed = dict(k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED)
    check(w, 24, partition_tokens=0, q_scale=2.0, **mixed)
    for pk in ({}, mixed):
        out, lse = run(to_device(w), params_for(w, 0, **pk))
        compare(out, lse, *oracle.decode_attention(w), f"decode {w.name} {pk}")
