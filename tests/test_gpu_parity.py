"""HIP path vs the float64 oracle on small and ragged workloads (GPU).

Tolerances: max-abs 1e-3 on out and 1e-4 on lse, the bar set for the
workloads; empty rows must give out = 0 and lse = -inf exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_182_amd as pkv
import synth
from synth.device import to_device
from synth.layout import BF16, BIT1, FP8, FP16, INT2, INT4, INT8
from gpu_util import rewrite_bf16, compare, params_for, poison_tails, run

pytestmark = pytest.mark.gpu

PAIRS = [(FP16, FP16), (BF16, BF16), (FP8, FP8), (INT8, INT4), (INT8, INT8), (INT4, INT4),
         (FP8, FP16), (INT4, FP8), (FP16, INT8),
         (INT2, INT2), (BIT1, BIT1), (INT8, INT2), (INT2, BIT1), (BIT1, FP16)]


def small(seq_lens, kc, vc, hq, hkv, dim, page, seed=7, **kw):
    return synth.build_workload(f"gpu_{kc}{vc}", rows=len(seq_lens), hq=hq, hkv=hkv, dim=dim,
                                page=page, seq_lens=seq_lens,
                                codec_of=kw.pop("codec_of", lambda r, lp: (kc, vc)), seed=seed, **kw)


def check(w, partition_tokens=None, what="", **pk):
    dw = to_device(w)
    out, lse = run(dw, params_for(w, partition_tokens, **pk))
    ref_out, ref_lse = oracle.decode_attention(w)
    return compare(out, lse, ref_out, ref_lse, what or w.name)


@pytest.mark.parametrize("kc,vc", PAIRS)
@pytest.mark.parametrize("dim", [64, 128])
def test_codec_pairs_ragged(kc, vc, dim):
    print(f"case codecs=({kc},{vc}) dim={dim}", flush=True)
    w = poison_tails(small([1, 15, 17, 300, 513], kc, vc, hq=8, hkv=2, dim=dim, page=32))
    check(w, partition_tokens=64)
    check(w, partition_tokens=0)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 1), (14, 2), (16, 2), (32, 8), (16, 1)])
def test_group_sizes(hq, hkv):
    print(f"case hq={hq} hkv={hkv}", flush=True)
    w = poison_tails(small([77, 250], FP8, FP8, hq=hq, hkv=hkv, dim=128, page=16))
    check(w, partition_tokens=64)


@pytest.mark.parametrize("dim", [64, 128])
def test_mixed_codecs_per_page(dim):
    print(f"case mixed dim={dim}", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8), (INT8, INT4), (BF16, INT8), (INT4, FP16), (BF16, BF16), (FP16, INT4),
           (INT2, INT2), (BIT1, BIT1), (INT2, FP8), (BIT1, INT2)]
    w = poison_tails(small([40, 333, 160], None, None, hq=8, hkv=2, dim=dim, page=16,
                           codec_of=lambda r, lp: cyc[(r + lp) % len(cyc)]))
    check(w, partition_tokens=32)
    check(w, partition_tokens=0)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_configs_small(cid):
    print(f"case config {cid} small", flush=True)
    w = synth.config(cid, small=cid != 1)
    if not w.sparse:
        poison_tails(w)
    check(w)


def test_partition_invariance_and_determinism():
    """Every partition size matches the oracle; sizes agree with each other to
    1e-4 (each partition has its own running max, so the fp16 softmax weights
    round differently: per token a relative 2^-11, about |v| * 2^-11 * sqrt(sum
    w^2) on out, a few 1e-5 here); a repeated launch is bit-identical."""
    print("case partition invariance", flush=True)
    w = small([2000, 1111], FP8, FP8, hq=16, hkv=2, dim=128, page=16, q_scale=3.0)
    dw = to_device(w)
    ref = oracle.decode_attention(w)
    res = []
    for T in (16, 64, 512, 2048):
        o, l = run(dw, params_for(w, T))
        compare(o, l, *ref, f"partition_tokens={T}")
        res.append((o, l))
    for o, l in res[1:]:
        assert np.max(np.abs(o - res[0][0])) <= 1e-4 and np.max(np.abs(l - res[0][1])) <= 1e-5
    o2, l2 = run(dw, params_for(w, 64))
    assert np.array_equal(o2, res[1][0]) and np.array_equal(l2, res[1][1])


def test_empty_rows_and_partitions():
    print("case empty", flush=True)
    w = small([0, 5, 0, 1000], INT8, INT4, hq=8, hkv=2, dim=128, page=16)
    check(w, partition_tokens=16)
    ws = synth.config(4, small=True)
    ws.sel_lens[0] = 0
    ws.sel_lens[2] = 3
    check(ws)


def test_many_short_rows():
    """1,500 rows of 0 to 200 tokens (a decode batch of short sequences): rows x
    KV heads far above one round of resident workgroups, so the library picks
    one partition per row and writes out/lse directly; and 64-token
    partitions, folded."""
    print("case many short rows", flush=True)
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 201, 1500).tolist()
    lens[:3] = [0, 1, 200]
    w = small(lens, FP8, FP8, hq=8, hkv=2, dim=64, page=16)
    assert pkv.num_partitions(params_for(w, 0)) == 1
    check(w, partition_tokens=0)
    check(w, partition_tokens=64)


# ------------------------------------------------ partitions finer than a page, even splits
@pytest.mark.parametrize("kc,vc,page", [(FP8, FP8, 64), (INT8, INT4, 64), (FP16, FP16, 1024), (None, None, 1024)])
def test_sub_page_partitions(kc, vc, page):
    """Partitions of any multiple of 16 tokens, also inside one page, and the
    library's even split (partition_tokens = 0) match the oracle."""
    print(f"case sub-page partitions ({kc},{vc}) page={page}", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8)]
    codec_of = (lambda r, lp: cyc[(r + lp) % 2]) if kc is None else (lambda r, lp: (kc, vc))
    w = poison_tails(small([1, 40, 1500, 2100, 3000], kc, vc, hq=16, hkv=2, dim=128 if page == 64 else 64,
                           page=page, codec_of=codec_of))
    for T in (16, 48, 80, 0):
        check(w, partition_tokens=T, what=f"{w.name} page={page} T={T}")


@pytest.mark.parametrize("kc,vc", [(FP8, FP8), (INT8, INT4), (None, None)])
def test_page_size_not_power_of_two(kc, vc):
    """48-token pages (three tiles): the tile's page comes from a division
    instead of a shift; fixed, sub-page and even-split partitions."""
    print(f"case page 48 ({kc},{vc})", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8), (INT8, INT4)]
    codec_of = (lambda r, lp: cyc[(r + lp) % 3]) if kc is None else (lambda r, lp: (kc, vc))
    w = poison_tails(small([47, 48, 49, 700, 1201], kc, vc, hq=8, hkv=2, dim=128, page=48, codec_of=codec_of))
    for T in (48, 32, 144, 0):
        check(w, partition_tokens=T, what=f"{w.name} page=48 T={T}")


@pytest.mark.parametrize("dim", [64, 128])
def test_float_class_pages(dim):
    """PKV_CODEC_MIXED_FLOAT: every page FP16, BF16 or FP8 for both planes,
    chosen per page (the smaller per-page kernel), any partition size."""
    print(f"case float class dim={dim}", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8), (BF16, BF16)]
    w = poison_tails(small([5, 300, 1000, 2047], None, None, hq=16, hkv=2, dim=dim, page=64,
                           codec_of=lambda r, lp: cyc[(r + 2 * lp) % 3]))
    assert params_for(w).k_codec == pkv.CODEC_MIXED_FLOAT
    for T in (0, 48, 256):
        check(w, partition_tokens=T, what=f"float class dim={dim} T={T}")


def test_float_class_rejects_other_pages():
    """Under the float declaration an INT page and a page with different K and
    V codecs are device-visible errors: counted and skipped."""
    print("case float class errors", flush=True)
    codes = {(0, 0): (FP16, FP16), (0, 1): (INT8, INT4), (0, 2): (FP8, FP8),
             (1, 0): (FP8, FP16), (1, 1): (FP8, FP8), (1, 2): (BF16, BF16)}
    w = small([48, 48], None, None, hq=8, hkv=2, dim=128, page=16, codec_of=lambda r, lp: codes[(r, lp)])
    dw = to_device(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = run(dw, params_for(w, 16, k_codec=pkv.CODEC_MIXED_FLOAT, v_codec=pkv.CODEC_MIXED_FLOAT), err=err)
    assert int(err.item()) == 2
    w.page_sel, w.sel_lens = np.array([[0, 2], [1, 2]], dtype=np.int32), np.array([2, 2], dtype=np.int32)
    compare(out, lse, *oracle.decode_attention(w), "float class skips other pages")


def test_sparse_sub_page_partitions():
    """Sparse mode: a partition's tiles run through the selected pages in list
    order, so partitions finer than a page split selected pages."""
    print("case sparse sub-page partitions", flush=True)
    rng = np.random.default_rng(5)
    lens = [1000, 777, 64]
    sel = []
    for L in lens:
        last = -(-L // 64) - 1
        rest = rng.choice([x for x in range(16) if x != last], 5, replace=False)
        sel.append(rng.permutation(np.concatenate([[last], rest])))
    sel = np.array(sel, dtype=np.int32)
    w = synth.build_workload("gpu_sparse64", rows=3, hq=8, hkv=2, dim=128, page=64, seq_lens=lens,
                             codec_of=lambda r, lp: (FP8, FP8), seed=11, selection=sel)
    w.sel_lens = np.array([6, 4, 6], dtype=np.int32)
    for T in (16, 32, 96, 0):
        check(w, partition_tokens=T, what=f"sparse page=64 T={T}")


def test_bad_page_counted_per_partition():
    """A bad page is counted once by every partition whose tiles reach it."""
    print("case bad page per partition", flush=True)
    w = small([128, 128], FP8, FP8, hq=8, hkv=2, dim=128, page=64)
    dw = to_device(w)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_pages + 5
    dw.block_table = torch.from_numpy(bt).cuda()
    results = []
    for T, expect in ((64, 1), (32, 2), (16, 4)):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out, lse = run(dw, params_for(w, T, k_codec=FP8, v_codec=FP8), err=err)
        assert int(err.item()) == expect, (T, int(err.item()))
        results.append((T, out, lse))
    # expected: row 0 without its bad page (sparse oracle over the good pages)
    w.page_sel, w.sel_lens = np.array([[0, 0], [0, 1]], dtype=np.int32), np.array([1, 2], dtype=np.int32)
    ref = oracle.decode_attention(w)
    for T, out, lse in results:
        compare(out, lse, *ref, f"bad page skipped T={T}")


def test_sparse_selection_order_and_unselected_poison():
    print("case sparse order", flush=True)
    w = synth.config(4, small=True)
    dw = to_device(w)
    p = params_for(w)
    o1, l1 = run(dw, p)
    rng = np.random.default_rng(1)
    for r in range(w.rows):
        w.page_sel[r] = rng.permutation(w.page_sel[r])
    dw2 = to_device(w)
    o2, l2 = run(dw2, p)
    ref = oracle.decode_attention(w)
    compare(o2, l2, *ref, "shuffled selection")
    assert np.max(np.abs(o1 - o2)) <= 1e-5 and np.max(np.abs(l1 - l2)) <= 1e-5


def test_device_errors_counted_and_skipped():
    print("case device errors", flush=True)
    w = small([64, 64, 64], FP8, FP8, hq=8, hkv=2, dim=128, page=16)
    dw = to_device(w)
    bt = w.block_table.copy()
    bt[0, 1] = w.num_pages + 5          # out-of-range physical page
    bt[1, 2] = -3
    dw.block_table = torch.from_numpy(bt).cuda()
    codec = w.page_codec.copy()
    codec[int(w.block_table[2, 0])] = 0x99   # unknown codec nibbles
    dw.page_codec = torch.from_numpy(codec).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = run(dw, params_for(w, 16, k_codec=FP8, v_codec=FP8), err=err)
    assert int(err.item()) == 3
    # expected: each row without its bad page (sparse oracle over the good pages)
    sel = np.array([[0, 2, 3], [0, 1, 3], [1, 2, 3]], dtype=np.int32)
    w.page_sel, w.sel_lens = sel, np.full(3, 3, dtype=np.int32)
    ref = oracle.decode_attention(w)
    compare(out, lse, *ref, "bad pages skipped")


def test_declared_codec_mismatch_is_counted():
    print("case codec mismatch", flush=True)
    w = small([48], INT8, INT4, hq=4, hkv=1, dim=64, page=16)
    dw = to_device(w)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, lse = run(dw, params_for(w, 16, k_codec=FP8, v_codec=FP8), err=err)
    assert int(err.item()) == 3 and np.all(out == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------- every code, exactly (V path)
def one_token_v_codes(codec, codes_for_row):
    """Workload with one token per row whose V values are given codes; q = 0
    makes out = V of that token exactly."""
    rows = len(codes_for_row)
    w = small([1] * rows, FP16, codec, hq=2, hkv=1, dim=128, page=16)
    from oracle.layout import BITS, code_position
    arr = w.pool.as_array()
    idx = code_position(16, 128, codec, True)[0][0]   # token 0, dims 0..127
    for r, codes in enumerate(codes_for_row):
        pp = int(w.block_table[r, 0])
        off = int(w.page_v_off[pp])
        if BITS[codec] == 16:
            b = np.asarray(codes, dtype="<u2").view(np.uint8).reshape(-1, 2)
            arr[off + idx] = b[:, 0]                      # byte offsets, little-endian
            arr[off + idx + 1] = b[:, 1]
        elif BITS[codec] == 8:
            arr[off + idx] = np.asarray(codes, dtype=np.uint8)
        else:
            raise AssertionError
        if codec == INT8:
            sc = off + 16 * 128
            arr[sc:sc + 8] = np.frombuffer(np.float16([1, 1, 1, 1]).tobytes(), np.uint8)
    w.page_scale[:] = 1.0
    w.q[:] = 0
    return w


@pytest.mark.parametrize("codec", [FP8, INT8])
def test_every_byte_code_exact(codec):
    print(f"case all codes {codec}", flush=True)
    codes = np.arange(256)
    if codec == FP8:
        codes = codes[(codes & 0x7F) != 0x7F]     # drop the two NaN codes
    codes = np.resize(codes, 256).reshape(2, 128)
    w = one_token_v_codes(codec, list(codes))
    out, _ = run(to_device(w), params_for(w, 0))
    ref, _ = oracle.decode_attention(w)
    assert np.array_equal(out, ref.astype(np.float32).astype(np.float64))


def test_fp16_codes_exact():
    print("case fp16 codes", flush=True)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 1 << 16, size=(8, 128)).astype(np.uint16)
    codes[(codes & 0x7C00) == 0x7C00] = 0x3C00       # no inf/NaN
    w = one_token_v_codes(FP16, list(codes))
    out, _ = run(to_device(w), params_for(w, 0))
    ref, _ = oracle.decode_attention(w)
    assert np.array_equal(out, ref.astype(np.float32).astype(np.float64))


# ------------------------------------------------ partials and the fold alone
def test_decode_partials_match_oracle_partials():
    print("case partials", flush=True)
    w = small([300, 17, 0, 129], FP8, INT8, hq=8, hkv=2, dim=128, page=16)
    T = 64
    check_partials(w, T, lambda L, n: [min(L, i * T) for i in range(n + 1)])


def test_even_split_partials_bounds():
    """partition_tokens = 0: partition i of a row of n_t = ceil(L / 16) tiles
    covers tiles [i c, (i + 1) c), c = max(1, ceil(n_t / n))."""
    print("case even-split partials", flush=True)
    w = small([300, 17, 0, 2000], FP8, FP8, hq=8, hkv=2, dim=128, page=64)

    def bounds(L, n):
        c = max(1, -(-(-(-L // 16)) // n))
        return [min(L, 16 * c * i) for i in range(n + 1)]
    n = check_partials(w, 0, bounds)
    assert n == 16          # 128 tiles at most per row, at least 8 per partition


def check_partials(w, T, bounds_of):
    """pkv_decode_partials against the oracle's partials over the token ranges
    bounds_of(L, n) of each row."""
    dw = to_device(w)
    p = params_for(w, T)
    n = pkv.num_partitions(p)
    acc, ml = pkv.decode_partials(p, *dw.args())
    torch.cuda.synchronize()
    acc, ml = acc.cpu().numpy().astype(np.float64), ml.cpu().numpy().astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    from oracle.attention import gather_kv
    for r in range(w.rows):
        L = int(w.seq_lens[r])
        bounds = bounds_of(L, n)
        for h in range(w.num_kv_heads):
            K, V = gather_kv(w, r, h)
            q = w.q[r, h * G:(h + 1) * G].astype(np.float64)
            oa, om, ol = oracle.partials(K, V, q, w.softmax_scale, bounds)
            ga, gm, gl = acc[r, h * G:(h + 1) * G], ml[r, h * G:(h + 1) * G, :, 0], ml[r, h * G:(h + 1) * G, :, 1]
            empty = ol == 0
            assert np.array_equal(gl == 0, empty) and np.all(np.isneginf(gm[empty]))
            ok = ~empty
            assert np.max(np.abs(gm[ok] - om[ok]), initial=0) <= 1e-5
            # acc/l is the partition's own normalised output
            assert np.max(np.abs(ga[ok] / gl[ok][:, None] - oa[ok] / ol[ok][:, None]), initial=0) <= 1e-3
            assert np.max(np.abs(np.log(gl[ok]) - np.log(ol[ok])), initial=0) <= 1e-4
    return n


@pytest.mark.parametrize("rows,parts,dim,shift", [
    (5, 1, 128, 0), (16, 512, 128, 0), (7, 33, 64, 0), (3, 9, 30, 0), (2, 4, 512, 0),
    (3, 130, 30, 0),      # many parts, head_dim not a multiple of 4
    (4, 200, 128, 1),     # part_acc only 4-byte aligned (one float into its buffer)
    (2, 1000, 64, 3),
    # the wide fold (head_dim a multiple of 32, up to 512 parts): each part
    # count per thread, part counts just past a slice boundary, head_dim 96
    (16, 65, 128, 0), (3, 256, 64, 0), (5, 257, 96, 0), (14, 128, 64, 0), (2, 12, 32, 0),
    (6, 300, 128, -1),    # part_ml only 4-byte aligned (part_acc aligned): the per-4-dims fold
    # the per-(row, dim) fold: every part in one batch (maximum first), (m, l)
    # as pairs and as single floats; more parts than a batch (running
    # log-sum-exp); 17-64 parts with head_dim a multiple of 32 (wide fold)
    (130, 12, 128, 0), (130, 12, 128, -1), (600, 20, 30, 0), (600, 40, 30, 0), (336, 21, 64, 0),
])
def test_lse_combine_matches_oracle_fold(rows, parts, dim, shift):
    print(f"case fold {rows} {parts} {dim} shift {shift}", flush=True)
    ml_shift = 1 if shift < 0 else 0
    shift = max(shift, 0)
    rng = np.random.default_rng(rows * 1000 + parts)
    m = (3 * rng.standard_normal((rows, parts))).astype(np.float32)
    l = rng.uniform(0.5, 50, (rows, parts)).astype(np.float32)
    acc = (rng.standard_normal((rows, parts, dim)) * l[..., None]).astype(np.float32)
    empty = rng.random((rows, parts)) < 0.2
    m[empty], l[empty], acc[empty] = -np.inf, 0, 0
    # parts marked empty by one field only, with junk in the others: never read
    half = rng.random((rows, parts)) < 0.1
    m[half & ~empty], acc[half & ~empty] = -np.inf, 1e30
    zero_l = (rng.random((rows, parts)) < 0.1) & ~empty & ~half
    l[zero_l], m[zero_l], acc[zero_l] = 0, 80.0, -1e30
    if rows > 2:
        m[1], l[1], acc[1] = -np.inf, 0, 0                  # a row with no tokens at all
    ml = np.stack([m, l], axis=-1)
    buf = torch.zeros(acc.size + shift, dtype=torch.float32, device="cuda")
    acc_t = buf[shift:].view(rows, parts, dim)
    acc_t.copy_(torch.from_numpy(acc))
    ml_buf = torch.zeros(ml.size + ml_shift, dtype=torch.float32, device="cuda")
    ml_t = ml_buf[ml_shift:].view(rows, parts, 2)
    ml_t.copy_(torch.from_numpy(ml))
    out, lse = pkv.lse_combine(acc_t, ml_t)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.fold(acc.astype(np.float64), m.astype(np.float64), l.astype(np.float64))
    out, lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(out - ref_out)) <= 1e-5 and np.max(np.abs(lse[fin] - ref_lse[fin]), initial=0) <= 1e-5


# ------------------------------------------- partitions of more than 256 pages
# The kernel stages a partition's page descriptors in LDS 256 at a time; a
# partition that reaches more pages takes a second (third, ...) staging round.
@pytest.mark.parametrize("kc,vc", [(FP8, FP8), (INT8, INT4), (None, None)])
def test_partitions_over_256_pages(kc, vc):
    """partition_tokens = 8192 at 16-token pages: 512 pages per partition, so
    every full partition stages its descriptors in two rounds; rows end inside
    the first round, on its boundary, inside the second and past one
    partition. The even split (partition_tokens = 0) is checked as well."""
    print(f"case >256 pages per partition ({kc},{vc})", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8), (INT8, INT4), (BF16, INT8)]
    codec_of = (lambda r, lp: cyc[(r + lp) % 4]) if kc is None else (lambda r, lp: (kc, vc))
    w = poison_tails(small([9000, 4096, 4097, 8192, 12001, 300], kc, vc, hq=8, hkv=2, dim=128, page=16,
                           codec_of=codec_of, seed=21))
    p = params_for(w, 8192)
    assert pkv.num_partitions(p) == 2
    check(w, partition_tokens=8192, what=f"{w.name} T=8192")
    check(w, partition_tokens=0, what=f"{w.name} T=0")


def test_library_single_partition_over_256_pages():
    """partition_tokens = 0 with more (row, KV head) units than one round of
    resident workgroups: the library gives each row one partition, here of
    258-275 pages (two staging rounds), and writes out/lse directly."""
    print("case library-chosen single partition > 256 pages", flush=True)
    lens = np.random.default_rng(3).integers(4113, 4400, size=97)
    w = poison_tails(small(lens, INT8, INT4, hq=32, hkv=8, dim=128, page=16, seed=23))
    p = params_for(w, 0)
    assert pkv.num_partitions(p) == 1 and pkv.workspace_bytes(p) == 0
    check(w, partition_tokens=0, what="97 rows x 8 KV heads, one partition each")


def test_sparse_selection_over_256_pages():
    """Sparse mode with 300-400 selected pages in one partition (their
    descriptors staged in two rounds), in shuffled order, with the last page
    partial."""
    print("case sparse > 256 selected pages", flush=True)
    rng = np.random.default_rng(29)
    lens = [16384 - 5, 16000, 9999]
    nsel = [400, 300, 330]
    sel = np.zeros((3, 400), dtype=np.int32)
    for r, L in enumerate(lens):
        # 400 distinct pages per row (all generated); the first nsel[r],
        # the last page among them, are attended
        last = -(-L // 16) - 1
        rest = rng.choice(last, 399, replace=False)
        sel[r, :nsel[r]] = rng.permutation(np.concatenate([[last], rest[:nsel[r] - 1]]))
        sel[r, nsel[r]:] = rest[nsel[r] - 1:]
    w = synth.build_workload("gpu_sparse400", rows=3, hq=16, hkv=2, dim=128, page=16, seq_lens=lens,
                             codec_of=lambda r, lp: (FP8, FP8), seed=31, selection=sel,
                             logical_pages=1024)
    w.sel_lens = np.array(nsel, dtype=np.int32)
    assert pkv.num_partitions(params_for(w, 8192)) == 1
    check(w, partition_tokens=8192, what="sparse 300-400 pages, one partition")
    check(w, partition_tokens=4096, what="sparse 300-400 pages, 256-page partitions")
    check(w, partition_tokens=0, what="sparse 300-400 pages, even split")



@pytest.mark.parametrize("dim", [64, 128])
def test_tier_cascade_rows(dim):
    """A row whose pages sit in every tier of the cascade, newest FP16 to
    oldest 1-bit (FP16, FP8, INT8, INT4, INT2, 1-bit), read by the per-page
    kernel at fixed, sub-page and even-split partitions."""
    print(f"case tier cascade dim={dim}", flush=True)
    tiers = [BIT1, INT2, INT4, INT8, FP8, FP16]          # logical page 0 is the oldest

    def codec_of(r, lp):
        c = tiers[min(lp * len(tiers) // 12, len(tiers) - 1)]
        return (c, c)
    w = poison_tails(small([12 * 64 - 5, 700, 64], None, None, hq=16, hkv=2, dim=dim, page=64, codec_of=codec_of,
                           seed=19, q_scale=2.0))
    for T in (0, 48, 256):
        check(w, partition_tokens=T, what=f"tier cascade dim={dim} T={T}")


@pytest.mark.parametrize("codec", [INT2, BIT1])
@pytest.mark.parametrize("dim", [64, 128])
def test_subbyte_v_codes_exact(codec, dim):
    """q = 0 and one token per row: out is that token's V exactly. Every
    2-bit code (INT2: offset + step * u) or both signs (BIT1), with fp16
    steps and offsets whose sums are exact in fp32."""
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
    w.q[:] = 0
    out, _ = run(to_device(w), params_for(w, 0))
    ref, _ = oracle.decode_attention(w)
    assert np.array_equal(out, ref.astype(np.float32).astype(np.float64))


# ------------------------------------------------------- sliding-window decode
@pytest.mark.parametrize("kc,vc", [(FP8, FP8), (INT8, INT4), (None, None), (INT2, BIT1)])
def test_sliding_window_decode(kc, vc):
    """pkv_decode_attention with a sliding window: each row attends its last
    W positions; the partitions cover only the window's tiles (fixed,
    sub-page and even-split partitions), the window's first page and tile
    are masked below its start, and rows shorter than W attend everything."""
    print(f"case sliding-window decode ({kc},{vc})", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8), (INT8, INT4), (BF16, INT8), (INT2, INT2)]
    codec_of = (lambda r, lp: cyc[(r + lp) % len(cyc)]) if kc is None else (lambda r, lp: (kc, vc))
    w = poison_tails(small([1, 40, 300, 1000, 4097], kc, vc, hq=16, hkv=2, dim=128, page=32, codec_of=codec_of,
                           seed=37, q_scale=2.0))
    for W in (1, 15, 16, 17, 100, 333, 1000, 5000):
        w.window_tokens = W
        ref = oracle.decode_attention(w)
        for T in (0, 64, 16):
            p = params_for(w, T)
            p.window_tokens = W
            out, lse = run(to_device(w), p)
            compare(out, lse, *ref, f"window {W} T={T}")


def test_sliding_window_decode_sparse_and_partials():
    """A window in sparse mode masks the selected pages' tokens before it
    (pages wholly before it are skipped, not counted as errors); the
    partials of a windowed dense call fold to the windowed result."""
    print("case sliding-window sparse + partials", flush=True)
    w = synth.config(4, small=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for W in (16, 700, 2000):
        w.window_tokens = W
        p = params_for(w)
        p.window_tokens = W
        out, lse = run(to_device(w), p, err=err)
        compare(out, lse, *oracle.decode_attention(w), f"sparse window {W}")
    assert int(err.item()) == 0
    wd = small([3000, 900], FP8, FP8, hq=16, hkv=2, dim=128, page=64, seed=3)
    wd.window_tokens = 1000
    p = params_for(wd, 256)
    p.window_tokens = 1000
    assert pkv.num_partitions(p) == 4                      # ceil(1000 / 16) + 1 = 64 tiles in 16-tile partitions
    dw = to_device(wd)
    acc, ml = pkv.decode_partials(p, *dw.args())
    out, lse = pkv.lse_combine(acc.view(-1, 4, 128), ml.view(-1, 4, 2))
    torch.cuda.synchronize()
    compare(out.view(2, 16, 128).cpu().numpy().astype(np.float64), lse.view(2, 16).cpu().numpy().astype(np.float64),
            *oracle.decode_attention(wd), "windowed partials folded")


# ------------------------------------------------ BF16 over its whole range
def vmax_per_row(w):
    """Largest |V| each (row, query head) attends, from the decoded pages."""
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
    and below its 2^-24 stay exact. Rows: N(0,1) with 5% outliers x 1e5 (q x
    1e-4, scores of order one); K and V near 1e-30; K near 1e6 against q
    near 1e-6 (fp16 subnormals; scores again of order one). Bound on out: the weights keep 16
    significant bits (2^-16 relative) and every product is exact, so the
    error is below 2^-16 of the largest |V| a row attends plus fp32 rounding:
    3e-5 x that maximum, and 1e-3 absolute on top for rows of values near
    one. LSE: scores of order one, 1e-4 as everywhere. Each page class runs:
    the BF16 kernel, the float per-page kernel and the any-codec kernel."""
    print("case bf16 full range", flush=True)
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
    qs = np.array([1e-4, 1.0, 1e-6, 1e-4], dtype=np.float32)
    w.q = (w.q.astype(np.float32) * qs[:, None, None]).astype(np.float16)
    assert np.all(np.isfinite(w.q.astype(np.float32))) and np.count_nonzero(w.q[2]) > w.q[2].size // 2
    ref_out, ref_lse = oracle.decode_attention(w)
    assert np.all(np.isfinite(ref_out)) and np.all(np.isfinite(ref_lse))
    tol = 3e-5 * vmax_per_row(w)[:, :, None] + np.where(np.arange(w.rows) == 1, 0.0, 1e-3)[:, None, None]
    dw = to_device(w)
    for kc in (BF16, pkv.CODEC_MIXED_FLOAT, pkv.CODEC_MIXED):
        o, l = run(dw, params_for(w, 256, k_codec=kc, v_codec=kc))
        err = np.abs(o - ref_out)
        print(f"bf16 range kernel {kc}: out err / tol max {float(np.max(err / tol)):.3f}, "
              f"lse max-abs {float(np.max(np.abs(l - ref_lse))):.3e}", flush=True)
        assert np.all(np.isfinite(o)) and np.all(err <= tol), f"kernel {kc}"
        assert float(np.max(np.abs(l - ref_lse))) <= 1e-4
        # row 1 (values near 1e-30) is not flushed: its outputs match to 1e-4 relative
        assert np.max(np.abs(o[1] - ref_out[1])) <= 1e-4 * np.max(np.abs(ref_out[1]))


def test_bf16_planes_beside_other_codecs():
    """The any-codec kernel with BF16 on one plane only: K BF16 / V FP8 and
    K INT8 / V BF16 pages, values past fp16's range on the BF16 planes."""
    print("case bf16 mixed pairs", flush=True)
    w = small([900, 400], None, None, hq=16, hkv=2, dim=128, page=16, seed=5,
              codec_of=lambda r, lp: (BF16, FP8) if (r + lp) % 2 else (INT8, BF16))
    rng = np.random.default_rng(9)
    rewrite_bf16(w, lambda r, lp, is_v: rng.standard_normal((2, 16, 128)).astype(np.float32) * (1e5 if is_v else 2e5))
    w.q = (w.q.astype(np.float32) * 1e-5).astype(np.float16)
    ref_out, ref_lse = oracle.decode_attention(w)
    o, l = run(to_device(w), params_for(w, 128))
    tol = 3e-5 * vmax_per_row(w)[:, :, None] + 1e-3
    assert np.all(np.isfinite(o)) and np.all(np.abs(o - ref_out) <= tol)
    assert float(np.max(np.abs(l - ref_lse))) <= 1e-4
