"""Pins for the oracle's attention and fold (no GPU).

The pages print no attention output for any input, so the oracle is pinned by
what they state and by mathematics: FP16 pages equal exact SDPA (ARGUS "Why
decode is slow": the streaming path is covered against SDPA including GQA),
page-streamed online softmax equals full softmax ("Direct paged attention"),
GQA equals replicated-head MHA, log-sum-exp folding is invariant to how the
tokens are split (FreeToken PR #499 discussion: windows folded by
log-sum-exp), results do not depend on physical placement (PR #499 "Design":
block-table translation), plus brute force and closed forms on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import synth
from oracle import decode_attention, fold, gather_kv, partials
from oracle.layout import plane_values
from synth.layout import BF16, BIT1, FP8, FP16, INT2, INT4, INT8

ALL_PAIRS = [(FP16, FP16), (BF16, BF16), (FP8, FP8), (INT8, INT4), (INT4, INT8), (FP8, FP16),
             (INT2, INT2), (BIT1, BIT1), (INT2, BIT1), (INT8, INT2)]


def small(seq_lens, kc=FP16, vc=FP16, hq=4, hkv=2, dim=32, page=16, seed=5, **kw):
    return synth.build_workload("t", rows=len(seq_lens), hq=hq, hkv=hkv, dim=dim, page=page,
                                seq_lens=seq_lens, codec_of=kw.pop("codec_of", lambda r, lp: (kc, vc)),
                                seed=seed, keep_values=True, **kw)


def logical_values(w, row, h):
    """FP16 reference K, V in logical order straight from the pre-encoding values."""
    P, L = w.page_size, int(w.seq_lens[row])
    ks, vs = [], []
    for lp in range(-(-L // P)):
        xk, xv = w.info["values"][(row, lp)]
        n = min(P, L - lp * P)
        ks.append(xk[h, :n].astype(np.float16).astype(np.float64))
        vs.append(xv[h, :n].astype(np.float16).astype(np.float64))
    return np.concatenate(ks), np.concatenate(vs)


# ---------------------------------------------------------------- SDPA / GQA
def test_fp16_config1_equals_sdpa_with_gqa():
    w = synth.config(1)
    out, lse = decode_attention(w)
    hq, hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    K = np.stack([logical_values_cfg1(w, h)[0] for h in range(hkv)])   # [Hkv, N, D]
    V = np.stack([logical_values_cfg1(w, h)[1] for h in range(hkv)])
    q = torch.from_numpy(w.q[0].astype(np.float64))[None, :, None, :]  # [1, Hq, 1, D]
    Kt, Vt = torch.from_numpy(K)[None], torch.from_numpy(V)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, scale=w.softmax_scale,
                                                           enable_gqa=True)[0, :, 0].numpy()
    assert np.max(np.abs(out[0] - ref)) <= 1e-12
    # replicated-head MHA (repeat_interleave) equals the GQA result
    Kr, Vr = Kt.repeat_interleave(hq // hkv, dim=1), Vt.repeat_interleave(hq // hkv, dim=1)
    mha = torch.nn.functional.scaled_dot_product_attention(q, Kr, Vr, scale=w.softmax_scale)
    assert np.max(np.abs(out[0] - mha[0, :, 0].numpy())) <= 1e-12
    s = torch.einsum("hd,hnd->hn", q[0, :, 0], Kr[0]) * w.softmax_scale
    assert np.max(np.abs(lse[0] - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


def logical_values_cfg1(w, h):
    # the tiny FP16 workload is generated without keep_values; rebuild it with them
    global _CFG1
    try:
        w1 = _CFG1
    except NameError:
        w1 = _CFG1 = synth.build_workload(
            "t", rows=1, hq=14, hkv=2, dim=64, page=1024, seq_lens=[4096],
            codec_of=lambda r, lp: (FP16, FP16), seed=1001, keep_values=True)
    assert np.array_equal(w1.q, w.q) and np.array_equal(w1.block_table, w.block_table)
    return logical_values(w1, 0, h)


def test_gqa_head_mapping_small():
    w = small([37, 50], hq=6, hkv=2)
    out, _ = decode_attention(w)
    for r in range(2):
        for hq in range(6):
            K, V = logical_values(w, r, hq // 3)
            q = torch.from_numpy(w.q[r, hq].astype(np.float64))[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
                scale=w.softmax_scale)[0, 0, 0].numpy()
            assert np.max(np.abs(out[r, hq] - ref)) <= 1e-12


# --------------------------------------------------- streaming == full softmax
def streamed(w, row, h, q, tau):
    """Independent page-at-a-time online softmax over the row's pages."""
    P, L = w.page_size, int(w.seq_lens[row])
    m = np.full(q.shape[0], -np.inf)
    l = np.zeros(q.shape[0])
    acc = np.zeros((q.shape[0], w.head_dim))
    lps = (sorted(int(x) for x in w.page_sel[row, :w.sel_lens[row]]) if w.sparse
           else range(-(-L // P)))
    for lp in lps:
        n = max(0, min(P, L - lp * P))
        if n == 0:
            continue
        pp = int(w.block_table[row, lp])
        c = int(w.page_codec[pp])
        K = plane_values(w.pool, int(w.page_k_off[pp]), c & 15, w.num_kv_heads, P, w.head_dim,
                         h, w.page_scale[pp, h, 0], False, n)
        V = plane_values(w.pool, int(w.page_v_off[pp]), c >> 4, w.num_kv_heads, P, w.head_dim,
                         h, w.page_scale[pp, h, 1], True, n)
        s = tau * q @ K.T                            # [G, n]
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ V
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1)[:, None], 0), m + np.log(l)


@pytest.mark.parametrize("kc,vc", ALL_PAIRS)
def test_streaming_equals_full(kc, vc):
    w = small([100, 16, 67], kc, vc, hq=8, hkv=2, dim=64, page=32)
    out, lse = decode_attention(w)
    G = 4
    for r in range(w.rows):
        for h in range(2):
            q = w.q[r, h * G:(h + 1) * G].astype(np.float64)
            o, s = streamed(w, r, h, q, w.softmax_scale)
            assert np.max(np.abs(o - out[r, h * G:(h + 1) * G])) <= 1e-12
            assert np.max(np.abs(s - lse[r, h * G:(h + 1) * G])) <= 1e-12


def test_streaming_equals_full_configs_small():
    for cid in (2, 3, 4, 5):
        w = synth.config(cid, small=True)
        rows = range(min(w.rows, 2))
        out, lse = decode_attention(w, rows=rows)
        G = w.num_q_heads // w.num_kv_heads
        for ri, r in enumerate(rows):
            for h in range(w.num_kv_heads):
                q = w.q[r, h * G:(h + 1) * G].astype(np.float64)
                o, s = streamed(w, r, h, q, w.softmax_scale)
                assert np.max(np.abs(o - out[ri, h * G:(h + 1) * G])) <= 1e-11
                assert np.max(np.abs(s - lse[ri, h * G:(h + 1) * G])) <= 1e-11


# -------------------------------------------------- brute force, closed forms
def brute(K, V, q, tau):
    s = [tau * math.fsum(q[i] * K[t, i] for i in range(len(q))) for t in range(K.shape[0])]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = math.fsum(e)
    out = [math.fsum(e[t] * V[t, i] for t in range(len(e))) / l for i in range(V.shape[1])]
    return np.array(out), m + math.log(l)


@pytest.mark.parametrize("kc,vc", ALL_PAIRS)
@pytest.mark.parametrize("L", [1, 2, 5, 8])
def test_brute_force_tiny(kc, vc, L):
    # one row, one KV head, head_dim 32, at most 8 tokens (tiny synthetic shape)
    w = small([L], kc, vc, hq=2, hkv=1, dim=32, page=16)
    out, lse = decode_attention(w)
    K, V = gather_kv(w, 0, 0)
    for g in range(2):
        o, s = brute(K, V, w.q[0, g].astype(np.float64), w.softmax_scale)
        assert np.max(np.abs(o - out[0, g])) <= 1e-13
        assert abs(s - lse[0, g]) <= 1e-13


def test_closed_forms():
    w = small([1], hq=1, hkv=1, dim=32)
    out, lse = decode_attention(w)
    K, V = gather_kv(w, 0, 0)
    q = w.q[0, 0].astype(np.float64)
    assert np.array_equal(out[0, 0], V[0])                      # one token: out = V0
    assert abs(lse[0, 0] - w.softmax_scale * math.fsum(q * K[0])) <= 1e-14

    w = small([2], hq=1, hkv=1, dim=32)
    out, _ = decode_attention(w)
    K, V = gather_kv(w, 0, 0)
    q = w.q[0, 0].astype(np.float64)
    s0, s1 = (w.softmax_scale * math.fsum(q * K[t]) for t in (0, 1))
    sig = 1.0 / (1.0 + math.exp(s1 - s0))
    assert np.max(np.abs(out[0, 0] - (sig * V[0] + (1 - sig) * V[1]))) <= 1e-14

    w = small([45], hq=1, hkv=1, dim=32)
    w.q[:] = 0                                                   # q = 0: uniform weights
    out, lse = decode_attention(w)
    K, V = gather_kv(w, 0, 0)
    assert np.max(np.abs(out[0, 0] - V.mean(axis=0))) <= 1e-14
    assert abs(lse[0, 0] - math.log(45)) <= 1e-14


def test_empty_rows():
    w = small([0, 20])
    out, lse = decode_attention(w)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf) and np.all(np.isfinite(lse[1]))
    ws = synth.config(4, small=True)
    ws.sel_lens[1] = 0
    out, lse = decode_attention(ws, rows=[1])
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ------------------------------------------------------------- invariances
def test_placement_invariance():
    a = small([90, 61], FP8, INT4, seed=11)
    rng = synth.streams(11)
    rng["placement"] = np.random.default_rng(99)
    b = small([90, 61], FP8, INT4, seed=11, rng=rng)
    assert not np.array_equal(a.block_table, b.block_table)
    oa, la = decode_attention(a)
    ob, lb = decode_attention(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_selection_order_invariance():
    w = synth.config(4, small=True)
    oa, la = decode_attention(w)
    rng = np.random.default_rng(4)
    for r in range(w.rows):
        w.page_sel[r] = rng.permutation(w.page_sel[r])
    ob, lb = decode_attention(w)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@settings(max_examples=40, deadline=None)
@given(n=st.integers(1, 300), parts=st.integers(1, 16), seed=st.integers(0, 2**31 - 1),
       peak=st.floats(0.1, 8.0))
def test_fold_is_partition_invariant(n, parts, seed, peak):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((n, 16))
    V = rng.standard_normal((n, 16))
    q = peak * rng.standard_normal((3, 16))
    cuts = np.sort(rng.integers(0, n + 1, size=parts - 1))
    bounds = [0, *cuts.tolist(), n]                             # empty parts allowed
    acc, m, l = partials(K, V, q, 0.25, bounds)
    out, lse = fold(acc, m, l)
    full_acc, full_m, full_l = partials(K, V, q, 0.25, [0, n])
    ref_out, ref_lse = fold(full_acc, full_m, full_l)
    assert np.max(np.abs(out - ref_out)) <= 1e-12
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12
    # and the unsplit fold is the plain softmax definition
    s = 0.25 * q @ K.T
    p = np.exp(s - s.max(1, keepdims=True))
    assert np.max(np.abs(ref_out - (p @ V) / p.sum(1, keepdims=True))) <= 1e-12


@pytest.mark.parametrize("workers", [1, 4, 16, 512])
def test_fold_worker_counts(workers):
    rng = np.random.default_rng(workers)
    n = 2048
    K, V, q = rng.standard_normal((n, 32)), rng.standard_normal((n, 32)), 3 * rng.standard_normal((2, 32))
    bounds = np.linspace(0, n, workers + 1).astype(int).tolist()
    out, lse = fold(*partials(K, V, q, 0.2, bounds))
    ref_out, ref_lse = fold(*partials(K, V, q, 0.2, [0, n]))
    assert np.max(np.abs(out - ref_out)) <= 1e-12 and np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_fold_all_empty():
    out, lse = fold(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf), np.zeros((2, 3)))
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_fold_ignores_parts_marked_empty():
    """An empty part is marked by m = -inf or l = 0; its other fields are
    never read. Extra parts (-inf, l > 0, junk acc) and (finite m, 0, junk
    acc) -- the latter with a max far above every real one -- leave the fold
    of the real parts unchanged, and a row of only such parts is empty."""
    rng = np.random.default_rng(12)
    n, D = 600, 16
    K, V, q = rng.standard_normal((n, D)), rng.standard_normal((n, D)), 2 * rng.standard_normal((3, D))
    acc, m, l = partials(K, V, q, 0.3, [0, 100, 350, n])
    ref_out, ref_lse = fold(acc, m, l)
    junk = rng.standard_normal((3, 2, D)) * 1e3
    acc2 = np.concatenate([acc[:, :1], junk[:, :1], acc[:, 1:], junk[:, 1:]], axis=1)
    m2 = np.concatenate([m[:, :1], np.full((3, 1), -np.inf), m[:, 1:], np.full((3, 1), 1e4)], axis=1)
    l2 = np.concatenate([l[:, :1], np.full((3, 1), 5.0), l[:, 1:], np.zeros((3, 1))], axis=1)
    out, lse = fold(acc2, m2, l2)
    assert np.max(np.abs(out - ref_out)) <= 1e-12 and np.max(np.abs(lse - ref_lse)) <= 1e-12
    out, lse = fold(junk, np.stack([np.full(3, -np.inf), np.full(3, 1e4)], 1),
                    np.stack([np.full(3, 5.0), np.zeros(3)], 1))
    assert np.all(out == 0) and np.all(lse == -np.inf)


def dequant_reference(x, codec):
    """Pre-encoding float32 block [P, D] -> the value its codes denote (float64),
    computed from the codec definitions with library casts."""
    from synth.encode import encode_int_g32
    if codec == FP16:
        return x.astype(np.float16).astype(np.float64)
    if codec == BF16:
        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    if codec == FP8:
        s = np.float32(np.abs(x).max() / np.float32(448.0))
        c = torch.from_numpy(np.clip(x / s, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
        return c.to(torch.float64).numpy() * float(s)
    if codec == INT2:
        from synth.encode import encode_affine2_g32
        u, sc, z = encode_affine2_g32(x)
        return z.astype(np.float64).repeat(32, axis=-1) + u * sc.astype(np.float64).repeat(32, axis=-1)
    if codec == BIT1:
        from synth.encode import encode_sign1_g32
        b, sc = encode_sign1_g32(x)
        return np.where(b == 1, -1.0, 1.0) * sc.astype(np.float64).repeat(32, axis=-1)
    cq, sc = encode_int_g32(x, 127 if codec == INT8 else 7)
    return cq.astype(np.float64) * sc.astype(np.float64).repeat(32, axis=-1)


@pytest.mark.parametrize("kc,vc", ALL_PAIRS)
def test_gather_matches_pre_encoding_values(kc, vc):
    w = small([70, 33], kc, vc, hq=6, hkv=3, dim=64, page=32,
              codec_of=lambda r, lp: (kc, vc) if (r + lp) % 2 == 0 else (vc if vc != INT4 else INT8, kc))
    for r in range(w.rows):
        for h in range(w.num_kv_heads):
            K, V = gather_kv(w, r, h)
            L, P = int(w.seq_lens[r]), w.page_size
            rk, rv = [], []
            for lp in range(-(-L // P)):
                xk, xv = w.info["values"][(r, lp)]
                c = int(w.page_codec[w.block_table[r, lp]])
                n = min(P, L - lp * P)
                rk.append(dequant_reference(xk[h], c & 15)[:n])
                rv.append(dequant_reference(xv[h], c >> 4)[:n])
            assert np.array_equal(K, np.concatenate(rk))
            assert np.array_equal(V, np.concatenate(rv))


def test_gather_sparse_uses_selected_pages_only():
    w = synth.config(4, small=True)
    P = w.page_size
    for r in range(2):
        K, _ = gather_kv(w, r, 1)
        assert K.shape[0] == P * w.page_sel.shape[1]
        # the selected pages, ascending, are the only ones read: corrupting every
        # descriptor of an unselected page changes nothing
    keep = {int(w.block_table[r, lp]) for r in range(w.rows) for lp in w.page_sel[r]}
    before = decode_attention(w)
    for pp in range(w.num_pages):
        if pp not in keep:
            w.page_codec[pp] = 0xFF
            w.page_k_off[pp] = np.uint64(2**60)
    after = decode_attention(w)
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])


def test_sliding_window_decode_pins():
    """Sliding-window decode (each row attends its last W positions):
    W = 0 and W >= L leave the result unchanged; W = 1 gives the last
    token's V and score (closed form); any W equals the chunked-prefill
    oracle's query at T = 1 with the same window (its own masks)."""
    from oracle.prefill import prefill_attention
    w = small([1, 40, 300, 513], FP8, INT8, hq=8, hkv=2, dim=64, page=32, seed=4)
    full = decode_attention(w)
    for W in (0, 513, 10_000):
        o, l = decode_attention(w, window=W)
        assert np.array_equal(o, full[0]) and np.array_equal(l, full[1])
    o1, l1 = decode_attention(w, window=1)
    G = 4
    for r in range(w.rows):
        L = int(w.seq_lens[r])
        for h in range(2):
            K, V = gather_kv(w, r, h)
            q = w.q[r, h * G:(h + 1) * G].astype(np.float64)
            assert np.array_equal(o1[r, h * G:(h + 1) * G], np.broadcast_to(V[L - 1], (G, 64)))
            assert np.allclose(l1[r, h * G:(h + 1) * G], w.softmax_scale * (q @ K[L - 1]), rtol=0, atol=1e-12)
    q1 = w.q[:, None].astype(np.float16)
    for W in (1, 7, 32, 33, 100, 299):
        o, l = decode_attention(w, window=W)
        po, pl = prefill_attention(w, q1, window=W)
        assert np.max(np.abs(o - po[:, 0])) <= 1e-12 and np.max(np.abs(l - pl[:, 0])) <= 1e-12


def test_sliding_window_sparse_brute_force():
    """Sparse mode with a window: only the selected pages' tokens at
    positions >= L - W, by direct math.fsum evaluation."""
    w = synth.build_workload("win_sparse", rows=1, hq=1, hkv=1, dim=64, page=16, seq_lens=[100],
                             codec_of=lambda r, lp: (FP16, FP16), seed=8,
                             selection=np.array([[6, 1, 4]], np.int32), logical_pages=7)
    P, L, W = 16, 100, 40                                  # positions >= 60: page 4 from token 64, page 6 to 99
    o, l = decode_attention(w, window=W)
    K, V = gather_kv(w, 0, 0)                               # pages 1, 4, 6 ascending: 16 + 16 + 4 tokens
    pos = np.concatenate([np.arange(16, 32), np.arange(64, 80), np.arange(96, 100)])
    keep = pos >= L - W
    q = w.q[0, 0].astype(np.float64)
    s = [w.softmax_scale * math.fsum(q * k) for k in K[keep]]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    den = math.fsum(e)
    ref = np.array([math.fsum(e[i] * V[keep][i][d] for i in range(len(e))) / den for d in range(64)])
    assert np.max(np.abs(o[0, 0] - ref)) <= 1e-12 and abs(l[0, 0] - (m + math.log(den))) <= 1e-12
    assert keep.sum() == 20
