"""Pins for oracle/prefill.py (chunked-prefill attention and the window
fold), no GPU.

Checked against things other than the oracle: torch's scaled_dot_product_attention
in float64 with an explicit boolean mask built from the positions (a library
routine), the decode oracle at T = 1 (pinned on its own against SDPA),
closed forms at the causal edge, direct evaluation with math.fsum on a tiny
case, and the fold's identities (an empty window changes nothing, two equal
results keep out and add ln 2 to lse, order does not matter, and it equals
the partial-result fold of attention.fold with unit sums).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import decode_attention, fold, fold_into, prefill_attention
from synth.layout import BF16, FP8, FP16, INT4, INT8


def small(seq_lens, kc=FP16, vc=FP16, hq=4, hkv=2, dim=32, page=16, seed=5, **kw):
    return synth.build_workload("t", rows=len(seq_lens), hq=hq, hkv=hkv, dim=dim, page=page,
                                seq_lens=seq_lens, codec_of=kw.pop("codec_of", lambda r, lp: (kc, vc)),
                                seed=seed, keep_values=True, **kw)


def logical_values(w, row, h):
    """K, V float64 [L, D] in logical order from the pre-encoding values (FP16 pages)."""
    P, L = w.page_size, int(w.seq_lens[row])
    ks, vs = [], []
    for lp in range(-(-L // P)):
        xk, xv = w.info["values"][(row, lp)]
        n = min(P, L - lp * P)
        ks.append(xk[h, :n].astype(np.float16).astype(np.float64))
        vs.append(xv[h, :n].astype(np.float16).astype(np.float64))
    return np.concatenate(ks), np.concatenate(vs)


def sdpa_reference(w, q, kv_begin, kv_end, window=0):
    """torch SDPA (float64, GQA) with the causal/window mask as a boolean matrix."""
    T, hq, D = q.shape[1], w.num_q_heads, w.head_dim
    hkv = w.num_kv_heads
    outs, lses = [], []
    for r in range(w.rows):
        L = int(w.seq_lens[r])
        K = torch.from_numpy(np.stack([logical_values(w, r, h)[0] for h in range(hkv)]))[None]
        V = torch.from_numpy(np.stack([logical_values(w, r, h)[1] for h in range(hkv)]))[None]
        pos = L - T + torch.arange(T)
        j = torch.arange(L)
        mask = (j[None, :] <= pos[:, None]) & (j[None, :] >= max(kv_begin, 0))
        if kv_end is not None:
            mask &= j[None, :] < kv_end
        if window > 0:
            mask &= j[None, :] > pos[:, None] - window
        qt = torch.from_numpy(q[r].astype(np.float64)).permute(1, 0, 2)[None]    # [1, Hq, T, D]
        o = torch.nn.functional.scaled_dot_product_attention(qt, K, V, attn_mask=mask, scale=w.softmax_scale,
                                                             enable_gqa=True)
        outs.append(o[0].permute(1, 0, 2).numpy())
        Kr = K.repeat_interleave(hq // hkv, dim=1)
        s = (qt @ Kr.transpose(-1, -2)) * w.softmax_scale                       # [1, Hq, T, L]
        s = s.masked_fill(~mask, -math.inf)
        lses.append(torch.logsumexp(s, dim=-1)[0].permute(1, 0).numpy())
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("T,kv_begin,kv_end", [(7, 0, None), (16, 0, None), (5, 40, None), (9, 17, 80),
                                              (1, 0, None)])
def test_equals_sdpa_with_mask(T, kv_begin, kv_end):
    w = small([100, 64, 131], hq=6, hkv=2, dim=32)
    q = synth.prefill_queries(3, w.rows, T, w.num_q_heads, w.head_dim)
    out, lse = prefill_attention(w, q, kv_begin, kv_end)
    ref_o, ref_l = sdpa_reference(w, q, kv_begin, kv_end)
    assert np.max(np.abs(out - ref_o)) <= 1e-12
    assert np.max(np.abs(lse - ref_l)) <= 1e-12


@pytest.mark.parametrize("kc,vc", [(FP16, FP16), (FP8, FP8), (INT8, INT4), (BF16, FP8)])
def test_single_query_is_decode(kc, vc):
    w = small([70, 33], kc=kc, vc=vc, hq=8, hkv=2, dim=64)
    q = w.q[:, None].copy()                                   # [rows, 1, Hq, D]
    out, lse = prefill_attention(w, q)
    d_out, d_lse = decode_attention(w)
    assert np.array_equal(out[:, 0], d_out) and np.array_equal(lse[:, 0], d_lse)


def test_causal_edge_closed_forms():
    """A row that is all chunk (T = L): query 0 sees only token 0 (out = V_0,
    lse = s_0); query 1 sees tokens 0, 1 (sigmoid weights)."""
    w = small([12], hq=2, hkv=1, dim=32)
    T = 12
    q = synth.prefill_queries(9, 1, T, 2, 32)
    out, lse = prefill_attention(w, q)
    K, V = logical_values(w, 0, 0)
    tau = w.softmax_scale
    for hq in range(2):
        qq = q[0, :, hq].astype(np.float64)
        s0 = tau * qq[0] @ K[0]
        assert np.array_equal(out[0, 0, hq], V[0]) and lse[0, 0, hq] == pytest.approx(s0, abs=1e-14)
        a, b = tau * qq[1] @ K[0], tau * qq[1] @ K[1]
        w0 = 1 / (1 + math.exp(b - a))
        assert np.max(np.abs(out[0, 1, hq] - (w0 * V[0] + (1 - w0) * V[1]))) <= 1e-14
        assert lse[0, 1, hq] == pytest.approx(max(a, b) + math.log1p(math.exp(-abs(a - b))), abs=1e-13)


def test_brute_force_fsum():
    w = small([20], hq=2, hkv=1, dim=32, page=16)
    T = 3
    q = synth.prefill_queries(4, 1, T, 2, 32)
    out, lse = prefill_attention(w, q, 2, 19)
    K, V = logical_values(w, 0, 0)
    for t in range(T):
        pos = 20 - T + t
        js = range(2, min(19, pos + 1))
        for hq in range(2):
            qq = q[0, t, hq].astype(np.float64)
            s = [w.softmax_scale * math.fsum(qq[i] * K[j, i] for i in range(32)) for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            den = math.fsum(e)
            ref = [math.fsum(e[k] * V[j, i] for k, j in enumerate(js)) / den for i in range(32)]
            assert np.max(np.abs(out[0, t, hq] - ref)) <= 1e-13
            assert lse[0, t, hq] == pytest.approx(m + math.log(den), abs=1e-13)


def test_empty_key_sets():
    w = small([10, 40], hq=2, hkv=1, dim=32)
    T = 14                                       # T > L for row 0: queries 0..3 sit before the row
    q = synth.prefill_queries(5, 2, T, 2, 32)
    out, lse = prefill_attention(w, q)
    assert np.all(out[0, :4] == 0) and np.all(lse[0, :4] == -np.inf)
    assert np.all(np.isfinite(lse[0, 4:])) and np.all(np.isfinite(lse[1]))
    out, lse = prefill_attention(w, q, 40, None)  # window past every row
    assert np.all(out == 0) and np.all(lse == -np.inf)
    out, lse = prefill_attention(w, q, 5, 5)      # empty window
    assert np.all(out == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("cuts", [[0, 64, 128, 200], [0, 16, 17, 100, 151, 300], [0, 300]])
def test_window_fold_equals_whole_range(cuts):
    w = small([151, 96], kc=FP8, vc=INT8, hq=4, hkv=2, dim=64)
    T = 20
    q = synth.prefill_queries(6, 2, T, 4, 64)
    full_o, full_l = prefill_attention(w, q)
    acc_o = np.zeros_like(full_o)
    acc_l = np.full_like(full_l, -np.inf)
    order = list(range(len(cuts) - 1))
    for i in reversed(order):                    # any order
        o, l = prefill_attention(w, q, cuts[i], cuts[i + 1])
        acc_o, acc_l = fold_into(acc_o, acc_l, o, l)
    assert np.max(np.abs(acc_o - full_o)) <= 1e-12
    fin = np.isfinite(full_l)
    assert np.array_equal(fin, np.isfinite(acc_l)) and np.max(np.abs(acc_l[fin] - full_l[fin])) <= 1e-12


def test_fold_into_identities():
    rng = np.random.default_rng(1)
    o1, o2 = rng.standard_normal((5, 8)), rng.standard_normal((5, 8))
    l1, l2 = rng.standard_normal(5) * 3, rng.standard_normal(5) * 3
    empty_o, empty_l = np.zeros((5, 8)), np.full(5, -np.inf)
    a, b = fold_into(o1, l1, empty_o, empty_l)
    assert np.array_equal(a, o1) and np.array_equal(b, l1)
    a, b = fold_into(empty_o, empty_l, o1, l1)
    assert np.array_equal(a, o1) and np.array_equal(b, l1)
    a, b = fold_into(empty_o, empty_l, empty_o, empty_l)
    assert np.all(a == 0) and np.all(b == -np.inf)
    a, b = fold_into(o1, l1, o1, l1)
    assert np.max(np.abs(a - o1)) <= 1e-15 and np.max(np.abs(b - (l1 + math.log(2)))) <= 1e-14
    x, y = fold_into(o1, l1, o2, l2)
    u, v = fold_into(o2, l2, o1, l1)
    assert np.max(np.abs(x - u)) <= 1e-15 and np.max(np.abs(y - v)) <= 1e-15
    # the partial-result fold with unit sums: acc_p = out_p, m_p = lse_p, l_p = 1
    f_o, f_l = fold(np.stack([o1, o2], axis=1), np.stack([l1, l2], axis=1), np.ones((5, 2)))
    assert np.max(np.abs(x - f_o)) <= 1e-14 and np.max(np.abs(y - f_l)) <= 1e-14
    # an empty side's values are undefined and never enter the result
    junk = np.full((5, 8), np.nan)
    a, b = fold_into(o1, l1, junk, empty_l)
    assert np.array_equal(a, o1) and np.array_equal(b, l1)
    a, b = fold_into(junk, empty_l, junk, empty_l)
    assert np.all(a == 0) and np.all(b == -np.inf)
    # closed form: lse = ln(e^l1 + e^l2)
    assert np.max(np.abs(y - np.logaddexp(l1, l2))) <= 1e-14


def test_rejects_sparse_workloads():
    w = synth.build_workload("s", rows=1, hq=2, hkv=1, dim=32, page=16, seq_lens=[64],
                             codec_of=lambda r, lp: (FP16, FP16), seed=1, selection=np.array([[0, 2]]))
    with pytest.raises(ValueError):
        prefill_attention(w, np.zeros((1, 1, 2, 32), np.float16))


@pytest.mark.parametrize("window,kv_begin,kv_end", [(1, 0, None), (5, 0, None), (40, 0, None), (33, 20, 90),
                                                    (1000, 0, None)])
def test_sliding_window_equals_banded_sdpa(window, kv_begin, kv_end):
    w = small([100, 64, 131], hq=6, hkv=2, dim=32)
    T = 9
    q = synth.prefill_queries(8, w.rows, T, w.num_q_heads, w.head_dim)
    out, lse = prefill_attention(w, q, kv_begin, kv_end, window=window)
    ref_o, ref_l = sdpa_reference(w, q, kv_begin, kv_end, window)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin)                     # empty windows: -inf on both
    assert np.all(out[~fin] == 0)
    assert np.max(np.abs(out[fin] - ref_o[fin])) <= 1e-12 and np.max(np.abs(lse[fin] - ref_l[fin])) <= 1e-12


def test_sliding_window_closed_forms():
    """W = 1: every query sees only itself (out = V_pos, lse = s_pos); W at
    least the row: the plain causal result."""
    w = small([50], hq=2, hkv=1, dim=32)
    T = 6
    q = synth.prefill_queries(12, 1, T, 2, 32)
    out, lse = prefill_attention(w, q, window=1)
    K, V = logical_values(w, 0, 0)
    for t in range(T):
        pos = 50 - T + t
        for hq in range(2):
            assert np.array_equal(out[0, t, hq], V[pos])
            assert lse[0, t, hq] == pytest.approx(w.softmax_scale * q[0, t, hq].astype(np.float64) @ K[pos], abs=1e-13)
    full = prefill_attention(w, q)
    wide = prefill_attention(w, q, window=50)
    assert np.array_equal(full[0], wide[0]) and np.array_equal(full[1], wide[1])
