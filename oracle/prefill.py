"""Chunked-prefill (multi-query) attention over the paged cache, and the
fold of one window's result into a running accumulator, plain float64.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Definition followed (FreeToken PR #499 discussion, in-place host K/V design:
a prefill attends the cached pages window by window and folds the windows by
their log-sum-exp into a float32 accumulator; ARGUS "Why decode is slow" for
grouped-query attention). A chunk of T new query tokens per row has already
been appended to the cache, so it is the last T of the row's L tokens: query
t sits at position pos = L - T + t and, causally, attends the cached tokens
j <= pos. A call may restrict the keys to a window [kv_begin, kv_end):

    keys(t) = { j : max(kv_begin, 0, pos + 1 - W) <= j < min(kv_end, pos + 1) }
    s_j     = tau * sum_i q[t][hq][i] * K_j[h][i]            (h = hq // G)
    out     = sum_j exp(s_j - m) V_j[h] / sum_j exp(s_j - m),   m = max_j s_j
    lse     = m + ln(sum_j exp(s_j - m))                       (natural log)

with W the sliding-window length (ARGUS v0.5: direct attention supports
sliding-window masks): each query sees at most its last W positions, its
own included; W <= 0 means no sliding window. An empty key set (a window
that misses the query's range, or pos < 0 when T > L) gives out = 0 and
lse = -inf. With T = 1 and no sliding window this is the decode definition
of ``attention.decode_attention``.

``fold_into`` merges the result of one more window into an accumulator that
holds the result over the windows seen so far (both as (out, lse)):

    M = max(lse_a, lse_b);  w_a = exp(lse_a - M);  w_b = exp(lse_b - M)
    out = (w_a out_a + w_b out_b) / (w_a + w_b);  lse = M + ln(w_a + w_b)

with both empty (-inf) giving (0, -inf). An empty side holds no attended
token, so it contributes no term: its out values are undefined and are
never read into the result. Folding the windows of a partition of the key
range in any order gives the result over the whole range.

Pins: tests/test_oracle_prefill.py (torch SDPA with an explicit boolean mask
in float64, the decode oracle at T = 1, closed forms of the causal edge,
brute force with math.fsum, window fold against the whole range, fold
identities).
"""
from __future__ import annotations

import numpy as np

from .attention import _softmax_attention, gather_kv


def prefill_attention(w, q, kv_begin: int = 0, kv_end: int | None = None, rows=None, window: int = 0):
    """q: [rows_all, T, Hq, D] (fp16 values). Dense workloads only.

    Returns out float64 [len(rows), T, Hq, D] and lse float64 [len(rows), T, Hq]."""
    if w.page_sel is not None:
        raise ValueError("prefill attends the dense cache (no page selection)")
    q = np.asarray(q)
    T = q.shape[1]
    hq, hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = hq // hkv
    tau = float(w.softmax_scale)
    rows = list(range(w.rows) if rows is None else rows)
    out = np.zeros((len(rows), T, hq, D))
    lse = np.full((len(rows), T, hq), -np.inf)
    lo = max(int(kv_begin), 0)
    for ri, r in enumerate(rows):
        L = int(w.seq_lens[r])
        for h in range(hkv):
            K, V = gather_kv(w, r, h)                       # tokens 0 .. L-1, logical order
            for t in range(T):
                pos = L - T + t
                hi = pos + 1 if kv_end is None else min(int(kv_end), pos + 1)
                lo_t = max(lo, pos + 1 - int(window)) if window > 0 else lo
                if hi <= lo_t:
                    continue
                qt = q[r, t, h * G:(h + 1) * G].astype(np.float64)
                o, s = _softmax_attention(K[lo_t:hi], V[lo_t:hi], qt, tau)
                out[ri, t, h * G:(h + 1) * G] = o
                lse[ri, t, h * G:(h + 1) * G] = s
    return out, lse


def fold_into(acc_out, acc_lse, out, lse):
    """Returns the fold of (out, lse) into (acc_out, acc_lse); shapes
    [..., D] and [...]."""
    ao, al = np.asarray(acc_out, float), np.asarray(acc_lse, float)
    bo, bl = np.asarray(out, float), np.asarray(lse, float)
    M = np.maximum(al, bl)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wa = np.where(np.isfinite(al), np.exp(al - Ms), 0.0)
    wb = np.where(np.isfinite(bl), np.exp(bl - Ms), 0.0)
    den = wa + wb
    safe = np.where(finite, den, 1.0)
    ta = np.where((wa > 0)[..., None], wa[..., None] * ao, 0.0)    # an empty side adds no term
    tb = np.where((wb > 0)[..., None], wb[..., None] * bo, 0.0)
    res = np.where(finite[..., None], (ta + tb) / safe[..., None], 0.0)
    return res, np.where(finite, Ms + np.log(safe), -np.inf)
