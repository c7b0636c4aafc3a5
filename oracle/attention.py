"""Decode attention over a mixed-codec paged KV cache, plain float64.

Definition followed (ARGUS "Why decode is slow" and "Direct paged attention":
the page-streamed online softmax is exact, so its result is the ordinary
softmax attention below):

    s_t   = tau * sum_i q_i * K[t, i]               (tau = softmax_scale)
    m     = max_t s_t
    l     = sum_t exp(s_t - m)
    out   = sum_t exp(s_t - m) * V[t, :] / l
    lse   = m + ln(l)                               (natural log)

for every query head, with query head ``hq`` reading KV head ``hq // G``
(G = Hq / Hkv; grouped-query attention, "Why decode is slow"). The attended
tokens are, in logical order, tokens 0..L-1 reached through the block table
(FreeToken PR #499 "Design": logical -> physical translation), or in sparse
mode the tokens t < L of the selected logical pages only (PR #499 "Why this
works"). A sliding window of W tokens (ARGUS "v0.5": direct attention with
sliding-window masks) keeps only positions t >= L - W, the row's last W
positions; W <= 0 means none. An empty token set gives out = 0 and
lse = -inf.

``fold`` combines partial results by their log-sum-exp (PR #499 discussion,
in-place host K/V design).

Pins: tests/test_oracle_attention.py (torch SDPA in float64, an independent
page-streamed online softmax, brute force with math.fsum, closed forms, GQA
replication, placement and selection-order invariance, fold invariance).
"""
from __future__ import annotations

import numpy as np

from .layout import plane_values


def attended_pages(w, row: int) -> list[tuple[int, int]]:
    """(logical page, valid tokens) of one row, ascending logical order."""
    P = w.page_size
    L = int(w.seq_lens[row])
    if w.page_sel is not None:
        lps = sorted(int(x) for x in w.page_sel[row, : int(w.sel_lens[row])])
    else:
        lps = list(range(-(-L // P))) if L > 0 else []
    return [(lp, max(0, min(P, L - lp * P))) for lp in lps]


def attended_positions(w, row: int) -> np.ndarray:
    """Logical token positions of the row's attended tokens, in the order
    ``gather_kv`` returns them (before any sliding window)."""
    P = w.page_size
    pos = [np.arange(lp * P, lp * P + valid) for lp, valid in attended_pages(w, row) if valid > 0]
    return np.concatenate(pos) if pos else np.zeros(0, dtype=np.int64)


def gather_kv(w, row: int, h: int) -> tuple[np.ndarray, np.ndarray]:
    """K, V float64 [N, D] of KV head ``h`` over the row's attended tokens."""
    D, P, hkv = w.head_dim, w.page_size, w.num_kv_heads
    pages = [(lp, valid) for lp, valid in attended_pages(w, row) if valid > 0]
    n = sum(valid for _, valid in pages)
    K, V = np.empty((n, D)), np.empty((n, D))
    t = 0
    for lp, valid in pages:
        pp = int(w.block_table[row, lp])
        codec = int(w.page_codec[pp])
        kc, vc = codec & 0xF, codec >> 4
        sk, sv = w.page_scale[pp, h]
        K[t:t + valid] = plane_values(w.pool, int(w.page_k_off[pp]), kc, hkv, P, D, h, sk, False, valid)
        V[t:t + valid] = plane_values(w.pool, int(w.page_v_off[pp]), vc, hkv, P, D, h, sv, True, valid)
        t += valid
    return K, V


def _softmax_attention(K, V, q, tau):
    """q: [G, D] float64. Returns out [G, D], lse [G]."""
    G, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((G, D)), np.full(G, -np.inf)
    s = tau * (K @ q.T)                     # [N, G]
    m = s.max(axis=0)
    e = np.exp(s - m)
    l = e.sum(axis=0)
    out = (e.T @ V) / l[:, None]
    return out, m + np.log(l)


def decode_attention(w, rows=None, window=None):
    """out float64 [rows, Hq, D], lse float64 [rows, Hq]. ``window``: the
    sliding window in tokens (default: the workload's ``window_tokens``, if
    any; <= 0 means none)."""
    rows = range(w.rows) if rows is None else rows
    if window is None:
        window = int(getattr(w, "window_tokens", 0) or 0)
    hq, hkv, D = w.num_q_heads, w.num_kv_heads, w.head_dim
    G = hq // hkv
    rows = list(rows)
    out = np.zeros((len(rows), hq, D))
    lse = np.zeros((len(rows), hq))
    for ri, r in enumerate(rows):
        keep = None
        if window > 0:
            keep = attended_positions(w, r) >= int(w.seq_lens[r]) - window
        for h in range(hkv):
            K, V = gather_kv(w, r, h)
            if keep is not None:
                K, V = K[keep], V[keep]
            q = w.q[r, h * G:(h + 1) * G].astype(np.float64)
            o, s = _softmax_attention(K, V, q, float(w.softmax_scale))
            out[ri, h * G:(h + 1) * G] = o
            lse[ri, h * G:(h + 1) * G] = s
    return out, lse


def partials(K, V, q, tau, bounds):
    """Unnormalised partial results over token ranges.

    bounds: cut points 0 = b0 <= b1 <= ... <= bn = N. For part p with tokens
    [b_p, b_{p+1}): acc_p = sum exp(s_t - m_p) V[t], m_p = max s_t,
    l_p = sum exp(s_t - m_p); an empty part gives (0, -inf, 0).
    Returns acc [G, n, D], m [G, n], l [G, n].
    """
    G, D = q.shape
    n = len(bounds) - 1
    acc = np.zeros((G, n, D))
    m = np.full((G, n), -np.inf)
    l = np.zeros((G, n))
    for p in range(n):
        a, b = bounds[p], bounds[p + 1]
        if b <= a:
            continue
        s = tau * (K[a:b] @ q.T)
        mp = s.max(axis=0)
        e = np.exp(s - mp)
        acc[:, p] = e.T @ V[a:b]
        m[:, p] = mp
        l[:, p] = e.sum(axis=0)
    return acc, m, l


def fold(acc, m, l):
    """Fold partials along the part axis by log-sum-exp.

    acc [..., n, D], m [..., n], l [..., n] ->
    M = max_p m_p; w_p = exp(m_p - M); L = sum_p w_p l_p;
    out = sum_p w_p acc_p / L; lse = M + ln L. All parts empty -> (0, -inf).

    A part is empty unless l_p > 0 and m_p is finite (an empty partition
    leaves (0, -inf, 0)); empty parts take no part in M and their acc is
    never read.
    """
    acc, m, l = np.asarray(acc, float), np.asarray(m, float), np.asarray(l, float)
    live = np.isfinite(m) & (l > 0)
    M = np.where(live, m, -np.inf).max(axis=-1)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wts = np.where(live, np.exp(np.where(live, m, 0.0) - Ms[..., None]), 0.0)
    L = (wts * l).sum(axis=-1)
    num = (np.where(live[..., None], wts[..., None] * np.where(live[..., None], acc, 0.0), 0.0)).sum(axis=-2)
    safe = np.where(finite & (L > 0), L, 1.0)
    out = np.where((finite & (L > 0))[..., None], num / safe[..., None], 0.0)
    lse = np.where(finite & (L > 0), Ms + np.log(safe), -np.inf)
    return out, lse
