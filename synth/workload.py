"""Seeded synthetic decode workloads: encoded pages, tables and queries.

Every random quantity comes from its own numpy PCG64 stream spawned from
``SeedSequence(seed)`` (roles: q, K, V, outliers, lengths, placement,
selection, spare), so changing one role never shifts another.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional

import numpy as np

from .layout import (CODECS, FP8, align, encode_plane, plane_bytes)
from .pool import Pool

ROLES = ("q", "k", "v", "outlier", "lengths", "placement", "selection", "spare")


def streams(seed: int) -> dict[str, np.random.Generator]:
    kids = np.random.SeedSequence(seed).spawn(len(ROLES))
    return {r: np.random.Generator(np.random.PCG64(s)) for r, s in zip(ROLES, kids)}


@dataclasses.dataclass
class Workload:
    name: str
    rows: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    softmax_scale: float
    partition_tokens: int
    q: np.ndarray               # float16 [rows, Hq, D]
    seq_lens: np.ndarray        # int32 [rows]
    block_table: np.ndarray     # int32 [rows, max_pages]
    page_sel: Optional[np.ndarray]   # int32 [rows, max_sel] or None (dense)
    sel_lens: Optional[np.ndarray]   # int32 [rows] or None
    page_k_off: np.ndarray      # uint64 [num_pages]
    page_v_off: np.ndarray      # uint64 [num_pages]
    page_codec: np.ndarray      # uint8 [num_pages]: low nibble K codec, high nibble V codec
    page_scale: np.ndarray      # float32 [num_pages, Hkv, 2]
    pool: Pool
    info: dict = dataclasses.field(default_factory=dict)
    window_tokens: int = 0      # sliding window of the decode call (0: none)

    @property
    def num_pages(self) -> int:
        return int(self.page_codec.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_sel(self) -> int:
        return 0 if self.page_sel is None else int(self.page_sel.shape[1])

    @property
    def sparse(self) -> bool:
        return self.page_sel is not None

    def attended_pages(self) -> list[list[tuple[int, int]]]:
        """Per row: (logical page, valid tokens) in the order the row lists them."""
        out = []
        p = self.page_size
        for r in range(self.rows):
            L = int(self.seq_lens[r])
            if self.sparse:
                lps = [int(x) for x in self.page_sel[r, : int(self.sel_lens[r])]]
            else:
                lps = list(range(-(-L // p)))
            out.append([(lp, max(0, min(p, L - lp * p))) for lp in lps])
        return out


def build_workload(name: str, *, rows: int, hq: int, hkv: int, dim: int, page: int,
                   seq_lens, codec_of: Callable[[int, int], tuple[int, int]],
                   seed: int, q_scale: float = 1.0, outlier_frac: float = 0.0,
                   outlier_mult: float = 8.0, selection: Optional[np.ndarray] = None,
                   logical_pages: Optional[int] = None, max_pages: Optional[int] = None,
                   partition_tokens: int = 0, rng: Optional[dict] = None,
                   chunk_pages: int = 256, info: Optional[dict] = None,
                   keep_values: bool = False) -> Workload:
    """Generate one workload.

    seq_lens      tokens per row.
    codec_of      (row, logical page) -> (K codec, V codec).
    selection     None (dense) or int [rows, nsel] logical pages per row.
    logical_pages logical pages that exist per row (default ceil(max L / P));
                  in sparse mode every one of them has a physical page, but
                  only selected pages carry generated data.
    keep_values   keep the float32 values of every generated page (before
                  encoding) in ``info["values"][(row, lp)] = (K, V)``, each
                  [Hkv, P, D]; for small test workloads.
    """
    info = dict(info or {})
    if keep_values:
        info["values"] = {}
    rng = rng or streams(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(rows)
    need = [-(-int(L) // page) for L in seq_lens]
    if logical_pages is None:
        logical_pages = max(need) if selection is None else max(need)
    width = max_pages if max_pages is not None else logical_pages
    assert width >= logical_pages

    # Logical pages that get a physical page, in (row, lp) order.
    if selection is None:
        owned = [(r, lp) for r in range(rows) for lp in range(need[r])]
    else:
        owned = [(r, lp) for r in range(rows) for lp in range(logical_pages)]
    num_pages = len(owned)
    perm = rng["placement"].permutation(num_pages).astype(np.int64)
    block_table = np.full((rows, width), -1, dtype=np.int32)
    phys_of = {}
    for i, (r, lp) in enumerate(owned):
        block_table[r, lp] = perm[i]
        phys_of[(r, lp)] = int(perm[i])

    # Codec per physical page and per-codec-pair contiguous regions.
    page_codec = np.zeros(num_pages, dtype=np.uint8)
    pair_of = np.zeros((num_pages, 2), dtype=np.int64)
    for (r, lp), pp in phys_of.items():
        kc, vc = codec_of(r, lp)
        assert kc in CODECS and vc in CODECS
        page_codec[pp] = kc | (vc << 4)
        pair_of[pp] = (kc, vc)
    page_k_off = np.zeros(num_pages, dtype=np.uint64)
    page_v_off = np.zeros(num_pages, dtype=np.uint64)
    base = 0
    region = {}
    for kc, vc in sorted({(int(a), int(b)) for a, b in pair_of}):
        members = np.nonzero((pair_of[:, 0] == kc) & (pair_of[:, 1] == vc))[0]  # ascending pp
        kb = align(plane_bytes(kc, hkv, page, dim))
        vb = align(plane_bytes(vc, hkv, page, dim))
        slot = kb + vb
        page_k_off[members] = base + np.arange(members.size, dtype=np.uint64) * slot
        page_v_off[members] = page_k_off[members] + kb
        region[(kc, vc)] = (base, slot, kb)
        base += members.size * slot
    pool = Pool(base)
    page_scale = np.ones((num_pages, hkv, 2), dtype=np.float32)

    # Which pages carry generated values, in generation order.
    if selection is None:
        gen = owned
    else:
        selection = np.asarray(selection, dtype=np.int32)
        gen = [(r, int(lp)) for r in range(rows) for lp in np.sort(selection[r])]
    dense_pool = selection is None
    if dense_pool:
        arena = np.zeros(base, dtype=np.uint8)

    shape = (hkv, page, dim)
    for c0 in range(0, len(gen), chunk_pages):
        chunk = gen[c0:c0 + chunk_pages]
        n = len(chunk)
        xk = rng["k"].standard_normal((n, *shape), dtype=np.float32)
        xv = rng["v"].standard_normal((n, *shape), dtype=np.float32)
        if outlier_frac > 0:
            mk = rng["outlier"].random((n, *shape)) < outlier_frac
            mv = rng["outlier"].random((n, *shape)) < outlier_frac
            xk = np.where(mk, xk * np.float32(outlier_mult), xk)
            xv = np.where(mv, xv * np.float32(outlier_mult), xv)
        if keep_values:
            for j, c in enumerate(chunk):
                info["values"][c] = (xk[j].copy(), xv[j].copy())
        pps = np.array([phys_of[c] for c in chunk], dtype=np.int64)
        pairs = pair_of[pps]
        for kc, vc in {(int(a), int(b)) for a, b in pairs}:
            sel = np.nonzero((pairs[:, 0] == kc) & (pairs[:, 1] == vc))[0]
            kbytes, ks = encode_plane(xk[sel], kc, v_order=False)
            vbytes, vs = encode_plane(xv[sel], vc, v_order=True)
            for j, idx in enumerate(sel):
                pp = int(pps[idx])
                ko, vo = int(page_k_off[pp]), int(page_v_off[pp])
                page_scale[pp, :, 0] = ks[j]
                page_scale[pp, :, 1] = vs[j]
                if dense_pool:
                    arena[ko:ko + kbytes.shape[1]] = kbytes[j]
                    arena[vo:vo + vbytes.shape[1]] = vbytes[j]
                else:
                    _, slot, kb = region[(kc, vc)]
                    seg = np.zeros(slot, dtype=np.uint8)
                    seg[:kbytes.shape[1]] = kbytes[j]
                    seg[kb:kb + vbytes.shape[1]] = vbytes[j]
                    pool.add_segment(ko, seg)
    if dense_pool:
        pool.add_segment(0, arena)

    q = (np.float32(q_scale) * rng["q"].standard_normal((rows, hq, dim), dtype=np.float32)).astype(np.float16)
    if selection is None:
        page_sel = sel_lens = None
    else:
        page_sel = np.ascontiguousarray(selection, dtype=np.int32)
        sel_lens = np.full(rows, page_sel.shape[1], dtype=np.int32)
    return Workload(name=name, rows=rows, num_q_heads=hq, num_kv_heads=hkv, head_dim=dim,
                    page_size=page, softmax_scale=1.0 / math.sqrt(dim),
                    partition_tokens=partition_tokens, q=q, seq_lens=seq_lens,
                    block_table=block_table, page_sel=page_sel, sel_lens=sel_lens,
                    page_k_off=page_k_off, page_v_off=page_v_off, page_codec=page_codec,
                    page_scale=page_scale, pool=pool, info=info)


def prefill_queries(seed: int, rows: int, tokens: int, hq: int, dim: int, q_scale: float = 1.0) -> np.ndarray:
    """float16 [rows, tokens, Hq, D]: the queries of a chunk of new tokens per
    row, N(0, q_scale^2) before rounding, from a stream of their own (the
    workload's streams are untouched)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x5052])))
    x = g.standard_normal((rows, tokens, hq, dim), dtype=np.float32)
    return (np.float32(q_scale) * x).astype(np.float16)
