"""Copies a generated workload into device memory (torch used for memory only).

Byte ranges of the pool that hold no generated page are filled with random
filler bytes from their own seeded device generator; nothing may read them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from .workload import Workload

FILLER_SEED = 0x5EED


@dataclasses.dataclass
class DeviceWorkload:
    w: Workload
    q: torch.Tensor
    pool: torch.Tensor
    page_k_off: torch.Tensor
    page_v_off: torch.Tensor
    page_codec: torch.Tensor
    page_scale: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    page_sel: Optional[torch.Tensor]
    sel_lens: Optional[torch.Tensor]

    def args(self, pool: Optional[torch.Tensor] = None):
        """Positional tensors of decode_attention after the params."""
        return (self.q, self.pool if pool is None else pool, self.page_k_off, self.page_v_off,
                self.page_codec, self.page_scale, self.block_table, self.seq_lens,
                self.page_sel, self.sel_lens)


def _t(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def upload_pool(w: Workload, device, filler_seed: int = FILLER_SEED) -> torch.Tensor:
    pool = torch.empty(w.pool.nbytes, dtype=torch.uint8, device=device)
    if pool.data_ptr() % 256:
        raise RuntimeError("device pool not 256-byte aligned")
    if w.pool.is_dense:
        pool.copy_(torch.from_numpy(w.pool.as_array()))
        return pool
    gen = torch.Generator(device=device)
    gen.manual_seed(filler_seed)
    step = 1 << 28
    for off in range(0, pool.numel(), step):
        n = min(step, pool.numel() - off)
        pool[off:off + n] = torch.randint(0, 256, (n,), dtype=torch.uint8, device=device, generator=gen)
    segs = w.pool.segments()
    sizes = {d.size for _, d in segs}
    if len(sizes) == 1:
        size = sizes.pop()
        offs = np.array([o for o, _ in segs], dtype=np.int64)
        if np.all(offs % size == 0) and pool.numel() % size == 0:
            blocks = torch.from_numpy(np.stack([d for _, d in segs])).to(device)
            idx = torch.from_numpy(offs // size).to(device)
            pool.view(-1, size).index_copy_(0, idx, blocks)
            return pool
    for off, d in segs:
        pool[off:off + d.size].copy_(torch.from_numpy(d))
    return pool


def to_device(w: Workload, device="cuda") -> DeviceWorkload:
    dev = torch.device(device)
    return DeviceWorkload(
        w=w, q=_t(w.q, dev), pool=upload_pool(w, dev),
        page_k_off=_t(w.page_k_off.astype(np.uint64), dev),
        page_v_off=_t(w.page_v_off.astype(np.uint64), dev),
        page_codec=_t(w.page_codec, dev), page_scale=_t(w.page_scale, dev),
        block_table=_t(w.block_table, dev), seq_lens=_t(w.seq_lens, dev),
        page_sel=None if w.page_sel is None else _t(w.page_sel, dev),
        sel_lens=None if w.sel_lens is None else _t(w.sel_lens, dev))
