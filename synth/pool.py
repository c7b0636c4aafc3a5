"""Host-side byte arena holding the encoded pages, possibly sparsely.

A pool is ``nbytes`` long; only some byte ranges (segments) carry generated
pages. Ranges outside every segment are filler that nothing may read: the
device copy fills them with random bytes (which include FP8 NaN codes) so a
stray read shows up as a wrong or non-finite result.
"""
from __future__ import annotations

import bisect

import numpy as np


class Pool:
    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self._offs: list[int] = []
        self._data: list[np.ndarray] = []

    # -- building ---------------------------------------------------------
    def add_segment(self, offset: int, data: np.ndarray) -> None:
        data = np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)
        assert 0 <= offset and offset + data.size <= self.nbytes
        i = bisect.bisect_left(self._offs, offset)
        if i > 0:
            assert self._offs[i - 1] + self._data[i - 1].size <= offset, "overlap"
        if i < len(self._offs):
            assert offset + data.size <= self._offs[i], "overlap"
        self._offs.insert(i, int(offset))
        self._data.insert(i, data)

    @classmethod
    def dense(cls, data: np.ndarray) -> "Pool":
        p = cls(data.size)
        p.add_segment(0, data)
        return p

    # -- reading ----------------------------------------------------------
    def read(self, offset: int, n: int) -> np.ndarray:
        """Bytes [offset, offset+n); they must lie inside one segment."""
        i = bisect.bisect_right(self._offs, offset) - 1
        if i < 0:
            raise IndexError(f"pool read at {offset} outside written data")
        rel = offset - self._offs[i]
        seg = self._data[i]
        if rel + n > seg.size:
            raise IndexError(f"pool read [{offset}, {offset + n}) outside written data")
        return seg[rel:rel + n]

    def segments(self):
        return list(zip(self._offs, self._data))

    @property
    def is_dense(self) -> bool:
        return len(self._offs) == 1 and self._offs[0] == 0 and self._data[0].size == self.nbytes

    def as_array(self) -> np.ndarray:
        if self.is_dense:
            return self._data[0]
        out = np.zeros(self.nbytes, dtype=np.uint8)
        for off, d in self.segments():
            out[off:off + d.size] = d
        return out

    def copy(self) -> "Pool":
        p = Pool(self.nbytes)
        p._offs = list(self._offs)
        p._data = [d.copy() for d in self._data]
        return p
