"""Reads one (page, KV head) plane from the byte arena as float64 values.

In-page layout being read (the library's own definition; the pages give codec
semantics, not a bit layout): a plane is the codes of every KV head, head by
head, then -- for INT8/INT4 only -- fp16 group scales ``[Hkv][P][D/32]``.
Within one head's codes, element (t, i) sits at element index

* K:  t*D + i;
* V:  (t // 16)*16*D + ((t % 16)//4 * 16 + i % 16) * (D//16) * 4
      + (i // 16) * 4 + t % 4;

and INT4 packs eight elements per 32-bit little-endian word: element e is in
word e // 8 at nibble slot (r % 2)*4 + r // 2 with r = e % 8 (even elements
in the low half-word, odd ones in the high half-word).
Pinned in tests/test_oracle_layout.py by hand-placed single codes.
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_bf16, decode_fp8_e4m3, decode_fp16, decode_int4, decode_int8

FP16, BF16, FP8, INT8, INT4 = 0, 1, 2, 3, 4
BITS = {FP16: 16, BF16: 16, FP8: 8, INT8: 8, INT4: 4}
_FP8_TABLE = decode_fp8_e4m3(np.arange(256))
_INT8_TABLE = decode_int8(np.arange(256))


def _read(pool, off: int, n: int) -> np.ndarray:
    if isinstance(pool, np.ndarray):
        if off < 0 or off + n > pool.size:
            raise IndexError("pool read out of range")
        return pool[off:off + n]
    return pool.read(off, n)


def element_index(P: int, D: int, is_v: bool) -> np.ndarray:
    """[P, D] element index of (t, i) inside one head's codes."""
    t = np.arange(P)[:, None]
    i = np.arange(D)[None, :]
    if not is_v:
        return t * D + i
    return ((t // 16) * 16 * D + ((t % 16) // 4 * 16 + i % 16) * (D // 16) * 4
            + (i // 16) * 4 + t % 4)


def plane_values(pool, off: int, codec: int, hkv: int, P: int, D: int, h: int,
                 fp8_scale: float, is_v: bool, valid: int) -> np.ndarray:
    """float64 [valid, D]: the first ``valid`` tokens of head ``h``."""
    if codec not in BITS:
        raise ValueError(f"unknown codec {codec}")
    head_bytes = P * D * BITS[codec] // 8
    raw = _read(pool, int(off) + h * head_bytes, head_bytes)
    if codec == FP16:
        vals = decode_fp16(raw.view("<u2"))
    elif codec == BF16:
        vals = decode_bf16(raw.view("<u2"))
    elif codec == FP8:
        vals = _FP8_TABLE[raw]
    elif codec == INT8:
        vals = _INT8_TABLE[raw]
    else:
        vals = decode_int4(raw)
    x = vals[element_index(P, D, is_v)[:valid]]
    if codec == FP8:
        x = x * float(fp8_scale)
    elif codec in (INT8, INT4):
        sc_off = int(off) + hkv * head_bytes + h * P * (D // 32) * 2
        sc = decode_fp16(_read(pool, sc_off, P * (D // 32) * 2).view("<u2")).reshape(P, D // 32)
        x = x * np.repeat(sc[:valid], 32, axis=1)
    return x
