"""Reads one (page, KV head) plane from the byte arena as float64 values.

In-page layout being read (the library's own definition; the pages give codec
semantics, not a bit layout). A plane is the codes of every KV head, head
after head, then -- for INT8/INT4 only -- fp16 group scales
``[Hkv][P][D/32]`` (token-major). One head's codes are P/16 tiles of 16
tokens, each TB = 16*D*bits/8 bytes. Inside a tile, each of 64 "lanes" owns
a run of R = TB/64 bytes:

* K, codecs with one scale per page (FP16, BF16, FP8): lane 16*kq + t holds
  token t, dims (D/4)*kq + e, e = 0 .. D/4-1 (run element e);
* K, group-scale codecs (INT8, INT4): lane 16*kq + t holds token t, dims
  32*c + 8*kq + j as run element e = 8*c + j;
* V (all codecs): lane 16*qd + c holds tokens 4*qd + j and dims 16*n + c as
  run element e = 4*n + j.

* K of the other group-scale codecs (INT2, BIT1): as INT8/INT4.

Run element e occupies run bytes e*bits/8 for 8- and 16-bit codes. Codes of
fewer bits fill the run in units of U = min(32, run bits) bits, m = U / bits
codes each: code r = e % m of unit e // m sits at slot (r % 2)*(m/2) + r // 2,
bits*slot .. bits*slot + bits - 1 of the little-endian unit (INT4: eight
codes per 32-bit word; INT2: sixteen; BIT1: thirty-two, or sixteen in a
16-bit unit when the run is 2 bytes). Run byte rb of lane L is stored at tile
offset (rb // 16)*1024 + 16*L + rb % 16 when R >= 16, else at R*L + rb.

After the codes of every head, the group-scale codecs (INT8, INT4, INT2,
BIT1) hold fp16 scales [Hkv][P][D/32]; INT2 then holds fp16 offsets
[Hkv][P][D/32]. Values: INT8/INT4 c*s; INT2 z + s*u (u = 0..3, the unsigned
affine 2-bit kind); BIT1 (1 - 2*b)*s.

Pinned in tests/test_oracle_layout.py by hand-placed single codes.
"""
from __future__ import annotations

import functools

import numpy as np

from .codecs import decode_bf16, decode_bit1, decode_fp8_e4m3, decode_fp16, decode_int8, decode_uint2

FP16, BF16, FP8, INT8, INT4, INT2, BIT1 = 0, 1, 2, 3, 4, 5, 6
BITS = {FP16: 16, BF16: 16, FP8: 8, INT8: 8, INT4: 4, INT2: 2, BIT1: 1}
GROUP_SCALED = (INT8, INT4, INT2, BIT1)
_FP8_TABLE = decode_fp8_e4m3(np.arange(256))
_INT8_TABLE = decode_int8(np.arange(256))
_INT4_TABLE = np.array([v - 16 if v >= 8 else v for v in range(16)], dtype=np.float64)


def _read(pool, off: int, n: int) -> np.ndarray:
    if isinstance(pool, np.ndarray):
        if off < 0 or off + n > pool.size:
            raise IndexError("pool read out of range")
        return pool[off:off + n]
    return pool.read(off, n)


@functools.lru_cache(maxsize=None)
def code_bits(P: int, D: int, codec: int, is_v: bool):
    """Byte offset inside one head's codes of element (t, i), shape [P, D],
    and the bit where its code starts inside that byte (0 for codes of 8
    bits or more); read-only."""
    bits = BITS[codec]
    t = np.arange(P)[:, None]
    i = np.arange(D)[None, :]
    tile, tt = t // 16, t % 16
    if is_v:
        lane = 16 * (tt // 4) + i % 16
        e = 4 * (i // 16) + tt % 4
    elif codec in GROUP_SCALED:
        lane = 16 * ((i % 32) // 8) + tt
        e = 8 * (i // 32) + i % 8
    else:
        lane = 16 * (i // (D // 4)) + tt
        e = i % (D // 4)
    tb = 16 * D * bits // 8
    run = tb // 64
    if bits < 8:
        unit = min(32, run * 8)
        m = unit // bits
        r = e % m
        bitpos = (e // m) * unit + bits * ((r % 2) * (m // 2) + r // 2)
        rb, shift = bitpos // 8, bitpos % 8
    else:
        rb, shift = e * (bits // 8), 0 * e
    if run >= 16:
        off = tile * tb + (rb // 16) * 1024 + 16 * lane + rb % 16
    else:
        off = tile * tb + run * lane + rb
    off = np.broadcast_to(off, (P, D)).copy()
    shift = np.broadcast_to(shift, (P, D)).copy()
    off.setflags(write=False)
    shift.setflags(write=False)
    return off, shift


@functools.lru_cache(maxsize=None)
def code_position(P: int, D: int, codec: int, is_v: bool):
    """Byte offset inside one head's codes of element (t, i), shape [P, D],
    and for INT4 the nibble (0 = bits 0..3, 1 = bits 4..7); read-only. For
    INT2 and BIT1 use ``code_bits``."""
    if codec in (INT2, BIT1):
        raise ValueError("codes of fewer than four bits: use code_bits")
    bits = BITS[codec]
    t = np.arange(P)[:, None]
    i = np.arange(D)[None, :]
    tile, tt = t // 16, t % 16
    if is_v:
        lane = 16 * (tt // 4) + i % 16
        e = 4 * (i // 16) + tt % 4
    elif codec in (INT8, INT4):
        lane = 16 * ((i % 32) // 8) + tt
        e = 8 * (i // 32) + i % 8
    else:
        lane = 16 * (i // (D // 4)) + tt
        e = i % (D // 4)
    tb = 16 * D * bits // 8
    run = tb // 64
    nib = None
    if bits == 4:
        r = e % 8
        slot = (r % 2) * 4 + r // 2
        rb = 4 * (e // 8) + slot // 2
        nib = np.broadcast_to(slot % 2, (P, D)).copy()
        nib.setflags(write=False)
    else:
        rb = e * (bits // 8)
    if run >= 16:
        off = tile * tb + (rb // 16) * 1024 + 16 * lane + rb % 16
    else:
        off = tile * tb + run * lane + rb
    off = np.broadcast_to(off, (P, D)).copy()
    off.setflags(write=False)
    return off, nib


def plane_values(pool, off: int, codec: int, hkv: int, P: int, D: int, h: int,
                 fp8_scale: float, is_v: bool, valid: int) -> np.ndarray:
    """float64 [valid, D]: the first ``valid`` tokens of head ``h``."""
    if codec not in BITS:
        raise ValueError(f"unknown codec {codec}")
    head_bytes = P * D * BITS[codec] // 8
    raw = _read(pool, int(off) + h * head_bytes, head_bytes)
    pos, nib = code_position(P, D, codec, is_v) if codec not in (INT2, BIT1) else (None, None)
    pos = None if pos is None else pos[:valid]
    if codec in (FP16, BF16):
        code = raw[pos].astype(np.int64) | (raw[pos + 1].astype(np.int64) << 8)
        x = decode_fp16(code) if codec == FP16 else decode_bf16(code)
    elif codec == FP8:
        x = _FP8_TABLE[raw[pos]]
    elif codec == INT8:
        x = _INT8_TABLE[raw[pos]]
    elif codec == INT4:
        x = _INT4_TABLE[(raw[pos] >> (4 * nib[:valid])) & 0xF]
    elif codec == INT2:
        bpos, shift = code_bits(P, D, codec, is_v)
        x = decode_uint2((raw[bpos[:valid]] >> shift[:valid]) & 0x3)
    else:
        bpos, shift = code_bits(P, D, codec, is_v)
        x = decode_bit1((raw[bpos[:valid]] >> shift[:valid]) & 0x1)
    if codec == FP8:
        x = x * float(fp8_scale)
    elif codec in GROUP_SCALED:
        groups = P * (D // 32) * 2                       # bytes of one head's scales
        sc_off = int(off) + hkv * head_bytes + h * groups
        sc = decode_fp16(_read(pool, sc_off, groups).view("<u2")).reshape(P, D // 32)
        x = x * np.repeat(sc[:valid], 32, axis=1)
        if codec == INT2:
            z_off = int(off) + hkv * head_bytes + hkv * groups + h * groups
            z = decode_fp16(_read(pool, z_off, groups).view("<u2")).reshape(P, D // 32)
            x = x + np.repeat(z[:valid], 32, axis=1)
    return x
