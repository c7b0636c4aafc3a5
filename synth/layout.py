"""Writes physical pages (all KV heads) into their K and V planes.

In-page layout (this library's own definition; the pages fix codec semantics
but no bit layout). A plane is ``codes[Hkv][...]`` followed, for INT8/INT4, by
``scales[Hkv][P][D/32]`` fp16 (token-major, one scale per 32 dims).

One head's codes are P/16 tiles of 16 tokens. A tile is stored as the image
of 64 lanes' registers: lane L owns a run of R = tile_bytes / 64 bytes, and
for R >= 16 the runs are interleaved in 16-byte chunks (chunk i of every
lane, lane after lane, then chunk i+1), so each 16-byte-per-lane load covers
1 KB of consecutive bytes. Which elements a lane's run holds:

* K, one scale per page (FP16/BF16/FP8): lane 16*kq + t = token t, dims
  (D/4)*kq .. (D/4)*kq + D/4 - 1;
* K, group scales (INT8/INT4): lane 16*kq + t = token t, dims 32*c + 8*kq + j
  in the order (c, j);
* V: lane 16*qd + c = tokens 4*qd + j and dims 16*n + c in the order (n, j).

INT4 packs 8 elements per 32-bit word: even elements in the low half-word,
odd elements in the high half-word, each half in element order. INT2 and
BIT1 follow the same rule with 16 and 32 elements per word (a 16-bit unit
for BIT1 at head_dim 64, whose runs are 2 bytes). INT2 and BIT1 use the
grouped K order of INT8/INT4; INT2 planes hold fp16 offsets
``[Hkv][P][D/32]`` after the scales.
"""
from __future__ import annotations

import numpy as np
import torch

from .encode import (FP8_MAX, encode_affine2_g32, encode_bf16, encode_fp16, encode_int_g32, encode_sign1_g32,
                     pack_int4, pack_subbyte)

FP16, BF16, FP8, INT8, INT4, INT2, BIT1 = 0, 1, 2, 3, 4, 5, 6
CODECS = (FP16, BF16, FP8, INT8, INT4, INT2, BIT1)
GROUPED = (INT8, INT4, INT2, BIT1)
CODEC_NAMES = {FP16: "fp16", BF16: "bf16", FP8: "fp8_e4m3", INT8: "int8_g32", INT4: "int4_g32",
               INT2: "int2_affine_g32", BIT1: "bit1_g32"}
CODEC_BITS = {FP16: 16, BF16: 16, FP8: 8, INT8: 8, INT4: 4, INT2: 2, BIT1: 1}
PLANE_ALIGN = 256


def codes_bytes(codec: int, hkv: int, page: int, dim: int) -> int:
    return hkv * page * dim * CODEC_BITS[codec] // 8


def scale_bytes(codec: int, hkv: int, page: int, dim: int) -> int:
    """Group scales (and, for INT2, the group offsets after them)."""
    per = hkv * page * (dim // 32) * 2
    return 2 * per if codec == INT2 else (per if codec in GROUPED else 0)


def plane_bytes(codec: int, hkv: int, page: int, dim: int) -> int:
    return codes_bytes(codec, hkv, page, dim) + scale_bytes(codec, hkv, page, dim)


def align(n: int, a: int = PLANE_ALIGN) -> int:
    return (n + a - 1) // a * a


def lane_runs(x: np.ndarray, is_v: bool, grouped: bool) -> np.ndarray:
    """[..., P, D] natural values -> [..., P/16, 64, D/4]: per tile, per lane,
    the lane's run of elements."""
    *lead, p, d = x.shape
    nl = len(lead)
    ax = list(range(nl))
    if is_v:
        y = x.reshape(*lead, p // 16, 4, 4, d // 16, 16)           # tile, qd, j, n, c
        y = y.transpose(*ax, nl, nl + 1, nl + 4, nl + 3, nl + 2)    # tile, qd, c, n, j
    elif grouped:
        y = x.reshape(*lead, p // 16, 16, d // 32, 4, 8)           # tile, t, c, kq, j
        y = y.transpose(*ax, nl, nl + 3, nl + 1, nl + 2, nl + 4)    # tile, kq, t, c, j
    else:
        y = x.reshape(*lead, p // 16, 16, 4, d // 4)               # tile, t, kq, e
        y = y.transpose(*ax, nl, nl + 2, nl + 1, nl + 3)            # tile, kq, t, e
    return y.reshape(*lead, p // 16, 64, d // 4)


def interleave_chunks(b: np.ndarray) -> np.ndarray:
    """Run bytes [..., T, 64, R] -> [..., T*64*R]: for R >= 16 chunk i of all
    64 lanes is stored before chunk i+1."""
    *lead, t, lanes, r = b.shape
    if r >= 16:
        b = b.reshape(*lead, t, lanes, r // 16, 16).swapaxes(-3, -2)
    return np.ascontiguousarray(b).reshape(*lead, t * lanes * r)


def fp8_scales(x: np.ndarray) -> np.ndarray:
    """fp32 absmax/448 per block over the last two axes (1.0 for all-zero)."""
    amax = np.max(np.abs(x), axis=(-2, -1)).astype(np.float32)
    s = (amax / np.float32(FP8_MAX)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def encode_plane(x: np.ndarray, codec: int, v_order: bool) -> tuple[np.ndarray, np.ndarray]:
    """x: float32 [n, Hkv, P, D] for n pages.

    Returns (plane bytes uint8 [n, plane_bytes], fp8 scales float32 [n, Hkv];
    the scales are 1.0 for codecs other than FP8).
    """
    n, hkv, p, d = x.shape
    ones = np.ones((n, hkv), dtype=np.float32)
    grouped = codec in GROUPED

    def place(codes_elems: np.ndarray) -> np.ndarray:
        runs = lane_runs(codes_elems, v_order, grouped)              # [n, Hkv, T, 64, D/4]
        if codec == INT4:
            rb = pack_int4(runs)                                      # [..., D/8] bytes
        elif codec in (INT2, BIT1):
            rb = pack_subbyte(runs, CODEC_BITS[codec])                # [..., D*bits/32] bytes
        else:
            rb = np.ascontiguousarray(runs).view(np.uint8)            # little-endian bytes
        return interleave_chunks(rb).reshape(n, -1)

    if codec in (FP16, BF16):
        enc = encode_fp16 if codec == FP16 else encode_bf16
        return place(enc(x).astype("<u2")), ones
    if codec == FP8:
        s = fp8_scales(x)
        y = np.clip(x / s[..., None, None], -FP8_MAX, FP8_MAX).astype(np.float32)
        codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
        return place(codes.view(torch.uint8).numpy()), s
    if codec in (INT8, INT4):
        qmax = 127 if codec == INT8 else 7
        codes, scales = encode_int_g32(x, qmax)
        body = place(codes)
        sc = np.ascontiguousarray(scales).astype("<f2").view(np.uint8)
        return np.concatenate([body, sc.reshape(n, -1)], axis=1), ones
    if codec == INT2:
        codes, scales, offs = encode_affine2_g32(x)
        sc = np.ascontiguousarray(scales).astype("<f2").view(np.uint8).reshape(n, -1)
        zo = np.ascontiguousarray(offs).astype("<f2").view(np.uint8).reshape(n, -1)
        return np.concatenate([place(codes), sc, zo], axis=1), ones
    if codec == BIT1:
        codes, scales = encode_sign1_g32(x)
        sc = np.ascontiguousarray(scales).astype("<f2").view(np.uint8).reshape(n, -1)
        return np.concatenate([place(codes), sc], axis=1), ones
    raise ValueError(f"unknown codec {codec}")
