"""Encoders that turn float values into page codes (input preparation only).

These produce the bytes that both the HIP path and the oracle read. They
quantize; they never decode, and nothing here computes attention.

Codec definitions (ARGUS page, "v0.5" and "Direct paged attention": FP16/BF16
pages plus GGML-style Q8/Q4 pages; FreeToken PR #499 update: FP8 pages hold
e4m3 codes plus fp32 scales):

* FP16  -- IEEE binary16, round to nearest even.
* BF16  -- top half of binary32, round to nearest even.
* FP8   -- OCP E4M3FN codes of x / s, s = absmax / 448 (fp32) per
           (page, kv head, K|V) block, saturated to +-448 before the cast.
* INT8  -- symmetric groups of 32 along head_dim: s = fp16(absmax / 127),
           c = clip(rint(x / s), -127, 127).
* INT4  -- as INT8 with 7 in place of 127; two's-complement nibbles packed
           eight to a 32-bit word (see ``pack_int4``).
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0


def encode_fp16(x: np.ndarray) -> np.ndarray:
    """float -> binary16 codes as uint16."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 codes (uint16), round to nearest even (finite x)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = 0x7FFF + ((bits >> 16) & 1)
    return ((bits + rounding) >> 16).astype(np.uint16)


def encode_int_g32(x: np.ndarray, qmax: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric per-32-group quantization along the last axis.

    Returns (codes int8 [..., D], scales float16 [..., D/32]).
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    assert d % 32 == 0
    g = x.reshape(*x.shape[:-1], d // 32, 32)
    amax = np.max(np.abs(g), axis=-1)
    with np.errstate(over="ignore"):
        s16 = (amax / np.float32(qmax)).astype(np.float16)
    # kept inside fp16's positive finite range; an all-zero group gets 1
    s16 = np.clip(s16, np.float16(2.0 ** -24), np.float16(65504.0))
    s16 = np.where(amax == 0, np.float16(1.0), s16)
    s32 = s16.astype(np.float32)[..., None]
    c = np.clip(np.rint(g / s32), -qmax, qmax).astype(np.int8)
    return c.reshape(x.shape), s16


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Pack int4 values (int8 in [-8, 7]) along the last axis, 8 per 32-bit
    little-endian word: element r of each group of 8 goes to nibble slot
    (r % 2) * 4 + r // 2 (bits 4*slot .. 4*slot+3), i.e. the even elements
    fill the low half-word and the odd ones the high half-word, in order."""
    c = (np.asarray(codes).astype(np.int64) & 0xF).astype(np.uint32)
    *lead, n = c.shape
    assert n % 8 == 0
    g = c.reshape(*lead, n // 8, 8)
    word = np.zeros((*lead, n // 8), dtype=np.uint32)
    for r in range(8):
        word |= g[..., r] << np.uint32(4 * ((r % 2) * 4 + r // 2))
    return word.astype("<u4").view(np.uint8).reshape(*lead, n // 2)
