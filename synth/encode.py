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
* INT2  -- the 2-bit tier of ARGUS's cascade, as the unsigned-affine kind of
           its "Pluggable tiers" (``unsigned_affine``, bits = 2): per group of
           32 along head_dim an fp16 offset z (the group minimum) and an fp16
           step s = (max - z) / 3; codes u = clip(rint((x - z) / s), 0, 3),
           value z + s*u (see ``encode_affine2_g32``).
* BIT1  -- the 1-bit tier: sign bits with one fp16 scale per group of 32,
           s = mean |x|; bit 1 for x < 0, value (1 - 2*bit)*s.
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


def encode_affine2_g32(x: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """2-bit unsigned affine quantization per 32-group along the last axis,
    every step in float32: z = fp16(min) (clamped to fp16's finite range),
    d = max - z, s = fp16(d / 3) kept inside [2^-24, 65504] (1 when d <= 0),
    u = clip(rint((x - z) / s), 0, 3).

    Returns (codes uint8 [..., D], scales float16 [..., D/32], offsets
    float16 [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    g = x.reshape(*x.shape[:-1], d // 32, 32)
    lo, hi = g.min(axis=-1), g.max(axis=-1)
    with np.errstate(over="ignore"):
        z16 = np.clip(lo.astype(np.float16), np.float16(-65504.0), np.float16(65504.0))
    z32 = z16.astype(np.float32)
    span = (hi - z32).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = np.clip((span / np.float32(3.0)).astype(np.float32).astype(np.float16),
                      np.float16(2.0 ** -24), np.float16(65504.0))
    s16 = np.where(span > 0, s16, np.float16(1.0))
    s32 = s16.astype(np.float32)
    q = ((g - z32[..., None]).astype(np.float32) / s32[..., None]).astype(np.float32)
    u = np.clip(np.rint(q), 0, 3).astype(np.uint8)
    return u.reshape(x.shape), s16, z16


def encode_sign1_g32(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """1-bit sign quantization per 32-group along the last axis: bit = x < 0,
    s = fp16(fp32(sum |x| / 32)) with the sum taken in float64 (exact for
    16-bit inputs), capped at 65504. Returns (bits uint8 [..., D], scales
    float16 [..., D/32])."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    g = x.reshape(*x.shape[:-1], d // 32, 32)
    mean = (np.abs(g).astype(np.float64).sum(axis=-1) / 32.0).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = np.minimum(mean.astype(np.float16), np.float16(65504.0))
    bits = (g < 0).astype(np.uint8)
    return bits.reshape(x.shape), s16


def pack_subbyte(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack unsigned ``bits``-bit codes (2 or 1) of each lane's run along the
    last axis. The run is cut into units of min(32, run bits) bits holding m
    codes each; code r of a unit goes to slot (r % 2) * (m / 2) + r // 2
    (bits * slot .. bits * slot + bits - 1): even codes fill the low half of
    the unit and odd codes the high half, each half in order. Units are
    little-endian."""
    c = np.asarray(codes).astype(np.uint64) & np.uint64((1 << bits) - 1)
    *lead, n = c.shape
    m = min(32 // bits, n)
    unit_bytes = m * bits // 8
    g = c.reshape(*lead, n // m, m)
    word = np.zeros((*lead, n // m), dtype=np.uint64)
    for r in range(m):
        word |= g[..., r] << np.uint64(bits * ((r % 2) * (m // 2) + r // 2))
    out = np.zeros((*lead, n // m, unit_bytes), dtype=np.uint8)
    for b in range(unit_bytes):
        out[..., b] = ((word >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
    return out.reshape(*lead, n // m * unit_bytes)
