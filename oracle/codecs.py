"""Codec values from their definitions, as float64.

Each decoder maps raw codes to the real number the code denotes; scales
(and the INT2 offsets) are applied by the caller. Pinned in
tests/test_oracle_codecs.py against library conversions (numpy float16, torch
bfloat16 and float8_e4m3fn) over every code, and against brute-force integer
enumeration for INT8/INT4/INT2/BIT1.
"""
from __future__ import annotations

import numpy as np


def _sign(bit: np.ndarray) -> np.ndarray:
    return np.where(bit != 0, -1.0, 1.0)


def decode_fp16(codes: np.ndarray) -> np.ndarray:
    """IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits."""
    u = np.asarray(codes).astype(np.int64)
    s, e, m = (u >> 15) & 1, (u >> 10) & 0x1F, u & 0x3FF
    sub = np.ldexp(m / 1024.0, -14)
    nor = np.ldexp(1.0 + m / 1024.0, (e - 15).astype(np.int64))
    val = np.where(e == 0, sub, nor)
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return _sign(s) * val


def decode_bf16(codes: np.ndarray) -> np.ndarray:
    """bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits."""
    u = np.asarray(codes).astype(np.int64)
    s, e, m = (u >> 15) & 1, (u >> 7) & 0xFF, u & 0x7F
    sub = np.ldexp(m / 128.0, -126)
    nor = np.ldexp(1.0 + m / 128.0, (e - 127).astype(np.int64))
    val = np.where(e == 0, sub, nor)
    val = np.where(e == 255, np.where(m == 0, np.inf, np.nan), val)
    return _sign(s) * val


def decode_fp8_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;
    exponent 15 with mantissa 7 is NaN (so the largest finite value is 448)."""
    u = np.asarray(codes).astype(np.int64)
    s, e, m = (u >> 7) & 1, (u >> 3) & 0xF, u & 0x7
    sub = np.ldexp(m / 8.0, -6)
    nor = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    val = np.where(e == 0, sub, nor)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return _sign(s) * val


def decode_int8(codes: np.ndarray) -> np.ndarray:
    """Two's-complement byte."""
    u = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(u >= 128, u - 256, u).astype(np.float64)


def decode_int4(packed: np.ndarray) -> np.ndarray:
    """Bytes holding two's-complement nibbles, eight per 32-bit little-endian
    word: element r (0..7) of each word sits at nibble slot (r % 2)*4 + r//2,
    slot s being bits 4s..4s+3. Returns two values per byte, in element order."""
    u = np.asarray(packed).astype(np.int64) & 0xFF
    *lead, nb = u.shape
    assert nb % 4 == 0
    b = u.reshape(*lead, nb // 4, 4)
    word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    out = np.empty((*lead, nb // 4, 8), dtype=np.int64)
    for r in range(8):
        out[..., r] = (word >> (4 * ((r % 2) * 4 + r // 2))) & 0xF
    out = np.where(out >= 8, out - 16, out)
    return out.reshape(*lead, nb * 2).astype(np.float64)


def decode_uint2(codes: np.ndarray) -> np.ndarray:
    """Unsigned 2-bit code u in 0..3 (the step count of the unsigned affine
    kind, ARGUS "Pluggable tiers": value = offset + scale * u)."""
    u = np.asarray(codes).astype(np.int64)
    if np.any((u < 0) | (u > 3)):
        raise ValueError("2-bit codes are 0..3")
    return u.astype(np.float64)


def decode_bit1(bits: np.ndarray) -> np.ndarray:
    """1-bit sign code: 0 -> +1, 1 -> -1 (times the group scale)."""
    b = np.asarray(bits).astype(np.int64)
    if np.any((b < 0) | (b > 1)):
        raise ValueError("1-bit codes are 0 or 1")
    return np.where(b == 1, -1.0, 1.0)
