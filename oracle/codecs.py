"""Codec values from their definitions, as float64.

Each decoder maps raw codes to the real number the code denotes; scales are
applied by the caller. Pinned in tests/test_oracle_codecs.py against library
conversions (numpy float16, torch bfloat16 and float8_e4m3fn) over every code,
and against brute-force integer enumeration for INT8/INT4.
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
    """Bytes holding two two's-complement nibbles; element 2k is the low nibble
    of byte k. Returns twice as many values as bytes, in element order."""
    u = np.asarray(packed).astype(np.int64) & 0xFF
    lo, hi = u & 0xF, (u >> 4) & 0xF
    out = np.empty(u.shape[:-1] + (u.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.float64)
