"""Page encode (demotion) and token append, from their definitions.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

What the device path computes (the write side of the paged cache):

* Append. The new token's K and V (fp16 values, one vector per KV head) are
  stored in slot ``L mod P`` of logical page ``L // P`` of their row, L being
  the row's length before the append, in the page's own codec (FP16 or
  BF16). The newest page of a sequence stays in a 16-bit codec while it fills
  (ARGUS "Adaptive activation": recent pages stay FP16).
* Encode. A full FP16/BF16 page is re-encoded into a compact codec, the
  demotion of older pages to a cheaper tier (ARGUS "v0.5" and "Adaptive
  activation"; FreeToken PR #499 update, item 1: FP8 pages hold e4m3 codes
  plus fp32 scales; GGML Q8/Q4 pages with one scale per group of 32):

  - FP8: one fp32 scale per (page, KV head, plane),
    s = fp32(absmax / 448), or 1 for an all-zero block; the code is the e4m3
    value nearest to fp32(x / s), ties to the even code. |x / s| <= 448 up to
    the rounding of the division, and the quotient is clipped to +-448.
  - INT8 / INT4: one fp16 scale per (token, group of 32 dims),
    s = fp16(fp32(absmax) / qmax) with qmax 127 / 7, kept inside fp16's
    positive finite range [2^-24, 65504] (a tiny group's scale would round to
    0, a huge BF16 group's to infinity), or 1 for an all-zero group; the
    code is clip(rint(fp32(x) / fp32(s)), -qmax, qmax), rint rounding half
    to even.

  - INT2 (the 2-bit tier of ARGUS's cascade, taken as the unsigned-affine
    2-bit kind of its "Pluggable tiers"): per (token, group of 32 dims) an
    fp16 offset z = fp16(min) (clamped to +-65504) and an fp16 step
    s = fp16(fp32(max - z) / 3), kept inside [2^-24, 65504], or 1 when
    max - z <= 0; the code is u = clip(rint(fp32(x - z) / s), 0, 3) and
    denotes z + s*u.
  - BIT1 (the 1-bit tier): per (token, group of 32 dims) the sign bit
    b = [x < 0] and one fp16 scale s = fp16(fp32(mean |x|)), the mean of
    the 32 magnitudes taken exactly rounded in float64 (math.fsum; exact for
    16-bit inputs) and capped at 65504; b denotes (1 - 2b)*s. An all-zero
    group gets s = 0 and decodes to zeros.

  Every code is decided in fp32 (the division and the rounding), the
  precision the device path computes in.

Bytes are placed with ``layout.code_position`` (the library's in-page
layout). Pinned in tests/test_oracle_encode.py.
"""
from __future__ import annotations

import numpy as np

import math

from .codecs import decode_bf16, decode_fp8_e4m3, decode_fp16
from .layout import BITS, BF16, BIT1, FP8, FP16, INT2, INT4, INT8, code_bits, code_position

FP8_MAX = np.float32(448.0)
# Non-negative finite e4m3 values in code order 0x00 .. 0x7E (0x7F is NaN):
# the order of the codes is the order of the values.
_E4M3_POS = decode_fp8_e4m3(np.arange(0x7F))


def fp32_to_e4m3(y: np.ndarray) -> np.ndarray:
    """Codes (uint8) of the e4m3 values nearest to float32 ``y``, ties to the
    even code; |y| <= 448 and finite. The sign bit follows y (-0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    if np.any(~np.isfinite(a)) or np.any(a > 448.0):
        raise ValueError("fp32_to_e4m3 takes finite values with |y| <= 448")
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)   # exact hits
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def encode_block_fp8(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """x: float32 [P, D] (one page, one KV head, one plane).
    Returns (codes uint8 [P, D], fp32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x)))
    s = np.float32(1.0) if amax == 0 else np.float32(amax / FP8_MAX)
    y = np.clip((x / s).astype(np.float32), -FP8_MAX, FP8_MAX)
    return fp32_to_e4m3(y), s


def encode_groups_int(x: np.ndarray, qmax: int) -> tuple[np.ndarray, np.ndarray]:
    """x: float32 [P, D]; groups of 32 along D.
    Returns (codes int8 [P, D], scales float16 [P, D/32])."""
    x = np.asarray(x, dtype=np.float32)
    p, d = x.shape
    g = x.reshape(p, d // 32, 32)
    amax = np.max(np.abs(g), axis=-1).astype(np.float32)
    with np.errstate(over="ignore"):                      # a huge group's scale overflows, then is clamped
        s = (amax / np.float32(qmax)).astype(np.float32).astype(np.float16)
    s = np.minimum(np.maximum(s, np.float16(2.0 ** -24)), np.float16(65504.0))   # inside fp16's finite range
    s = np.where(amax == 0, np.float16(1.0), s)
    q = np.rint((g / s.astype(np.float32)[..., None]).astype(np.float32))
    return np.clip(q, -qmax, qmax).astype(np.int8).reshape(p, d), s


def encode_groups_affine2(x: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """x: float32 [P, D]; groups of 32 along D, one at a time.
    Returns (codes uint8 [P, D] in 0..3, scales float16 [P, D/32], offsets
    float16 [P, D/32])."""
    x = np.asarray(x, dtype=np.float32)
    p, d = x.shape
    codes = np.zeros((p, d), np.uint8)
    scales = np.zeros((p, d // 32), np.float16)
    offs = np.zeros((p, d // 32), np.float16)
    f16max = np.float16(65504.0)
    for t in range(p):
        for g in range(d // 32):
            v = x[t, 32 * g: 32 * g + 32]
            lo, hi = np.float32(v.min()), np.float32(v.max())
            with np.errstate(over="ignore"):
                z = np.float16(lo)
            z = min(max(z, -f16max), f16max)                     # a BF16 minimum beyond fp16 saturates
            z32 = np.float32(z)
            span = np.float32(hi - z32)
            if span > 0:
                with np.errstate(over="ignore"):
                    st = np.float16(np.float32(span / np.float32(3.0)))
                st = min(max(st, np.float16(2.0 ** -24)), f16max)
            else:
                st = np.float16(1.0)
            q = (v - z32).astype(np.float32) / np.float32(st)
            codes[t, 32 * g: 32 * g + 32] = np.clip(np.rint(q.astype(np.float32)), 0, 3).astype(np.uint8)
            scales[t, g], offs[t, g] = st, z
    return codes, scales, offs


def encode_groups_sign1(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x: float32 [P, D]; groups of 32 along D. Returns (bits uint8 [P, D],
    1 for x < 0; scales float16 [P, D/32] = fp16(fp32(mean |x|)), the mean
    exactly rounded in float64, capped at 65504)."""
    x = np.asarray(x, dtype=np.float32)
    p, d = x.shape
    bits = (x < 0).astype(np.uint8)
    scales = np.zeros((p, d // 32), np.float16)
    for t in range(p):
        for g in range(d // 32):
            mean = math.fsum(abs(float(a)) for a in x[t, 32 * g: 32 * g + 32]) / 32.0
            with np.errstate(over="ignore"):
                scales[t, g] = min(np.float16(np.float32(mean)), np.float16(65504.0))
    return bits, scales


def _plane_head_values(pool: np.ndarray, off: int, codec: int, hkv: int, P: int, D: int, h: int,
                       is_v: bool) -> np.ndarray:
    """float32 [P, D]: every slot of head h of a 16-bit plane (exact)."""
    hb = P * D * 2
    raw = pool[int(off) + h * hb: int(off) + (h + 1) * hb]
    pos, _ = code_position(P, D, codec, is_v)
    code = raw[pos].astype(np.int64) | (raw[pos + 1].astype(np.int64) << 8)
    val = decode_fp16(code) if codec == FP16 else decode_bf16(code)
    return val.astype(np.float32)


def _put_codes(pool: np.ndarray, off: int, codec: int, P: int, D: int, h: int, is_v: bool,
               codes: np.ndarray) -> None:
    """Store codes [P, D] of head h at their layout positions (in place)."""
    hb = P * D * BITS[codec] // 8
    base = int(off) + h * hb
    if codec in (INT2, BIT1):
        # several codes per byte: OR each into place at its bit
        bpos, shift = code_bits(P, D, codec, is_v)
        block = np.zeros(hb, dtype=np.uint64)
        vals = (codes.astype(np.uint64) & np.uint64((1 << BITS[codec]) - 1)) << shift.astype(np.uint64)
        np.bitwise_or.at(block, bpos.ravel(), vals.ravel())
        pool[base: base + hb] = block.astype(np.uint8)
        return
    pos, nib = code_position(P, D, codec, is_v)
    if codec in (FP16, BF16):
        c = codes.astype(np.uint16)
        pool[base + pos] = (c & 0xFF).astype(np.uint8)
        pool[base + pos + 1] = (c >> 8).astype(np.uint8)
    elif codec in (FP8, INT8):
        pool[base + pos] = codes.astype(np.int64).astype(np.uint8)
    else:
        # every byte of the head's codes holds two elements, one per nibble
        nibs = (codes.astype(np.int64) & 0xF).astype(np.uint8)
        block = np.zeros(hb, dtype=np.uint8)
        low = nib == 0
        block[pos[low]] |= nibs[low]
        block[pos[~low]] |= (nibs[~low] << 4).astype(np.uint8)
        pool[base: base + hb] = block


def _fp16_codes(x: np.ndarray, codec: int) -> np.ndarray:
    """float32 values exactly representable in fp16 -> FP16 or BF16 codes
    (BF16 by round to nearest even from the float32 bits)."""
    if codec == FP16:
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    bits = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)


def append_token(pool: np.ndarray, k_off: int, v_off: int, codec_byte: int, hkv: int, P: int, D: int,
                 slot: int, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Copy of ``pool`` with token ``slot`` of the page at (k_off, v_off) set
    to k, v (fp16 values [Hkv, D]); the page's codecs must be 16-bit."""
    kc, vc = codec_byte & 15, codec_byte >> 4
    if kc not in (FP16, BF16) or vc not in (FP16, BF16):
        raise ValueError("append needs FP16 or BF16 planes")
    out = pool.copy()
    for plane, off, c, val in ((False, k_off, kc, k), (True, v_off, vc, v)):
        pos, _ = code_position(P, D, c, plane)
        for h in range(hkv):
            code = _fp16_codes(np.asarray(val[h], dtype=np.float16).astype(np.float32), c)
            base = int(off) + h * P * D * 2
            pool_pos = base + pos[slot]
            out[pool_pos] = (code & 0xFF).astype(np.uint8)
            out[pool_pos + 1] = (code >> 8).astype(np.uint8)
    return out


def encode_page(pool: np.ndarray, src_k: int, src_v: int, src_codec: int, dst_k: int, dst_v: int,
                dst_codec: int, hkv: int, P: int, D: int) -> tuple[np.ndarray, np.ndarray]:
    """Copy of ``pool`` with the page at (dst_k, dst_v) holding the re-encoding
    of the 16-bit page at (src_k, src_v), and the FP8 scales [Hkv, 2] (K, V;
    1.0 for a plane in another codec). Codec bytes: K in the low nibble."""
    out = pool.copy()
    scales = np.ones((hkv, 2), dtype=np.float32)
    for i, (is_v, s_off, d_off) in enumerate(((False, src_k, dst_k), (True, src_v, dst_v))):
        sc = (src_codec >> 4) if is_v else (src_codec & 15)
        dc = (dst_codec >> 4) if is_v else (dst_codec & 15)
        if sc not in (FP16, BF16):
            raise ValueError("encode reads FP16 or BF16 planes")
        for h in range(hkv):
            x = _plane_head_values(pool, s_off, sc, hkv, P, D, h, is_v)
            if dc in (FP16, BF16):
                _put_codes(out, d_off, dc, P, D, h, is_v, _fp16_codes(x, dc))
            elif dc == FP8:
                codes, s = encode_block_fp8(x)
                _put_codes(out, d_off, dc, P, D, h, is_v, codes)
                scales[h, i] = s
            elif dc in (INT8, INT4, INT2, BIT1):
                z16 = None
                if dc in (INT8, INT4):
                    codes, s16 = encode_groups_int(x, 127 if dc == INT8 else 7)
                elif dc == INT2:
                    codes, s16, z16 = encode_groups_affine2(x)
                else:
                    codes, s16 = encode_groups_sign1(x)
                _put_codes(out, d_off, dc, P, D, h, is_v, codes)
                gb = P * (D // 32) * 2                           # bytes of one head's scales
                sc_off = int(d_off) + hkv * P * D * BITS[dc] // 8 + h * gb
                out[sc_off: sc_off + gb] = np.ascontiguousarray(s16).astype("<f2").view(np.uint8).ravel()
                if z16 is not None:                              # INT2 offsets after every head's scales
                    z_off = int(d_off) + hkv * P * D * BITS[dc] // 8 + hkv * gb + h * gb
                    out[z_off: z_off + gb] = np.ascontiguousarray(z16).astype("<f2").view(np.uint8).ravel()
            else:
                raise ValueError(f"unknown codec {dc}")
    return out, scales
