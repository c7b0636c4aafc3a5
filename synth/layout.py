"""Writes physical pages (all KV heads) into their K and V planes.

In-page layout (this library's own definition; the pages fix codec semantics
but no bit layout). For a page of P tokens, Hkv heads and head_dim D, each
plane is ``codes[Hkv][...]`` followed, for INT8/INT4, by
``scales[Hkv][P][D/32]`` fp16 (token-major, one scale per 32 dims).

* K codes, per head: token-major rows, element (t, i) at element index t*D + i.
* V codes, per head: 16-token tiles; inside a tile the element order is
  (token quad qd, dim-in-block c, dim block n, token-in-quad j) with
  t = 16*tile + 4*qd + j and i = 16*n + c.
* INT4 packs 8 elements per 32-bit word: even elements in the low half-word,
  odd elements in the high half-word, each half in element order.
"""
from __future__ import annotations

import numpy as np
import torch

from .encode import FP8_MAX, encode_bf16, encode_fp16, encode_int_g32, pack_int4

FP16, BF16, FP8, INT8, INT4 = 0, 1, 2, 3, 4
CODECS = (FP16, BF16, FP8, INT8, INT4)
CODEC_NAMES = {FP16: "fp16", BF16: "bf16", FP8: "fp8_e4m3", INT8: "int8_g32", INT4: "int4_g32"}
CODEC_BITS = {FP16: 16, BF16: 16, FP8: 8, INT8: 8, INT4: 4}
PLANE_ALIGN = 256


def codes_bytes(codec: int, hkv: int, page: int, dim: int) -> int:
    return hkv * page * dim * CODEC_BITS[codec] // 8


def scale_bytes(codec: int, hkv: int, page: int, dim: int) -> int:
    return hkv * page * (dim // 32) * 2 if codec in (INT8, INT4) else 0


def plane_bytes(codec: int, hkv: int, page: int, dim: int) -> int:
    return codes_bytes(codec, hkv, page, dim) + scale_bytes(codec, hkv, page, dim)


def align(n: int, a: int = PLANE_ALIGN) -> int:
    return (n + a - 1) // a * a


def v_tile_order(x: np.ndarray) -> np.ndarray:
    """[..., P, D] natural values -> [..., P*D] in the V tile order."""
    *lead, p, d = x.shape
    assert p % 16 == 0 and d % 16 == 0
    y = x.reshape(*lead, p // 16, 4, 4, d // 16, 16)          # tile, qd, j, n, c
    nl = len(lead)
    perm = list(range(nl)) + [nl + 0, nl + 1, nl + 4, nl + 3, nl + 2]  # tile, qd, c, n, j
    return y.transpose(perm).reshape(*lead, p * d)


def _k_order(x: np.ndarray) -> np.ndarray:
    return x.reshape(*x.shape[:-2], x.shape[-2] * x.shape[-1])


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
    order = v_tile_order if v_order else _k_order
    ones = np.ones((n, hkv), dtype=np.float32)
    if codec in (FP16, BF16):
        enc = encode_fp16 if codec == FP16 else encode_bf16
        body = np.ascontiguousarray(order(enc(x))).astype("<u2").view(np.uint8)
        return body.reshape(n, -1), ones
    if codec == FP8:
        s = fp8_scales(x)
        y = np.clip(x / s[..., None, None], -FP8_MAX, FP8_MAX).astype(np.float32)
        codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn)
        codes = codes.view(torch.uint8).numpy()
        return np.ascontiguousarray(order(codes)).reshape(n, -1), s
    if codec in (INT8, INT4):
        qmax = 127 if codec == INT8 else 7
        codes, scales = encode_int_g32(x, qmax)
        flat = np.ascontiguousarray(order(codes))               # [n, Hkv, P*D] int8
        body = flat.view(np.uint8) if codec == INT8 else pack_int4(flat)
        sc = np.ascontiguousarray(scales).astype("<f2").view(np.uint8)
        return np.concatenate([body.reshape(n, -1), sc.reshape(n, -1)], axis=1), ones
    raise ValueError(f"unknown codec {codec}")
