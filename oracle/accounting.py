"""Bytes of codes + scales per token and KV head, per codec.

Pinned in tests/test_oracle_accounting.py to the figures ARGUS prints for its
engine at 32K tokens ("Direct paged attention": 24 query / 4 KV heads,
head_dim 256, 128-token pages; FP16 136.16 MiB vs q4_0 44.16 MiB): FP16 K+V
is 128 MiB and a 4-bit group-of-32 codec with a 2-byte scale is 36 MiB, each
plus the same 8.16 MiB of other memory.
"""
from __future__ import annotations

FP16, BF16, FP8, INT8, INT4, INT2, BIT1 = 0, 1, 2, 3, 4, 5, 6


def kv_bytes_per_token(codec: int, head_dim: int, page_size: int) -> float:
    """Bytes one token of one KV head costs in one plane (K or V).

    FP16/BF16: 2 bytes per value. FP8: 1 byte per value plus one fp32 scale
    per page (4 / page_size per token). INT8/INT4 with groups of 32: 1 or 1/2
    byte per value plus one fp16 scale per 32 values. INT2: 1/4 byte per value
    plus an fp16 scale and an fp16 offset per 32. BIT1: 1/8 byte per value
    plus an fp16 scale per 32.
    """
    if codec in (FP16, BF16):
        return 2.0 * head_dim
    if codec == FP8:
        return float(head_dim) + 4.0 / page_size
    if codec == INT8:
        return head_dim + 2.0 * head_dim / 32
    if codec == INT4:
        return head_dim / 2 + 2.0 * head_dim / 32
    if codec == INT2:          # 2-bit steps, an fp16 scale and an fp16 offset per 32 values
        return head_dim / 4 + 4.0 * head_dim / 32
    if codec == BIT1:          # sign bits and an fp16 scale per 32 values
        return head_dim / 8 + 2.0 * head_dim / 32
    raise ValueError(codec)
