"""Pins for byte accounting against figures printed on the pages (no GPU)."""
import json
import os

import pytest

import synth
from oracle.accounting import FP16, FP8, INT4, INT8, kv_bytes_per_token
from oracle.attention import attended_pages

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
MIB = 1024 * 1024


def test_argus_engine_memory_figures():
    g = GOLDEN["argus_engine_32k"]
    geo = g["geometry"]
    tokens, hkv, d, p = g["context_tokens"], geo["kv_heads"], geo["head_dim"], geo["page_tokens"]
    fp16 = 2 * tokens * hkv * kv_bytes_per_token(FP16, d, p) / MIB       # K and V planes
    q4 = 2 * tokens * hkv * kv_bytes_per_token(INT4, d, p) / MIB
    assert fp16 == 128.0 and q4 == 36.0
    # the same non-KV overhead explains both printed totals
    assert round(g["fp16_total_mib"] - fp16, 2) == round(g["q4_0_total_mib"] - q4, 2) == 8.16
    assert round(g["fp16_total_mib"] / g["q4_0_total_mib"], 1) == g["memory_ratio_printed"]


def test_freetoken_capacity_figure():
    g = GOLDEN["freetoken_capacity"]
    pages = g["gpu_pages"] + g["host_pages"]
    assert g["logical_tokens"] % pages == 0 and g["logical_tokens"] // pages == 64


def test_int8_group_cost_matches_q8_0_size():
    # 32 int8 values + one 2-byte scale = 34 bytes, the Q8_0 block size
    assert kv_bytes_per_token(INT8, 32, 16) == 34.0
    assert kv_bytes_per_token(FP8, 128, 64) == 128 + 4 / 64


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_generator_effective_bytes_agree(cid):
    """The benchmark's byte count (from the generator) equals the pinned accounting."""
    w = synth.config(cid, small=cid != 1)
    total = 0.0
    for r in range(w.rows):
        for lp, valid in attended_pages(w, r):
            pp = int(w.block_table[r, lp])
            c = int(w.page_codec[pp])
            for codec in (c & 15, c >> 4):
                total += valid * w.num_kv_heads * kv_bytes_per_token(codec, w.head_dim, w.page_size)
    # FP8 scales are charged per page: a page counts 4 bytes per head per plane
    # whatever its valid tokens; all these workloads' FP8 pages are full.
    assert synth.effective_kv_bytes_formula(w) == pytest.approx(total, rel=0, abs=1e-6)


def test_subbyte_group_costs_match_their_planes():
    """INT2: 2 bits per value + an fp16 step and an fp16 offset per 32
    values (3 bits per value); BIT1: 1 bit + an fp16 scale per 32 (1.5 bits
    per value); each equals the generator's plane size per token."""
    from oracle.accounting import kv_bytes_per_token
    from synth.layout import BIT1, INT2, plane_bytes
    for D in (64, 128):
        assert kv_bytes_per_token(INT2, D, 16) == D * 3 / 8
        assert kv_bytes_per_token(BIT1, D, 16) == D * 1.5 / 8
        for codec in (INT2, BIT1):
            assert kv_bytes_per_token(codec, D, 16) * 4 * 16 == plane_bytes(codec, 4, 16, D)
