"""C-ABI checks that need no GPU: the library loads, exports every function
include/pkv.h declares, sizes partitions and workspaces, and rejects bad
arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_182_amd as pkv
from paged_kv_cache_182_amd._lib import Params

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = pkv.load()
    names = declared_functions()
    assert set(names) == set(pkv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pkv_abi_version() == 4


def test_one_hip_runtime_in_process():
    pkv.load()
    assert len(pkv.hip_runtime_copies()) == 1


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(pkv.status_string(st), str)


def base(**kw):
    d = dict(rows=1, num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=64,
             num_pages=16384, max_pages_per_row=16384, pool_bytes=1 << 29, partition_tokens=2048,
             k_codec=pkv.FP8_E4M3, v_codec=pkv.FP8_E4M3)
    d.update(kw)
    return pkv.make_params(**d)


def test_partitions_and_workspace():
    p = base()
    assert pkv.num_partitions(p) == 512
    assert pkv.workspace_bytes(p) == 1 * 16 * 512 * 130 * 4
    one = base(num_pages=4, max_pages_per_row=4, page_size=1024, partition_tokens=4096)
    assert pkv.num_partitions(one) == 1 and pkv.workspace_bytes(one) == 0
    sparse = base(rows=48, page_size=16, max_pages_per_row=16384, max_sel_pages=128, partition_tokens=256)
    assert pkv.num_partitions(sparse) == 8
    # partitions of any multiple of 16 tokens, also finer than a page
    sub = base(num_pages=16, max_pages_per_row=16, page_size=1024, partition_tokens=48)
    assert pkv.num_partitions(sub) == 342                     # ceil(1024 tiles / 3)
    # 0: each row split evenly into as many partitions as fill one round of
    # resident workgroups (256 compute units x waves per SIMD of the kernel),
    # at least 8 tiles per partition
    auto = base(rows=8, num_q_heads=32, num_kv_heads=8, page_size=16, max_pages_per_row=2048,
                partition_tokens=0, k_codec=pkv.INT8_G32, v_codec=pkv.INT4_G32)
    assert pkv.num_partitions(auto) == 768 // 64               # three waves per SIMD
    auto8 = base(rows=8, num_q_heads=32, num_kv_heads=8, page_size=16, max_pages_per_row=2048,
                 partition_tokens=0)
    assert pkv.num_partitions(auto8) == 1024 // 64             # FP8: four waves per SIMD
    layer = base(num_q_heads=14, head_dim=64, page_size=1024, num_pages=16, max_pages_per_row=16,
                 partition_tokens=0, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED)
    assert pkv.num_partitions(layer) == 128                    # 1024 tiles, at least 8 per partition
    # a declared pair without a kernel of its own runs the per-page kernel
    # (two waves per SIMD at head_dim 128, three at 64)
    fp8k_fp16v = base(rows=2, partition_tokens=0, v_codec=pkv.FP16)
    assert pkv.num_partitions(fp8k_fp16v) == 512 // 4
    d64 = base(rows=2, head_dim=64, partition_tokens=0)       # FP8 at head_dim 64: six waves
    assert pkv.num_partitions(d64) == 1536 // 4
    # float pages of several codecs (each page one of FP16/BF16/FP8 for K and V):
    # four waves per SIMD at head_dim 64, two at 128
    flt = base(num_q_heads=14, head_dim=64, page_size=1024, num_pages=16, max_pages_per_row=16, rows=24,
               partition_tokens=0, k_codec=pkv.CODEC_MIXED_FLOAT, v_codec=pkv.CODEC_MIXED_FLOAT)
    assert pkv.num_partitions(flt) == 1024 // 48
    many = base(rows=2000, partition_tokens=0)
    assert pkv.num_partitions(many) == 1


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, -2), ("head_dim", 256, -2), ("page_size", 8, -1), ("page_size", 24, -1),
    ("num_q_heads", 15, -1), ("num_q_heads", 34, -2), ("partition_tokens", 100, -1),
    ("partition_tokens", 8, -1), ("partition_tokens", -16, -1),
    ("k_codec", -2, -1),   # the float class is declared for both planes or neither
    ("num_rows", -1, -1), ("max_pages_per_row", 0, -1), ("k_codec", 9, -1),
    ("page_size", 1 << 21, -2),   # in-page slot counts are 24-bit on the device
])
def test_bad_params_rejected(field, value, status):
    p = base()
    setattr(p, field, value)
    assert pkv.load().pkv_num_partitions(ctypes.byref(p)) == status
    assert pkv.workspace_bytes(p) == 0


def test_planes_of_4_gib_rejected():
    # one page's 16-bit plane of Hkv * P * D * 2 bytes is addressed with 32-bit offsets
    lib = pkv.load()
    big = base(num_q_heads=16, num_kv_heads=16, page_size=1 << 20, num_pages=1, max_pages_per_row=1)
    assert 16 * (1 << 20) * 128 * 2 == 1 << 32
    assert lib.pkv_num_partitions(ctypes.byref(big)) == -2
    below = base(num_q_heads=8, num_kv_heads=8, page_size=1 << 20, num_pages=1, max_pages_per_row=1)
    assert lib.pkv_num_partitions(ctypes.byref(below)) > 0
    good = [4096] * 8
    assert lib.pkv_append_kv(ctypes.byref(wbase(num_kv_heads=16, page_size=1 << 20)), *good, 0, 0) == -2
    assert lib.pkv_append_kv(ctypes.byref(wbase(page_size=1 << 21)), *good, 0, 0) == -2


def call(p, **ptrs):
    """pkv_decode_attention with fake (never dereferenced) pointers; only for
    arguments the host check must reject before any launch."""
    names = ["q", "pool", "koff", "voff", "codec", "scale", "bt", "lens", "sel", "sel_lens", "out", "lse"]
    vals = {n: 4096 for n in names}
    vals.update(sel=0, sel_lens=0)
    vals.update(ptrs)
    ws = vals.pop("ws", 0)
    wsb = vals.pop("wsb", 0)
    return pkv.load().pkv_decode_attention(ctypes.byref(p), *[vals[n] for n in names], ws, wsb, 0, 0)


def test_host_rejects_bad_pointers_and_workspace():
    p = base()
    assert call(p, q=0) == -1
    assert call(p, q=4098) == -1                       # q not 16-byte aligned
    assert call(p, pool=4096 + 128) == -1              # pool not 256-byte aligned
    assert call(p, scale=0) == -1                      # FP8 declared without scales
    assert call(p) == -3                               # 512 partitions need a workspace
    assert call(p, ws=4096, wsb=100) == -3
    sp = base(max_sel_pages=128)
    assert call(sp) == -1                              # sparse mode without page_sel
    p0 = base(rows=0)
    assert call(p0, q=0) == 0                          # nothing to do
    assert pkv.load().pkv_lse_combine(4, 0, 128, 4096, 4096, 4096, 4096, 0) == -1
    assert pkv.load().pkv_lse_combine(4, 2, 1024, 4096, 4096, 4096, 4096, 0) == -1
    assert pkv.load().pkv_lse_combine(0, 2, 128, 0, 0, 0, 0, 0) == 0


def wbase(**kw):
    d = dict(rows=4, num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=64, num_pages=64,
             max_pages_per_row=16, pool_bytes=1 << 24)
    d.update(kw)
    return pkv.make_params(**d)


def test_append_host_checks():
    lib = pkv.load()
    p = wbase()
    good = [4096] * 8          # fake addresses: every call below must be rejected on the host
    assert lib.pkv_append_kv(ctypes.byref(p), 0, *good[1:], 0, 0) == -1           # k_new missing
    assert lib.pkv_append_kv(ctypes.byref(p), 4097, *good[1:], 0, 0) == -1        # k_new odd address
    assert lib.pkv_append_kv(ctypes.byref(p), 4096, 4096, 4096 + 16, *good[3:], 0, 0) == -1  # pool alignment
    assert lib.pkv_append_kv(ctypes.byref(wbase(head_dim=96)), *good, 0, 0) == -2
    assert lib.pkv_append_kv(ctypes.byref(wbase(page_size=24)), *good, 0, 0) == -1
    assert lib.pkv_append_kv(ctypes.byref(wbase(rows=0)), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == 0


def test_encode_host_checks():
    lib = pkv.load()
    p = wbase()
    args = [4096] * 5                                  # pool, k_off, v_off, codec, scale
    assert lib.pkv_encode_pages(ctypes.byref(p), 0, 0, 0, 0x22, *args, 0, 0) == 0      # nothing to do
    assert lib.pkv_encode_pages(ctypes.byref(p), -1, 4096, 4096, 0x22, *args, 0, 0) == -1
    assert lib.pkv_encode_pages(ctypes.byref(p), 4, 4096, 4096, 0x27, *args, 0, 0) == -1  # K nibble 7
    assert lib.pkv_encode_pages(ctypes.byref(p), 4, 4096, 4096, 0x122, *args, 0, 0) == -1  # > one byte
    assert lib.pkv_encode_pages(ctypes.byref(p), 4, 4096, 4096, 0x22, 4096, 4096, 4096, 4096, 0, 0, 0) == -1  # FP8 needs scales
    assert lib.pkv_encode_pages(ctypes.byref(p), 4, 0, 4096, 0x43, *args, 0, 0) == -1      # src missing
    assert lib.pkv_encode_pages(ctypes.byref(wbase(head_dim=256)), 4, 4096, 4096, 0x43, *args, 0, 0) == -2


def pcall(p, T=16, kv_begin=0, kv_end=-1, **ptrs):
    """pkv_prefill_attention with fake (never dereferenced) pointers; only for
    arguments the host check must reject before any launch."""
    names = ["q", "pool", "koff", "voff", "codec", "scale", "bt", "lens", "out", "lse"]
    vals = {n: 4096 for n in names}
    vals.update(ptrs)
    ws = vals.pop("ws", 0)
    wsb = vals.pop("wsb", 0)
    return pkv.load().pkv_prefill_attention(ctypes.byref(p), T, kv_begin, kv_end, 0, *[vals[n] for n in names],
                                            ws, wsb, 0, 0)


def test_prefill_partitions_and_workspace():
    p = base(partition_tokens=8192)                     # 1M tokens of 64-token pages
    assert pkv.prefill_num_partitions(p, 64) == 128
    assert pkv.prefill_workspace_bytes(p, 64) == 64 * 16 * 128 * 130 * 4
    # partitions start at kv_begin rounded down to a page and end at kv_end
    assert pkv.prefill_num_partitions(p, 64, 100, 8192 + 64) == 1   # [64, 8256): one partition
    assert pkv.prefill_num_partitions(p, 64, 100, 8192 + 65) == 2
    assert pkv.prefill_num_partitions(p, 64, 8192, 8192 * 2) == 1
    assert pkv.prefill_workspace_bytes(p, 64, 8192, 8192 * 2) == 0
    # 0: one round of resident workgroups: 256 compute units x 2 waves per SIMD
    # (FP8, head_dim 128) over 4 column groups x 2 KV heads
    auto = base(partition_tokens=0)
    n = pkv.prefill_num_partitions(auto, 64)
    assert n == 512 // 8
    assert pkv.prefill_num_partitions(auto, 64, 5, 5) == 1   # empty window
    # the same count per kernel as it runs (its waves per SIMD): 256 compute
    # units x waves over 8 workgroups per partition index; pairs without a
    # kernel of their own run the one-wave per-page kernel
    waves = {(64, pkv.FP16, pkv.FP16): 4, (64, pkv.FP8_E4M3, pkv.FP8_E4M3): 4, (64, pkv.BF16, pkv.BF16): 3,
             (64, pkv.INT8_G32, pkv.INT4_G32): 2, (64, pkv.FP8_E4M3, pkv.FP16): 1,
             (128, pkv.FP16, pkv.FP16): 2, (128, pkv.BF16, pkv.BF16): 2, (128, pkv.INT8_G32, pkv.INT4_G32): 1,
             (128, pkv.FP8_E4M3, pkv.FP16): 1, (128, pkv.INT4_G32, pkv.INT8_G32): 1}
    for (d, kc, vc), wv in waves.items():
        q = base(partition_tokens=0, head_dim=d, k_codec=kc, v_codec=vc)
        assert pkv.prefill_num_partitions(q, 64) == 256 * wv // 8, (d, kc, vc)


def test_prefill_host_checks():
    p = base()
    lib = pkv.load()
    # prefill partitions are whole pages (decode accepts any multiple of 16)
    assert lib.pkv_prefill_num_partitions(ctypes.byref(base(partition_tokens=48)), 4, 0, -1) == -1
    assert pkv.num_partitions(base(partition_tokens=48)) > 0
    assert lib.pkv_prefill_num_partitions(ctypes.byref(p), -1, 0, -1) == -1
    assert lib.pkv_prefill_num_partitions(ctypes.byref(p), 4, -3, -1) == -1
    assert lib.pkv_prefill_num_partitions(ctypes.byref(p), 4, 100, 50) == -1
    assert lib.pkv_prefill_num_partitions(ctypes.byref(base(max_sel_pages=8)), 4, 0, -1) == -1
    assert lib.pkv_prefill_num_partitions(ctypes.byref(base(head_dim=96)), 4, 0, -1) == -2
    assert pcall(p, T=-1) == -1
    assert pcall(p, kv_begin=10, kv_end=5) == -1
    assert pcall(p, q=0) == -1
    assert pcall(p, q=4104) == -1                       # q not 16-byte aligned
    assert pcall(p, pool=4096 + 64) == -1               # pool not 256-byte aligned
    assert pcall(p, scale=0) == -1                      # FP8 declared without scales
    assert pcall(p) == -3                               # 512 partitions need a workspace
    assert pcall(p, ws=4096, wsb=1000) == -3
    assert pcall(base(max_sel_pages=8)) == -1           # the prefill reads the dense cache
    assert pcall(p, T=0, q=0) == 0                      # nothing to do
    assert pcall(base(rows=0), q=0) == 0
    assert lib.pkv_lse_fold_into(4, 0, 4096, 4096, 4096, 4096, 0) == -1
    assert lib.pkv_lse_fold_into(4, 513, 4096, 4096, 4096, 4096, 0) == -1
    assert lib.pkv_lse_fold_into(4, 128, 0, 4096, 4096, 4096, 0) == -1
    assert lib.pkv_lse_fold_into(4, 128, 4098, 4096, 4096, 4096, 0) == -1
    assert lib.pkv_lse_fold_into(0, 128, 0, 0, 0, 0, 0) == 0


def test_select_capacity_and_host_checks():
    assert pkv.select_capacity(16, 16, 127, 0, 1) == 128
    assert pkv.select_capacity(16, 12, 32, 4, 4) == 2 * 32 + 8       # the pages' 2 * block_topk + 8
    assert pkv.select_capacity(16, 40, 10, 0, 0) == 30
    lib = pkv.load()
    assert lib.pkv_select_capacity(0, 16, 1, 0, 0) == -1
    assert lib.pkv_select_capacity(16, 16, -1, 0, 0) == -1
    p = pkv.make_params(rows=2, num_q_heads=1, num_kv_heads=1, head_dim=128, page_size=16, num_pages=1,
                        max_pages_per_row=64, pool_bytes=0, max_sel_pages=32)

    def sel(pp=p, bt=16, k=4, dim=64, mb=64, **ptr):
        v = dict(q=4096, slab=4096, lens=4096, scores=4096, out=4096, n=4096)
        v.update(ptr)
        return lib.pkv_select_pages(ctypes.byref(pp), bt, k, 0, 1, dim, mb, v["q"], v["slab"], v["lens"],
                                    v["scores"], v["out"], v["n"], 0, 0, 0)
    assert sel(dim=12) == -1                          # idx_dim not a multiple of 8
    assert sel(bt=0) == -1
    assert sel(k=-1) == -1
    assert sel(q=0) == -1
    assert sel(slab=4104) == -1                       # slab not 16-byte aligned
    assert sel(pp=pkv.make_params(rows=2, num_q_heads=1, num_kv_heads=1, head_dim=128, page_size=16,
                                  num_pages=1, max_pages_per_row=64, pool_bytes=0, max_sel_pages=0)) == -1
    assert sel(pp=pkv.make_params(rows=2, num_q_heads=1, num_kv_heads=1, head_dim=128, page_size=16,
                                  num_pages=1, max_pages_per_row=1 << 20, pool_bytes=0, max_sel_pages=8)) == -2
    assert sel(pp=pkv.make_params(rows=0, num_q_heads=1, num_kv_heads=1, head_dim=128, page_size=16,
                                  num_pages=1, max_pages_per_row=64, pool_bytes=0, max_sel_pages=8), q=0) == 0
    # a slab row is read through one 32-bit buffer range: (max_blocks + 64) * idx_dim * 2 < 4 GiB - 64 KiB
    assert sel(dim=4096, mb=(1 << 19) - 64) == -2               # 4 GiB exactly: refused
    assert sel(dim=8, mb=(1 << 28)) == -2


def test_noalloc_rejects_requests_beyond_its_scratch_on_the_host():
    """The allocation-free entry point refuses, before touching the device,
    a call whose partials exceed its built-in scratch (8 MiB); the 1M-token
    workload's 4.26 MB fit."""
    lib = pkv.load()
    assert pkv.noalloc_scratch_bytes() == 8 << 20
    assert pkv.workspace_bytes(base()) <= pkv.noalloc_scratch_bytes()
    big = base(rows=4)                                     # 4 x 16 x 512 x 130 x 4 B = 17 MB
    assert pkv.workspace_bytes(big) > pkv.noalloc_scratch_bytes()
    fake = ctypes.c_void_p(1 << 20)                        # never dereferenced: rejected first
    st = lib.pkv_decode_attention_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, fake, fake,
                                          None, None, fake, fake, None, None)
    assert st == pkv.ERR_SCRATCH
    assert "scratch" in pkv.status_string(st)


def test_window_partitions_on_the_host():
    """With a sliding window the partitions cover its tiles only: at most
    ceil(W / 16) + 1 tiles per row (dense); sparse calls are unchanged; a
    negative window is refused, as is a window given to the prefill."""
    p = base(partition_tokens=2048, window_tokens=8192)            # 513 tiles in 128-tile partitions
    assert pkv.num_partitions(p) == 5
    assert pkv.workspace_bytes(p) == 16 * 5 * 130 * 4
    assert pkv.num_partitions(base(partition_tokens=2048, window_tokens=10 ** 7)) == 512
    sparse = base(rows=48, page_size=16, max_pages_per_row=16384, max_sel_pages=128, partition_tokens=256,
                  window_tokens=100)
    assert pkv.num_partitions(sparse) == 8
    bad = base(window_tokens=-1)
    lib = pkv.load()
    assert lib.pkv_num_partitions(ctypes.byref(bad)) == pkv.ERR_INVALID_ARG
    assert lib.pkv_prefill_num_partitions(ctypes.byref(base(window_tokens=16)), 4, 0, -1) == pkv.ERR_INVALID_ARG
