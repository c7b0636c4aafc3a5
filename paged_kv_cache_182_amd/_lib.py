"""ctypes binding of libpkv (argument marshalling only).

Every step of decode attention runs in the HIP kernels behind the C ABI in
include/pkv.h; this module only checks tensor dtypes/devices, packs
``pkv_params`` and passes raw device pointers and the current HIP stream.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # loads the HIP runtime the library must share (import before libpkv)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

FP16, BF16, FP8_E4M3, INT8_G32, INT4_G32, INT2_G32, BIT1_G32, CODEC_MIXED, CODEC_MIXED_FLOAT = 0, 1, 2, 3, 4, 5, 6, -1, -2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5
EXPORTS = ("pkv_abi_version", "pkv_status_string", "pkv_num_partitions",
           "pkv_workspace_bytes", "pkv_decode_attention", "pkv_decode_partials",
           "pkv_lse_combine", "pkv_append_kv", "pkv_encode_pages", "pkv_prefill_num_partitions",
           "pkv_prefill_workspace_bytes", "pkv_prefill_attention", "pkv_lse_fold_into", "pkv_select_capacity",
           "pkv_select_pages", "pkv_decode_attention_noalloc", "pkv_noalloc_scratch_bytes")


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_row", ctypes.c_int32), ("max_sel_pages", ctypes.c_int32),
                ("partition_tokens", ctypes.c_int32), ("k_codec", ctypes.c_int32),
                ("v_codec", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("pool_bytes", ctypes.c_uint64), ("window_tokens", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpkv.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_182_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pp = ctypes.POINTER(Params)
    lib.pkv_abi_version.restype = ctypes.c_int
    lib.pkv_abi_version.argtypes = []
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_num_partitions.restype = ctypes.c_int
    lib.pkv_num_partitions.argtypes = [pp]
    lib.pkv_workspace_bytes.restype = sz
    lib.pkv_workspace_bytes.argtypes = [pp]
    lib.pkv_decode_attention.restype = ctypes.c_int
    lib.pkv_decode_attention.argtypes = [pp] + [vp] * 12 + [vp, sz, vp, vp]
    lib.pkv_decode_attention_noalloc.restype = ctypes.c_int
    lib.pkv_decode_attention_noalloc.argtypes = [pp] + [vp] * 12 + [vp, vp]
    lib.pkv_noalloc_scratch_bytes.restype = sz
    lib.pkv_noalloc_scratch_bytes.argtypes = []
    lib.pkv_decode_partials.restype = ctypes.c_int
    lib.pkv_decode_partials.argtypes = [pp] + [vp] * 12 + [vp, vp]
    lib.pkv_lse_combine.restype = ctypes.c_int
    lib.pkv_lse_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.pkv_append_kv.restype = ctypes.c_int
    lib.pkv_append_kv.argtypes = [pp] + [vp] * 10
    lib.pkv_encode_pages.restype = ctypes.c_int
    lib.pkv_encode_pages.argtypes = [pp, i32, vp, vp, i32] + [vp] * 7
    lib.pkv_prefill_num_partitions.restype = ctypes.c_int
    lib.pkv_prefill_num_partitions.argtypes = [pp, i32, i32, i32]
    lib.pkv_prefill_workspace_bytes.restype = sz
    lib.pkv_prefill_workspace_bytes.argtypes = [pp, i32, i32, i32]
    lib.pkv_prefill_attention.restype = ctypes.c_int
    lib.pkv_prefill_attention.argtypes = [pp, i32, i32, i32, i32] + [vp] * 10 + [vp, sz, vp, vp]
    lib.pkv_lse_fold_into.restype = ctypes.c_int
    lib.pkv_select_capacity.restype = ctypes.c_int
    lib.pkv_select_capacity.argtypes = [i32] * 5
    lib.pkv_select_pages.restype = ctypes.c_int
    lib.pkv_select_pages.argtypes = [pp] + [i32] * 6 + [vp] * 9
    lib.pkv_lse_fold_into.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    if lib.pkv_abi_version() != 4:  # window_tokens in pkv_params; INT2 and 1-bit codecs
        raise RuntimeError("libpkv ABI version mismatch")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pkv_status_string(status).decode()


def make_params(*, rows, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                max_pages_per_row, pool_bytes, max_sel_pages=0, partition_tokens=0,
                k_codec=CODEC_MIXED, v_codec=CODEC_MIXED, softmax_scale=None, window_tokens=0) -> Params:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return Params(rows, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                  max_pages_per_row, max_sel_pages, partition_tokens, k_codec, v_codec,
                  softmax_scale, pool_bytes, window_tokens)


def num_partitions(p: Params) -> int:
    n = load().pkv_num_partitions(ctypes.byref(p))
    if n < 0:
        raise PkvError(n, "pkv_num_partitions")
    return n


def workspace_bytes(p: Params) -> int:
    return int(load().pkv_workspace_bytes(ctypes.byref(p)))


def _ptr(t: Optional[torch.Tensor], dtype, name: str, device) -> int:
    if t is None:
        return 0
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def decode_attention(p: Params, q, page_pool, page_k_off, page_v_off, page_codec, page_scale,
                     block_table, seq_lens, page_sel=None, sel_lens=None, *, out=None, lse=None,
                     workspace=None, err_count=None, stream=None):
    """Enqueue pkv_decode_attention. Returns (out, lse); allocates them (and the
    workspace) with torch when not given. Raises PkvError on a bad status."""
    lib = load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a device tensor")
    if out is None:
        out = torch.empty((p.num_rows, p.num_q_heads, p.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((p.num_rows, p.num_q_heads), dtype=torch.float32, device=dev)
    need = workspace_bytes(p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = 0 if workspace is None else _ptr(workspace, torch.uint8, "workspace", dev)
    ws_len = 0 if workspace is None else workspace.numel()
    st = lib.pkv_decode_attention(
        ctypes.byref(p), _ptr(q, torch.float16, "q", dev),
        _ptr(page_pool, torch.uint8, "page_pool", dev),
        _ptr(page_k_off, torch.uint64, "page_k_off", dev),
        _ptr(page_v_off, torch.uint64, "page_v_off", dev),
        _ptr(page_codec, torch.uint8, "page_codec", dev),
        _ptr(page_scale, torch.float32, "page_scale", dev),
        _ptr(block_table, torch.int32, "block_table", dev),
        _ptr(seq_lens, torch.int32, "seq_lens", dev),
        _ptr(page_sel, torch.int32, "page_sel", dev),
        _ptr(sel_lens, torch.int32, "sel_lens", dev),
        _ptr(out, torch.float32, "out", dev), _ptr(lse, torch.float32, "lse", dev),
        ws_ptr, ws_len, _ptr(err_count, torch.int32, "err_count", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_decode_attention")
    return out, lse


def decode_attention_noalloc(p: Params, q, page_pool, page_k_off, page_v_off, page_codec, page_scale,
                             block_table, seq_lens, page_sel=None, sel_lens=None, *, out, lse,
                             err_count=None, stream=None):
    """Enqueue pkv_decode_attention_noalloc: out/lse must be given (nothing is
    allocated here or in the library). Raises PkvError on a bad status."""
    lib = load()
    dev = q.device
    st = lib.pkv_decode_attention_noalloc(
        ctypes.byref(p), _ptr(q, torch.float16, "q", dev),
        _ptr(page_pool, torch.uint8, "page_pool", dev),
        _ptr(page_k_off, torch.uint64, "page_k_off", dev),
        _ptr(page_v_off, torch.uint64, "page_v_off", dev),
        _ptr(page_codec, torch.uint8, "page_codec", dev),
        _ptr(page_scale, torch.float32, "page_scale", dev),
        _ptr(block_table, torch.int32, "block_table", dev),
        _ptr(seq_lens, torch.int32, "seq_lens", dev),
        _ptr(page_sel, torch.int32, "page_sel", dev),
        _ptr(sel_lens, torch.int32, "sel_lens", dev),
        _ptr(out, torch.float32, "out", dev), _ptr(lse, torch.float32, "lse", dev),
        _ptr(err_count, torch.int32, "err_count", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_decode_attention_noalloc")
    return out, lse


def noalloc_scratch_bytes() -> int:
    return int(load().pkv_noalloc_scratch_bytes())


def decode_partials(p: Params, q, page_pool, page_k_off, page_v_off, page_codec, page_scale,
                    block_table, seq_lens, page_sel=None, sel_lens=None, *, part_acc=None,
                    part_ml=None, err_count=None, stream=None):
    """Enqueue pkv_decode_partials. Returns (part_acc [B, Hq, n, D], part_ml [B, Hq, n, 2])."""
    lib = load()
    dev = q.device
    n = num_partitions(p)
    if part_acc is None:
        part_acc = torch.empty((p.num_rows, p.num_q_heads, n, p.head_dim), dtype=torch.float32, device=dev)
    if part_ml is None:
        part_ml = torch.empty((p.num_rows, p.num_q_heads, n, 2), dtype=torch.float32, device=dev)
    st = lib.pkv_decode_partials(
        ctypes.byref(p), _ptr(q, torch.float16, "q", dev),
        _ptr(page_pool, torch.uint8, "page_pool", dev),
        _ptr(page_k_off, torch.uint64, "page_k_off", dev),
        _ptr(page_v_off, torch.uint64, "page_v_off", dev),
        _ptr(page_codec, torch.uint8, "page_codec", dev),
        _ptr(page_scale, torch.float32, "page_scale", dev),
        _ptr(block_table, torch.int32, "block_table", dev),
        _ptr(seq_lens, torch.int32, "seq_lens", dev),
        _ptr(page_sel, torch.int32, "page_sel", dev),
        _ptr(sel_lens, torch.int32, "sel_lens", dev),
        _ptr(part_acc, torch.float32, "part_acc", dev), _ptr(part_ml, torch.float32, "part_ml", dev),
        _ptr(err_count, torch.int32, "err_count", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_decode_partials")
    return part_acc, part_ml


def lse_combine(part_acc, part_ml, out=None, lse=None, stream=None):
    """Enqueue pkv_lse_combine. part_acc [rows, parts, D], part_ml [rows, parts, 2]."""
    lib = load()
    rows, parts, d = part_acc.shape
    dev = part_acc.device
    if out is None:
        out = torch.empty((rows, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    st = lib.pkv_lse_combine(rows, parts, d, _ptr(part_acc, torch.float32, "part_acc", dev),
                             _ptr(part_ml, torch.float32, "part_ml", dev),
                             _ptr(out, torch.float32, "out", dev), _ptr(lse, torch.float32, "lse", dev),
                             _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_lse_combine")
    return out, lse


def append_kv(p: Params, k_new, v_new, page_pool, page_k_off, page_v_off, page_codec, block_table,
              seq_lens, *, err_count=None, stream=None) -> None:
    """Enqueue pkv_append_kv: k_new, v_new fp16 [rows, Hkv, D]; seq_lens are
    the lengths before the append. Raises PkvError on a bad status."""
    lib = load()
    dev = k_new.device
    st = lib.pkv_append_kv(
        ctypes.byref(p), _ptr(k_new, torch.float16, "k_new", dev), _ptr(v_new, torch.float16, "v_new", dev),
        _ptr(page_pool, torch.uint8, "page_pool", dev), _ptr(page_k_off, torch.uint64, "page_k_off", dev),
        _ptr(page_v_off, torch.uint64, "page_v_off", dev), _ptr(page_codec, torch.uint8, "page_codec", dev),
        _ptr(block_table, torch.int32, "block_table", dev), _ptr(seq_lens, torch.int32, "seq_lens", dev),
        _ptr(err_count, torch.int32, "err_count", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_append_kv")


def encode_pages(p: Params, src_pages, dst_pages, dst_codec: int, page_pool, page_k_off, page_v_off,
                 page_codec, page_scale=None, *, err_count=None, stream=None) -> None:
    """Enqueue pkv_encode_pages: re-encode pages src_pages[i] into dst_pages[i]
    with dst_codec (K | V << 4). Raises PkvError on a bad status."""
    lib = load()
    dev = page_pool.device
    n = int(src_pages.numel())
    if int(dst_pages.numel()) != n:
        raise ValueError("src_pages and dst_pages must have the same length")
    st = lib.pkv_encode_pages(
        ctypes.byref(p), n, _ptr(src_pages, torch.int32, "src_pages", dev),
        _ptr(dst_pages, torch.int32, "dst_pages", dev), int(dst_codec),
        _ptr(page_pool, torch.uint8, "page_pool", dev), _ptr(page_k_off, torch.uint64, "page_k_off", dev),
        _ptr(page_v_off, torch.uint64, "page_v_off", dev), _ptr(page_codec, torch.uint8, "page_codec", dev),
        _ptr(page_scale, torch.float32, "page_scale", dev), _ptr(err_count, torch.int32, "err_count", dev),
        _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_encode_pages")


def prefill_num_partitions(p: Params, q_tokens: int, kv_begin: int = 0, kv_end: int = -1) -> int:
    n = load().pkv_prefill_num_partitions(ctypes.byref(p), int(q_tokens), int(kv_begin), int(kv_end))
    if n < 0:
        raise PkvError(n, "pkv_prefill_num_partitions")
    return n


def prefill_workspace_bytes(p: Params, q_tokens: int, kv_begin: int = 0, kv_end: int = -1) -> int:
    return int(load().pkv_prefill_workspace_bytes(ctypes.byref(p), int(q_tokens), int(kv_begin), int(kv_end)))


def prefill_attention(p: Params, q, page_pool, page_k_off, page_v_off, page_codec, page_scale, block_table,
                      seq_lens, *, kv_begin: int = 0, kv_end: int = -1, window: int = 0, out=None, lse=None,
                      workspace=None, err_count=None, stream=None):
    """Enqueue pkv_prefill_attention: q fp16 [rows, T, Hq, D], the last T
    tokens of each row; `window` > 0 is a sliding window of that many positions. Returns (out [rows, T, Hq, D], lse [rows, T, Hq]);
    allocates them (and the workspace) with torch when not given."""
    lib = load()
    dev = q.device
    if dev.type != "cuda" or q.dim() != 4:
        raise ValueError("q must be a device tensor [rows, T, Hq, D]")
    T = int(q.shape[1])
    if out is None:
        out = torch.empty((p.num_rows, T, p.num_q_heads, p.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((p.num_rows, T, p.num_q_heads), dtype=torch.float32, device=dev)
    need = prefill_workspace_bytes(p, T, kv_begin, kv_end)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = 0 if workspace is None else _ptr(workspace, torch.uint8, "workspace", dev)
    ws_len = 0 if workspace is None else workspace.numel()
    st = lib.pkv_prefill_attention(
        ctypes.byref(p), T, int(kv_begin), int(kv_end), int(window), _ptr(q, torch.float16, "q", dev),
        _ptr(page_pool, torch.uint8, "page_pool", dev),
        _ptr(page_k_off, torch.uint64, "page_k_off", dev),
        _ptr(page_v_off, torch.uint64, "page_v_off", dev),
        _ptr(page_codec, torch.uint8, "page_codec", dev),
        _ptr(page_scale, torch.float32, "page_scale", dev),
        _ptr(block_table, torch.int32, "block_table", dev),
        _ptr(seq_lens, torch.int32, "seq_lens", dev),
        _ptr(out, torch.float32, "out", dev), _ptr(lse, torch.float32, "lse", dev),
        ws_ptr, ws_len, _ptr(err_count, torch.int32, "err_count", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_prefill_attention")
    return out, lse


def lse_fold_into(acc_out, acc_lse, out, lse, stream=None) -> None:
    """Enqueue pkv_lse_fold_into: fold (out, lse) into (acc_out, acc_lse) in
    place; acc_out/out [..., D], acc_lse/lse [...]."""
    lib = load()
    dev = acc_out.device
    d = int(acc_out.shape[-1])
    rows = int(acc_lse.numel())
    if acc_out.numel() != rows * d or out.numel() != rows * d or lse.numel() != rows:
        raise ValueError("lse_fold_into: shapes do not match")
    st = lib.pkv_lse_fold_into(rows, d, _ptr(acc_out, torch.float32, "acc_out", dev),
                               _ptr(acc_lse, torch.float32, "acc_lse", dev), _ptr(out, torch.float32, "out", dev),
                               _ptr(lse, torch.float32, "lse", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_lse_fold_into")


def select_capacity(page_size: int, block_tokens: int, block_topk: int, sink_pages: int = 0,
                    recent_pages: int = 0) -> int:
    n = load().pkv_select_capacity(int(page_size), int(block_tokens), int(block_topk), int(sink_pages),
                                   int(recent_pages))
    if n < 0:
        raise PkvError(n, "pkv_select_capacity")
    return n


def select_pages(p: Params, q_idx, slab, seq_lens, *, block_tokens: int, block_topk: int, sink_pages: int = 0,
                 recent_pages: int = 0, block_scores=None, page_sel=None, sel_lens=None, dropped=None,
                 err_count=None, stream=None):
    """Enqueue pkv_select_pages: q_idx fp16 [rows, idx_dim], slab fp16
    [rows, max_blocks, idx_dim]. Returns (page_sel [rows, max_sel_pages],
    sel_lens [rows], block_scores [rows, max_blocks]); allocates those not given."""
    lib = load()
    dev = q_idx.device
    rows, idx_dim = int(q_idx.shape[0]), int(q_idx.shape[1])
    max_blocks = int(slab.shape[1])
    if int(slab.shape[0]) != rows or int(slab.shape[2]) != idx_dim:
        raise ValueError("slab must be [rows, max_blocks, idx_dim]")
    if page_sel is None:
        page_sel = torch.empty((p.num_rows, p.max_sel_pages), dtype=torch.int32, device=dev)
    if sel_lens is None:
        sel_lens = torch.empty((p.num_rows,), dtype=torch.int32, device=dev)
    if block_scores is None:
        block_scores = torch.empty((rows, max(max_blocks, 1)), dtype=torch.float32, device=dev)
    st = lib.pkv_select_pages(
        ctypes.byref(p), int(block_tokens), int(block_topk), int(sink_pages), int(recent_pages), idx_dim, max_blocks,
        _ptr(q_idx, torch.float16, "q_idx", dev), _ptr(slab, torch.float16, "slab", dev),
        _ptr(seq_lens, torch.int32, "seq_lens", dev), _ptr(block_scores, torch.float32, "block_scores", dev),
        _ptr(page_sel, torch.int32, "page_sel", dev), _ptr(sel_lens, torch.int32, "sel_lens", dev),
        _ptr(dropped, torch.int32, "dropped", dev), _ptr(err_count, torch.int32, "err_count", dev), _stream(stream))
    if st != OK:
        raise PkvError(st, "pkv_select_pages")
    return page_sel, sel_lens, block_scores


def hip_runtime_copies() -> list[str]:
    """Paths of libamdhip64 mapped into this process (there must be one)."""
    seen = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                seen.add(line.split()[-1])
    return sorted(seen)
