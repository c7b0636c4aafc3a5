"""Shared helpers of the GPU tests (imported by tests only)."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_182_amd as pkv
import synth
from synth.device import to_device

OUT_TOL = 1e-3   # max-abs on out
LSE_TOL = 1e-4   # max-abs on lse


def params_for(w, partition_tokens=None, k_codec=None, v_codec=None):
    codes = {int(c) for c in w.page_codec}
    kcs, vcs = {c & 15 for c in codes}, {c >> 4 for c in codes}
    if len(codes) > 1 and all((c & 15) == (c >> 4) <= pkv.FP8_E4M3 for c in codes):
        # float pages of several codecs: the float per-page class, as the benchmark declares it
        kcs, vcs = {pkv.CODEC_MIXED_FLOAT}, {pkv.CODEC_MIXED_FLOAT}
    if k_codec is None:
        k_codec = kcs.pop() if len(kcs) == 1 else pkv.CODEC_MIXED
    if v_codec is None:
        v_codec = vcs.pop() if len(vcs) == 1 else pkv.CODEC_MIXED
    return pkv.make_params(
        rows=w.rows, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
        head_dim=w.head_dim, page_size=w.page_size, num_pages=w.num_pages,
        max_pages_per_row=w.max_pages, pool_bytes=w.pool.nbytes, max_sel_pages=w.max_sel,
        partition_tokens=w.partition_tokens if partition_tokens is None else partition_tokens,
        k_codec=k_codec, v_codec=v_codec, softmax_scale=w.softmax_scale)


def run(dw, p, err=None):
    out, lse = pkv.decode_attention(p, *dw.args(), err_count=err)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(out, lse, ref_out, ref_lse, what=""):
    """Max-abs check; empty rows must match exactly (out 0, lse -inf)."""
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: empty-row pattern differs"
    assert np.all(np.isfinite(out)), f"{what}: non-finite out"
    eo = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    el = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    print(f"parity {what}: out max-abs {eo:.3e} lse max-abs {el:.3e}", flush=True)
    assert eo <= OUT_TOL, f"{what}: out max-abs {eo:.3g} > {OUT_TOL}"
    assert el <= LSE_TOL, f"{what}: lse max-abs {el:.3g} > {LSE_TOL}"
    return eo, el


def poison_tails(w):
    """Overwrite every byte the row lengths exclude inside attended pages'
    tail tokens with bytes that decode to NaN/huge values in every codec."""
    from oracle.layout import BITS, code_bits, code_position
    P, D, hkv = w.page_size, w.head_dim, w.num_kv_heads
    arr = w.pool.as_array() if w.pool.is_dense else None
    assert arr is not None
    for r in range(w.rows):
        L = int(w.seq_lens[r])
        if L % P == 0:
            continue
        lp = L // P
        pp = int(w.block_table[r, lp])
        valid = L - lp * P
        c = int(w.page_codec[pp])
        for off, codec, is_v in ((int(w.page_k_off[pp]), c & 15, False), (int(w.page_v_off[pp]), c >> 4, True)):
            bits = BITS[codec]
            head_bytes = P * D * bits // 8
            if bits < 4:
                # every 2- or 1-bit code is a valid code: set the tail's codes
                # to all ones; the scales and offsets below carry the poison
                bpos, shift = code_bits(P, D, codec, is_v)
                ones = ((1 << bits) - 1) << shift[valid:].ravel()
                for h in range(hkv):
                    np.bitwise_or.at(arr, off + h * head_bytes + bpos[valid:].ravel(), ones.astype(np.uint8))
            else:
                pos, nib = code_position(P, D, codec, is_v)
                pos = pos[valid:].ravel()
            for h in range(hkv if bits >= 4 else 0):
                base = off + h * head_bytes
                if bits == 16:
                    arr[base + pos] = 0xFF                        # fp16/bf16 NaN
                    arr[base + pos + 1] = 0xFF
                elif bits == 8:
                    arr[base + pos] = 0x7F if codec == synth.FP8 else 0x80  # NaN / -128
                else:                                             # int4: nibble -8
                    hi = nib[valid:].ravel() == 1
                    b_hi, b_lo = base + pos[hi], base + pos[~hi]
                    arr[b_hi] = (arr[b_hi] & 0x0F) | 0x80
                    arr[b_lo] = (arr[b_lo] & 0xF0) | 0x08
            if codec in (synth.INT8, synth.INT4, synth.INT2, synth.BIT1):
                sc = off + hkv * P * D * bits // 8
                regions = 2 if codec == synth.INT2 else 1         # INT2: offsets after the scales
                for reg in range(regions):
                    base = sc + reg * hkv * P * (D // 32) * 2
                    for h in range(hkv):
                        s0 = base + (h * P + valid) * (D // 32) * 2
                        s1 = base + (h * P + P) * (D // 32) * 2
                        arr[s0:s1] = 0x7C                         # fp16 0x7C7C: NaN
    return w


def rewrite_bf16(w, make):
    """Replace the values of every BF16 plane with ``make(row, lp, is_v)``
    (float32 [Hkv, P, D]), encoded as the layout prescribes; other planes
    keep their bytes."""
    from synth.layout import BF16, encode_plane
    arr = w.pool.as_array()
    P, D, hkv = w.page_size, w.head_dim, w.num_kv_heads
    for r in range(w.rows):
        for lp in range(-(-int(w.seq_lens[r]) // P)):
            pp = int(w.block_table[r, lp])
            code = int(w.page_codec[pp])
            for is_v, codec, off in ((False, code & 15, int(w.page_k_off[pp])), (True, code >> 4, int(w.page_v_off[pp]))):
                if codec != BF16:
                    continue
                x = make(r, lp, is_v).astype(np.float32).reshape(1, hkv, P, D)
                b, _ = encode_plane(x, BF16, v_order=is_v)
                arr[off:off + b.shape[1]] = b[0]
