"""Mixed-codec paged decode attention for AMD MI355X (gfx950), with the write
side (token append, page demotion) and chunked prefill over the same pages.

The compute lives in ``libpkv.so`` (HIP kernels behind the C ABI declared in
``include/pkv.h``); ``_lib`` is a thin ctypes binding with the same names.
"""
from ._lib import (BF16, BIT1_G32, CODEC_MIXED, CODEC_MIXED_FLOAT, FP8_E4M3, FP16, INT2_G32, INT4_G32,  # noqa: F401
                   INT8_G32, EXPORTS,
                   ERR_INVALID_ARG, ERR_SCRATCH, ERR_UNSUPPORTED, LIB_PATH, Params, PkvError, append_kv, decode_attention,
                   decode_attention_noalloc, decode_partials, encode_pages, noalloc_scratch_bytes,
                   hip_runtime_copies, load, lse_combine, lse_fold_into, make_params, num_partitions,
                   prefill_attention, prefill_num_partitions, prefill_workspace_bytes, select_capacity,
                   select_pages, status_string, workspace_bytes)
