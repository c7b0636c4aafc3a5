"""Seeded synthetic inputs shared by the tests, the benchmark and smoke().

This package only generates and encodes inputs (queries, page codes, scales,
block tables, selections); it holds no attention arithmetic and imports
neither the oracle nor the HIP binding.
"""
from .layout import BF16, BIT1, CODEC_NAMES, CODECS, FP8, FP16, INT2, INT4, INT8  # noqa: F401
from .pool import Pool  # noqa: F401
from .workload import Workload, build_workload, prefill_queries, streams  # noqa: F401
from .configs import NAMES, config, effective_kv_bytes_formula  # noqa: F401
