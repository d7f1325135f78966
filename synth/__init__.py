"""Seeded synthetic inputs for the DSA forward path.

Shared by the GPU tests, ``bench.py`` and the oracle tests.  This package
holds input generation only (random draws, the storage encoders that turn
them into fp8 / bf16 bit patterns, the planted and tied structures of the
workloads, the block tables of paged caches); none of the indexer, top-k or
attention arithmetic lives here.
"""

from .encode import encode_bf16_rne, encode_e4m3fn_rne, quantize_per_token
from .pages import make_block_table, share_prefix
from .workloads import Workload, make_workload, standard_workload, WORKLOAD_NAMES

__all__ = [
    "encode_bf16_rne",
    "encode_e4m3fn_rne",
    "quantize_per_token",
    "Workload",
    "make_workload",
    "standard_workload",
    "WORKLOAD_NAMES",
    "make_block_table",
    "share_prefix",
]
