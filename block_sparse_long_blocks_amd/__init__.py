"""Block-sparse causal GQA prefill attention with mean correction (FlashPrefill V2
method) for AMD MI355X / gfx950.

The work runs in libfp2.so (hand-written HIP kernels behind the C ABI of
include/fp2.h); this package is its thin ctypes binding plus buffer setup.
Importing it raises if the library has not been built.
"""
from ._binding import (FP2_BF16, FP2_ERR_CAPACITY, FP2_ERR_HIP, FP2_ERR_INVALID, FP2_ERR_UNSUPPORTED,
                       FP2_FP8_E4M3, FP2_OK, Batch, Fp2Error, KVCache, Queries, exported_symbols,
                       fp2_block_stats, fp2_block_stats_cache_rows, fp2_block_stats_cached,
                       fp2_debug_bounds_word, fp2_gather_block_stats, fp2_plan_mask, fp2_plan_mask_noalloc, fp2_plan_max_nnz,
                       fp2_plan_workspace_bytes, fp2_prefill_run, fp2_run_workspace_bytes, fp2_stage1,
                       fp2_stage1_workspace_bytes, library_path)
from .runner import PrefillLayer, from_arrays, from_workload

__all__ = [
    "Batch", "Queries", "KVCache", "Fp2Error", "PrefillLayer", "from_arrays", "from_workload",
    "fp2_block_stats", "fp2_block_stats_cache_rows", "fp2_block_stats_cached", "fp2_debug_bounds_word",
    "fp2_gather_block_stats",
    "fp2_plan_mask", "fp2_plan_mask_noalloc", "fp2_plan_max_nnz", "fp2_plan_workspace_bytes",
    "fp2_prefill_run", "fp2_run_workspace_bytes", "fp2_stage1", "fp2_stage1_workspace_bytes",
    "exported_symbols", "library_path",
    "FP2_OK", "FP2_ERR_INVALID", "FP2_ERR_UNSUPPORTED", "FP2_ERR_CAPACITY", "FP2_ERR_HIP",
    "FP2_BF16", "FP2_FP8_E4M3",
]
