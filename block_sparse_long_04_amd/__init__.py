"""Block-sparse causal prefill attention (FlashPrefill-style) for MI355X.

The computation lives in the HIP library libflashprefill.so (C ABI declared
in include/flashprefill.h); this package is its thin binding plus the seeded
synthetic workloads.
"""
from ._lib import (  # noqa: F401
    FP_BF16, FP_F32, FP_FP8_E4M3, FP_OK, FP_ERR_HIP, FP_ERR_INVALID, FP_ERR_UNSUPPORTED,
    FP_ERR_WORKSPACE, FP_SELECT_TOPK, FP_SELECT_TOPP, FlashPrefillError, FpProblem, FpWsLayout,
    Prefill, alloc_workspace, fp_block_pool, fp_block_select, fp_block_select_group, fp_block_select_probe,
    fp_block_select_sorted,
    fp_sparse_prefill, fp_workspace_layout, load_library, make_problem, prefill, strerror,
    FpVarlen, FpWsLayoutVarlen, PrefillVarlen, fp_block_pool_varlen, fp_block_select_varlen,
    fp_sparse_prefill_varlen, fp_workspace_layout_varlen, FP_ERR_SCRATCH, FP_NOALLOC_SCRATCH_BYTES,
    fp_prefill_noalloc, validate_lists, fp_sparse_prefill_pack,
)
