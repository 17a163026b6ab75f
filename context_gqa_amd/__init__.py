"""Document-masked causal GQA attention for one context-parallel rank on
AMD Instinct MI355X (gfx950): a thin Python binding of the HIP library
libdocmask_gqa.so (C ABI in include/docmask_gqa.h)."""
from .binding import (  # noqa: F401
    DMGQA_ERR_HIP, DMGQA_ERR_INVALID_ARG, DMGQA_ERR_UNSUPPORTED, DMGQA_ERR_WORKSPACE,
    DMGQA_OK, LIB_PATH, SIGNATURES, DocmaskGQAError, docmask_gqa_attn_bwd,
    docmask_gqa_attn_fwd, docmask_gqa_bwd_workspace_size, docmask_gqa_bwd_workspace_size_min,
    docmask_gqa_check_cu_seqlens, docmask_gqa_doc_bounds, docmask_gqa_doc_bounds_size,
    docmask_gqa_check_docs, docmask_gqa_fwd_workspace_size, docmask_gqa_status_string,
    docmask_gqa_version, lib, status_string, docmask_gqa_timing_enable,
    docmask_gqa_kernel_times, docmask_gqa_interval_bounds, docmask_gqa_check_intervals,
    docmask_gqa_attn_fwd_cross, docmask_gqa_check_cross_intervals, docmask_gqa_attn_bwd_cross,
    docmask_gqa_bwd_workspace_size_full, docmask_gqa_bwd_path, DMGQA_BWD_PATH_RECOMPUTE,
    DMGQA_BWD_PATH_STASH, DMGQA_BWD_PATH_MIXED, docmask_gqa_attn_fwd_noalloc,
    docmask_gqa_batch_plan, docmask_gqa_batch_plan_size, docmask_gqa_bwd_cross_path,
)
