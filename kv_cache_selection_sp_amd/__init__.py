"""Sparse decode attention over a paged KV cache on MI355X (gfx950).

Quest page selection, H2O accumulated-score eviction and SnapKV prompt
selection, after "SparseEngine: Sparse-First Inference Engine" (Appendix
A.3), as hand-written HIP kernels
behind the C ABI of ``include/spdecode.h``.  This package holds the HIP
sources (``csrc/``), the build script and the ctypes binding.
"""
from ._lib import (  # noqa: F401
    LIB_PATH, EXPORTED, SpError, SpPagedKV, PagedKV, load,
    SP_OK, SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED, SP_ERR_MISALIGNED,
    SP_ERR_WORKSPACE, SP_ERR_HIP, SP_F32, SP_BF16,
    SP_OP_SELECT_PAGES, SP_OP_DECODE_ATTN, SP_OP_H2O_EVICT, SP_OP_SNAPKV_SCORES, SP_OP_H2O_PREFILL,
    SP_OP_OMNIKV_SELECT, SP_OP_QUEST_STEP,
    SP_GROUP_SUM, SP_GROUP_MAX,
    sp_build_page_meta, sp_select_pages, sp_select_pages_ex, sp_append_select_pages, sp_sparse_decode_attn,
    sp_sparse_decode_attn_noalloc, sp_quest_decode_step, sp_quest_step_error, sp_quest_step_single_launch,
    sp_h2o_accumulate,
    sp_decode_attn_accumulate,
    sp_h2o_evict_compact, sp_snapkv_scores, sp_h2o_prefill_scores, sp_omnikv_select,
    sp_sparse_decode_attn_masked, sp_workspace_bytes, workspace,
    page_token_view, read_slots, read_meta,
)
