"""Plain CPU fp64 oracle for query-dependent sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never calls it, shares no code, header, table or helper with it, and this
package imports nothing from the library.

Source: "SparseEngine: Sparse-First Inference Engine", Appendix A.1
("Attention over Selected Positions", "MHA, MQA, and GQA"), Appendix A.2
("Logical Positions and Physical Blocks") and Appendix A.3 ("H2O: Accumulated
Scores and Online Eviction", "SnapKV: Prompt Selection from an Observation
Window", "Quest: Query-Dependent Page Selection", "OmniKV").  The
pages' display equations did not survive extraction; every formula here is the
plainest reading of the surrounding prose, and each reading is stated where it
is used.

Precision: inputs (fp32 or bf16 values) are converted exactly to float64 and
every step runs in float64.  Positions are 0-based (the pages use 1-based j).

Parity pins: every public function is pinned by ``tests/test_oracle_*.py``
against brute force, closed forms, invariants or an independent library
routine (torch SDPA in float64).  The following readings are consistent with
the pages but not checkable against SparseEngine itself ("parity unpinned" as
a reading, though each is pinned as arithmetic): group aggregation of the
Quest bound by summation, candidate pages = all pages including the partial
last one, tie-breaks by lower index/position, H2O scores under GQA summed over
the group, recent window = largest positions, slot order after compaction =
ascending position.
"""
from .attention import attend, attend_heads, dense_decode
from .quest import (page_extrema, page_bound, group_bound, select_top_pages,
                    quest_decode_head, quest_decode)
from .h2o import H2OHeadState, h2o_retain, h2o_step_head, h2o_prefill_chunk, h2o_prefill
from .snapkv import snapkv_window_scores, snapkv_pool, snapkv_retain
from .omnikv import omnikv_token_scores, omnikv_select, omnikv_sparse_layer

__all__ = [
    "attend", "attend_heads", "dense_decode",
    "page_extrema", "page_bound", "group_bound", "select_top_pages",
    "quest_decode_head", "quest_decode",
    "H2OHeadState", "h2o_retain", "h2o_step_head", "h2o_prefill_chunk", "h2o_prefill",
    "snapkv_window_scores", "snapkv_pool", "snapkv_retain",
    "omnikv_token_scores", "omnikv_select", "omnikv_sparse_layer",
]
