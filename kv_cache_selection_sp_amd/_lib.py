"""ctypes binding of libspdecode.so (include/spdecode.h).

Argument marshalling only: tensors become device pointers, the descriptor
becomes the C struct, the current torch stream becomes the HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspdecode.so")

SP_OK, SP_ERR_NULL_PTR, SP_ERR_BAD_SHAPE, SP_ERR_UNSUPPORTED, SP_ERR_MISALIGNED, \
    SP_ERR_WORKSPACE, SP_ERR_HIP = range(7)
SP_F32, SP_BF16 = 0, 1
SP_OP_SELECT_PAGES, SP_OP_DECODE_ATTN, SP_OP_H2O_EVICT, SP_OP_SNAPKV_SCORES, SP_OP_H2O_PREFILL, \
    SP_OP_OMNIKV_SELECT, SP_OP_QUEST_STEP = 1, 2, 3, 4, 5, 6, 7
SP_GROUP_SUM, SP_GROUP_MAX = 0, 1

EXPORTED = ("sp_build_page_meta", "sp_select_pages", "sp_select_pages_ex", "sp_append_select_pages",
            "sp_quest_decode_step", "sp_quest_step_error_offset", "sp_quest_step_single_launch",
            "sp_sparse_decode_attn", "sp_sparse_decode_attn_noalloc", "sp_decode_attn_accumulate",
            "sp_h2o_accumulate", "sp_h2o_evict_compact", "sp_snapkv_scores", "sp_h2o_prefill_scores",
            "sp_omnikv_select", "sp_sparse_decode_attn_masked", "sp_workspace_bytes",
            "sp_status_str", "sp_last_error", "sp_version")


class SpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class SpPagedKV(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m kv_cache_selection_sp_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    KVP = ctypes.POINTER(SpPagedKV)
    sigs = {
        "sp_build_page_meta": (I32, [KVP, P, P, I32, P, P, P, I32, P]),
        "sp_select_pages": (I32, [KVP, P, P, I32, P, P, P, SZ, P]),
        "sp_select_pages_ex": (I32, [KVP, P, P, I32, I32, I32, I32, P, P, P, SZ, P]),
        "sp_append_select_pages": (I32, [KVP, P, P, P, P, I32, P, P, I32, I32, I32, I32, P, P, P, SZ, P]),
        "sp_sparse_decode_attn": (I32, [KVP, P, P, I32, F, P, P, P, I32, P, SZ, P]),
        "sp_quest_decode_step": (I32, [KVP, P, P, P, P, I32, P, P, I32, I32, I32, I32, F, P, P, P, P, P, SZ, P]),
        "sp_quest_step_error_offset": (SZ, [KVP]),
        "sp_quest_step_single_launch": (I32, [KVP, I32, P]),
        "sp_sparse_decode_attn_noalloc": (I32, [KVP, P, P, I32, F, P, P, P, I32, P]),
        "sp_h2o_accumulate": (I32, [KVP, P, P, I32, I32, P, I32, P]),
        "sp_h2o_evict_compact": (I32, [KVP, P, P, I32, I32, I32, P, SZ, P]),
        "sp_snapkv_scores": (I32, [KVP, P, I32, F, I32, I32, P, I32, P, SZ, P]),
        "sp_h2o_prefill_scores": (I32, [KVP, P, I32, F, P, I32, P, SZ, P]),
        "sp_omnikv_select": (I32, [KVP, P, I32, P, P, I32, P, I32, P, SZ, P]),
        "sp_sparse_decode_attn_masked": (I32, [KVP, P, P, P, I32, F, P, P, P, SZ, P]),
        "sp_decode_attn_accumulate": (I32, [KVP, P, F, P, P, P, I32, I32, P, I32, P, SZ, P]),
        "sp_workspace_bytes": (SZ, [I32, KVP, I32]),
        "sp_status_str": (ctypes.c_char_p, [I32]),
        "sp_last_error": (ctypes.c_char_p, []),
        "sp_version": (I32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _status_name(st: int) -> str:
    try:
        return load().sp_status_str(st).decode()
    except Exception:
        return f"status {st}"


def _check(st: int):
    if st != SP_OK:
        raise SpError(st, load().sp_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(t: Optional[torch.Tensor] = None):
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def dtype_code(dt: torch.dtype) -> int:
    return {torch.float32: SP_F32, torch.bfloat16: SP_BF16}[dt]


class PagedKV:
    """A paged KV cache: pools, block table and lengths (torch tensors on the
    GPU) plus the C descriptor that points at them."""

    def __init__(self, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, num_q_heads: int):
        nb, hkv, p, d = k_pool.shape
        self.k_pool, self.v_pool = k_pool, v_pool
        self.block_table, self.seq_lens = block_table, seq_lens
        self.num_q_heads, self.num_kv_heads, self.page_size, self.head_dim = num_q_heads, hkv, p, d
        self.num_blocks = nb
        self.batch, self.max_pages = block_table.shape
        self.dtype = k_pool.dtype
        self.desc = SpPagedKV(self.batch, num_q_heads, hkv, d, p, self.max_pages, nb,
                              dtype_code(k_pool.dtype), _ptr(k_pool), _ptr(v_pool),
                              _ptr(block_table), _ptr(seq_lens))

    @property
    def capacity(self) -> int:
        return self.max_pages * self.page_size

    @staticmethod
    def allocate(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                 max_pages: int, num_blocks: int, dtype: torch.dtype, block_table: torch.Tensor,
                 device="cuda") -> "PagedKV":
        """Zeroed pools [num_blocks][H_kv][P][D] (the per-page layout inside is
        the library's) and zero lengths."""
        shape = (num_blocks, num_kv_heads, page_size, head_dim)
        k = torch.zeros(shape, dtype=dtype, device=device)
        v = torch.zeros(shape, dtype=dtype, device=device)
        lens = torch.zeros(batch, dtype=torch.int32, device=device)
        bt = block_table.to(device=device, dtype=torch.int32).contiguous()
        assert bt.shape == (batch, max_pages)
        return PagedKV(k, v, bt, lens, num_q_heads)

    def new_meta(self) -> torch.Tensor:
        return torch.zeros((self.num_blocks, self.num_kv_heads, 2, self.head_dim),
                           dtype=self.dtype, device=self.k_pool.device)


# ------------------------------------------------------------------ the calls
def sp_build_page_meta(kv: PagedKV, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                       n_new: int, page_meta: Optional[torch.Tensor],
                       pos_new: Optional[torch.Tensor] = None,
                       slot_pos: Optional[torch.Tensor] = None, slot_cap: int = 0):
    _check(load().sp_build_page_meta(ctypes.byref(kv.desc), _ptr(k_new), _ptr(v_new), n_new,
                                     _ptr(page_meta), _ptr(pos_new), _ptr(slot_pos), slot_cap,
                                     _stream()))


def sp_workspace_bytes(op: int, kv: PagedKV, top_k: int) -> int:
    return int(load().sp_workspace_bytes(op, ctypes.byref(kv.desc), top_k))


def workspace(op: int, kv: PagedKV, top_k: int) -> torch.Tensor:
    """A zero-filled workspace of the size the library asks for (the
    decode-attention workspace starts with arrival counters that must be zero
    on first use; every call leaves them zero)."""
    n = sp_workspace_bytes(op, kv, top_k)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=kv.k_pool.device)


def sp_select_pages(kv: PagedKV, q: torch.Tensor, page_meta: torch.Tensor, top_k: int,
                    sel_pages: torch.Tensor, page_scores: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_select_pages(ctypes.byref(kv.desc), _ptr(q), _ptr(page_meta), top_k,
                                  _ptr(sel_pages), _ptr(page_scores), _ptr(ws), nbytes,
                                  _stream()))


def sp_select_pages_ex(kv: PagedKV, q: torch.Tensor, page_meta: torch.Tensor, top_k: int,
                       n_sink: int, n_recent: int, group_reduce: int, sel_pages: torch.Tensor,
                       page_scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_select_pages_ex(ctypes.byref(kv.desc), _ptr(q), _ptr(page_meta), top_k, n_sink,
                                     n_recent, group_reduce, _ptr(sel_pages), _ptr(page_scores),
                                     _ptr(ws), nbytes, _stream()))


def sp_append_select_pages(kv: PagedKV, k_new: torch.Tensor, v_new: torch.Tensor,
                           pos_new: Optional[torch.Tensor], slot_pos: Optional[torch.Tensor], slot_cap: int,
                           page_meta: torch.Tensor, q: torch.Tensor, top_k: int, n_sink: int, n_recent: int,
                           group_reduce: int, sel_pages: torch.Tensor,
                           page_scores: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_append_select_pages(ctypes.byref(kv.desc), _ptr(k_new), _ptr(v_new), _ptr(pos_new),
                                         _ptr(slot_pos), slot_cap, _ptr(page_meta), _ptr(q), top_k, n_sink,
                                         n_recent, group_reduce, _ptr(sel_pages), _ptr(page_scores),
                                         _ptr(ws), nbytes, _stream()))


def sp_sparse_decode_attn(kv: PagedKV, q: torch.Tensor, sel_pages: Optional[torch.Tensor],
                          top_k: int, scale: float, out: torch.Tensor,
                          lse: Optional[torch.Tensor] = None,
                          logits: Optional[torch.Tensor] = None, logit_cap: int = 0,
                          ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_sparse_decode_attn(ctypes.byref(kv.desc), _ptr(q), _ptr(sel_pages), top_k,
                                        float(scale), _ptr(out), _ptr(lse), _ptr(logits),
                                        logit_cap, _ptr(ws), nbytes, _stream()))


def sp_quest_decode_step(kv: PagedKV, k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor],
                         pos_new: Optional[torch.Tensor], slot_pos: Optional[torch.Tensor], slot_cap: int,
                         page_meta: torch.Tensor, q: torch.Tensor, top_k: int, n_sink: int, n_recent: int,
                         group_reduce: int, scale: float, sel_pages: torch.Tensor,
                         page_scores: Optional[torch.Tensor], out: torch.Tensor, lse: Optional[torch.Tensor],
                         ws: torch.Tensor):
    nbytes = ws.numel() * ws.element_size()
    _check(load().sp_quest_decode_step(ctypes.byref(kv.desc), _ptr(k_new), _ptr(v_new), _ptr(pos_new),
                                       _ptr(slot_pos), slot_cap, _ptr(page_meta), _ptr(q), top_k, n_sink,
                                       n_recent, group_reduce, float(scale), _ptr(sel_pages), _ptr(page_scores),
                                       _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream()))


def sp_quest_step_error(kv: PagedKV, ws: torch.Tensor) -> int:
    """The fused step's error word (0 unless a wait gave up); reads the device."""
    off = load().sp_quest_step_error_offset(ctypes.byref(kv.desc))
    return int(ws.view(torch.uint8)[off:off + 4].view(torch.int32).item())


def sp_quest_step_single_launch(kv: PagedKV, group_reduce: int = SP_GROUP_SUM) -> bool:
    """Whether sp_quest_decode_step runs as one launch for this cache on the
    current device (False: the two launches)."""
    flag = ctypes.c_int32(-1)
    _check(load().sp_quest_step_single_launch(ctypes.byref(kv.desc), group_reduce, ctypes.byref(flag)))
    return flag.value == 1


def sp_sparse_decode_attn_noalloc(kv: PagedKV, q: torch.Tensor, sel_pages: Optional[torch.Tensor],
                                  top_k: int, scale: float, out: torch.Tensor,
                                  lse: Optional[torch.Tensor] = None,
                                  logits: Optional[torch.Tensor] = None, logit_cap: int = 0):
    _check(load().sp_sparse_decode_attn_noalloc(ctypes.byref(kv.desc), _ptr(q), _ptr(sel_pages), top_k,
                                                float(scale), _ptr(out), _ptr(lse), _ptr(logits),
                                                logit_cap, _stream()))


def sp_h2o_accumulate(kv: PagedKV, logits: torch.Tensor, lse: torch.Tensor, logit_cap: int,
                      n_new: int, scores: torch.Tensor, slot_cap: int):
    _check(load().sp_h2o_accumulate(ctypes.byref(kv.desc), _ptr(logits), _ptr(lse), logit_cap,
                                    n_new, _ptr(scores), slot_cap, _stream()))


def sp_decode_attn_accumulate(kv: PagedKV, q: torch.Tensor, scale: float, out: torch.Tensor,
                              lse: torch.Tensor, logits: torch.Tensor, logit_cap: int, n_new: int,
                              scores: torch.Tensor, slot_cap: int, ws: torch.Tensor):
    nbytes = ws.numel() * ws.element_size()
    _check(load().sp_decode_attn_accumulate(ctypes.byref(kv.desc), _ptr(q), float(scale), _ptr(out),
                                            _ptr(lse), _ptr(logits), logit_cap, n_new, _ptr(scores),
                                            slot_cap, _ptr(ws), nbytes, _stream()))


def sp_h2o_evict_compact(kv: PagedKV, scores: torch.Tensor, slot_pos: Optional[torch.Tensor],
                         slot_cap: int, budget: int, recent_window: int,
                         ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_h2o_evict_compact(ctypes.byref(kv.desc), _ptr(scores), _ptr(slot_pos),
                                       slot_cap, budget, recent_window, _ptr(ws), nbytes,
                                       _stream()))


def sp_snapkv_scores(kv: PagedKV, q_obs: torch.Tensor, n_obs: int, scale: float, pool_kernel: int,
                     n_sink: int, scores: torch.Tensor, slot_cap: int,
                     ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_snapkv_scores(ctypes.byref(kv.desc), _ptr(q_obs), n_obs, float(scale),
                                   pool_kernel, n_sink, _ptr(scores), slot_cap, _ptr(ws), nbytes,
                                   _stream()))


def sp_h2o_prefill_scores(kv: PagedKV, q_chunk: torch.Tensor, n_q: int, scale: float,
                          scores: torch.Tensor, slot_cap: int, ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_h2o_prefill_scores(ctypes.byref(kv.desc), _ptr(q_chunk), n_q, float(scale),
                                        _ptr(scores), slot_cap, _ptr(ws), nbytes, _stream()))


def sp_omnikv_select(kv: PagedKV, q: torch.Tensor, top_b: int, sel_pages: torch.Tensor,
                     sel_mask: torch.Tensor, k_pages: int, token_scores: torch.Tensor, slot_cap: int,
                     ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_omnikv_select(ctypes.byref(kv.desc), _ptr(q), top_b, _ptr(sel_pages), _ptr(sel_mask),
                                   k_pages, _ptr(token_scores), slot_cap, _ptr(ws), nbytes, _stream()))


def sp_sparse_decode_attn_masked(kv: PagedKV, q: torch.Tensor, sel_pages: torch.Tensor,
                                 sel_mask: torch.Tensor, top_k: int, scale: float, out: torch.Tensor,
                                 lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().sp_sparse_decode_attn_masked(ctypes.byref(kv.desc), _ptr(q), _ptr(sel_pages),
                                               _ptr(sel_mask), top_k, float(scale), _ptr(out), _ptr(lse),
                                               _ptr(ws), nbytes, _stream()))


# ------------------------------------------------------------------ layout views
# Index arithmetic for the documented pool layouts, used by tests to read
# slots back (pure indexing; no part of the computation).
def page_token_view(kv: PagedKV, blocks: torch.Tensor, head: int):
    """Logical (token, dim) views of the K and V pages of `blocks` for one KV
    head: returns (K [n_blocks][P][D], V [n_blocks][P][D])."""
    P, D = kv.page_size, kv.head_dim
    E = 16 // kv.k_pool.element_size()
    kraw = kv.k_pool[blocks.long(), head].reshape(-1, D // E, P, E)      # [n][D/E][P][E]
    kt = kraw.permute(0, 2, 1, 3).reshape(-1, P, D)
    vraw = kv.v_pool[blocks.long(), head].reshape(-1, D, P)             # [n][D][P]
    vt = vraw.permute(0, 2, 1)
    return kt, vt


def read_slots(kv: PagedKV, b: int, head: int, n: int):
    """K, V [n][D] of slots [0, n) of sequence b, KV head `head`."""
    P = kv.page_size
    n_pages = -(-n // P)
    blocks = kv.block_table[b, :n_pages]
    kt, vt = page_token_view(kv, blocks, head)
    return kt.reshape(-1, kv.head_dim)[:n], vt.reshape(-1, kv.head_dim)[:n]


def read_meta(kv: PagedKV, meta: torch.Tensor, b: int, head: int, n_pages: int):
    """(mins [n_pages][D], maxs [n_pages][D]) of sequence b's logical pages."""
    blocks = kv.block_table[b, :n_pages].long()
    m = meta[blocks, head]
    return m[:, 0], m[:, 1]
