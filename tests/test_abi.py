"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments on the host before launching
anything (every call below fails validation, so no kernel is ever started)."""
import ctypes
import os
import re

import pytest

import kv_cache_selection_sp_amd as sp
from kv_cache_selection_sp_amd._lib import SpPagedKV

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spdecode.h")

FAKE = 0x10000          # a 16-byte aligned non-NULL pointer value that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sp.LIB_PATH):
        pytest.fail("libspdecode.so is not built (python -m kv_cache_selection_sp_amd.build)")
    return sp.load()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(sp.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(sp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert lib.sp_version() == 100
    assert lib.sp_status_str(0) == b"SP_OK"
    assert lib.sp_status_str(5) == b"SP_ERR_WORKSPACE"
    assert lib.sp_status_str(99) == b"SP_ERR_UNKNOWN"


def make_desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                max_pages_per_seq=8, num_blocks=16, dtype=sp.SP_BF16, k_pool=FAKE,
                v_pool=FAKE + 4096, block_table=FAKE + 8192, seq_lens=FAKE + 12288)
    base.update(kw)
    return SpPagedKV(**base)


def call_meta(lib, d, k_new=FAKE, v_new=FAKE, n_new=1, meta=FAKE, pos=None, slot_pos=None,
              slot_cap=0):
    return lib.sp_build_page_meta(ctypes.byref(d) if d is not None else None, k_new, v_new,
                                  n_new, meta, pos, slot_pos, slot_cap, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k_pool=None), sp.SP_ERR_NULL_PTR),
    (dict(seq_lens=None), sp.SP_ERR_NULL_PTR),
    (dict(batch=0), sp.SP_ERR_BAD_SHAPE),
    (dict(num_q_heads=6, num_kv_heads=4), sp.SP_ERR_BAD_SHAPE),
    (dict(num_q_heads=34, num_kv_heads=2), sp.SP_ERR_UNSUPPORTED),      # G = 17
    (dict(head_dim=96), sp.SP_ERR_UNSUPPORTED),
    (dict(page_size=8), sp.SP_ERR_UNSUPPORTED),
    (dict(dtype=7), sp.SP_ERR_UNSUPPORTED),
    (dict(max_pages_per_seq=0), sp.SP_ERR_BAD_SHAPE),
    (dict(max_pages_per_seq=1 << 27, page_size=16), sp.SP_ERR_BAD_SHAPE),  # capacity > 2^30
    (dict(k_pool=FAKE + 8), sp.SP_ERR_MISALIGNED),
    (dict(seq_lens=FAKE + 2), sp.SP_ERR_MISALIGNED),
])
def test_descriptor_validation(lib, kw, code):
    d = make_desc(**kw)
    assert call_meta(lib, d) == code
    assert lib.sp_last_error() != b""


def test_null_descriptor(lib):
    assert call_meta(lib, None) == sp.SP_ERR_NULL_PTR
    assert b"NULL" in lib.sp_last_error()


def test_build_page_meta_validation(lib):
    d = make_desc()
    assert call_meta(lib, d, n_new=-1) == sp.SP_ERR_BAD_SHAPE
    assert call_meta(lib, d, k_new=None) == sp.SP_ERR_NULL_PTR
    assert call_meta(lib, d, k_new=FAKE + 4) == sp.SP_ERR_MISALIGNED
    assert call_meta(lib, d, meta=FAKE + 8) == sp.SP_ERR_MISALIGNED
    # rebuild mode takes no new tokens and needs the summaries
    assert call_meta(lib, d, n_new=0) == sp.SP_ERR_BAD_SHAPE
    assert call_meta(lib, d, n_new=0, k_new=None, v_new=None, meta=None) == sp.SP_ERR_NULL_PTR
    # slot map narrower than the capacity (8 pages * 16 = 128 slots)
    assert call_meta(lib, d, slot_pos=FAKE, slot_cap=127) == sp.SP_ERR_BAD_SHAPE
    assert call_meta(lib, d, slot_pos=FAKE + 2, slot_cap=128) == sp.SP_ERR_MISALIGNED


def test_select_pages_validation(lib):
    d = make_desc()
    need = lib.sp_workspace_bytes(sp.SP_OP_SELECT_PAGES, ctypes.byref(d), 4)
    # 256-byte-rounded arrival counters, then the (sequence, KV head, page) scores
    assert need == 256 + 2 * 2 * 8 * 4

    def call(q=FAKE, meta=FAKE, k=4, sel=FAKE, scores=None, ws=FAKE, nbytes=need, desc=d):
        return lib.sp_select_pages(ctypes.byref(desc), q, meta, k, sel, scores, ws, nbytes, None)
    assert call(q=None) == sp.SP_ERR_NULL_PTR
    assert call(sel=None) == sp.SP_ERR_NULL_PTR
    assert call(k=0) == sp.SP_ERR_BAD_SHAPE
    assert call(q=FAKE + 8) == sp.SP_ERR_MISALIGNED
    assert call(ws=None) == sp.SP_ERR_WORKSPACE
    assert call(ws=None, scores=FAKE) == sp.SP_ERR_WORKSPACE     # needed even with page_scores
    assert call(nbytes=need - 1) == sp.SP_ERR_WORKSPACE
    assert b"workspace" in lib.sp_last_error()
    # rows longer than the select launch's own top-k (10 keys of 512 threads):
    # the scores 256-byte rounded, then the page counts of the separate top-k
    # launch (up to 32 keys of 1024 threads), and beyond that the per-unit
    # lists of the threshold search (header, 2048 bins, two counts per
    # 4096-page slice, up to every page)
    up = lambda x: (x + 255) // 256 * 256
    ws = lambda mp: lib.sp_workspace_bytes(sp.SP_OP_SELECT_PAGES, ctypes.byref(make_desc(max_pages_per_seq=mp)), 4)
    assert ws(5120) == 256 + 2 * 2 * 5120 * 4
    assert ws(5121) == 256 + up(2 * 2 * 5121 * 4) + up(2 * 4)
    assert ws(32768) == 256 + up(2 * 2 * 32768 * 4) + up(2 * 4)
    assert ws(32769) == 256 + up(2 * 2 * 32769 * 4) + up(2 * 4) + 2 * 2 * (16 + 2048 + 2 * 9 + 32769) * 4
    dl = make_desc(max_pages_per_seq=32769)
    assert call(desc=dl, nbytes=ws(32769) - 1) == sp.SP_ERR_WORKSPACE


def test_select_pages_ex_validation(lib):
    d = make_desc()                       # 4 query heads per KV head
    need = lib.sp_workspace_bytes(sp.SP_OP_SELECT_PAGES, ctypes.byref(d), 4)

    def call(k=4, n_sink=0, n_recent=0, red=sp.SP_GROUP_SUM, desc=d):
        return lib.sp_select_pages_ex(ctypes.byref(desc), FAKE, FAKE, k, n_sink, n_recent, red, FAKE,
                                      None, None, 0, None)
    # every call below fails validation; the first two only on the workspace
    assert call() == sp.SP_ERR_WORKSPACE
    assert call(n_sink=2, n_recent=2) == sp.SP_ERR_WORKSPACE          # 2 + 2 <= 4 is fine
    assert call(n_sink=3, n_recent=2) == sp.SP_ERR_BAD_SHAPE          # 5 forced > top_k
    assert call(n_sink=-1) == sp.SP_ERR_BAD_SHAPE
    assert call(n_recent=-1) == sp.SP_ERR_BAD_SHAPE
    assert call(red=2) == sp.SP_ERR_BAD_SHAPE
    assert call(red=sp.SP_GROUP_MAX) == sp.SP_ERR_WORKSPACE
    # the maximum over up to 16 query heads per KV head (the group size limit)
    assert call(red=sp.SP_GROUP_MAX, desc=make_desc(num_q_heads=32, num_kv_heads=2)) == sp.SP_ERR_WORKSPACE
    assert call(red=sp.SP_GROUP_MAX, desc=make_desc(num_q_heads=34, num_kv_heads=2)) == sp.SP_ERR_UNSUPPORTED
    assert need > 0


def test_append_select_validation(lib):
    d = make_desc()                       # 2 sequences x 2 KV heads, capacity 128
    need = lib.sp_workspace_bytes(sp.SP_OP_SELECT_PAGES, ctypes.byref(d), 4)
    # per-unit and per-sequence counters (256-byte rounded), then the scores
    assert need >= 256 + 2 * 2 * 8 * 4

    def call(kn=FAKE, vn=FAKE, pos=None, slot=None, cap=0, meta=FAKE, q=FAKE, k=4, n_sink=0, n_recent=0,
             red=sp.SP_GROUP_SUM, sel=FAKE, ws=FAKE, nbytes=need):
        return lib.sp_append_select_pages(ctypes.byref(d), kn, vn, pos, slot, cap, meta, q, k, n_sink,
                                          n_recent, red, sel, None, ws, nbytes, None)
    assert call(kn=None) == sp.SP_ERR_NULL_PTR
    assert call(vn=None) == sp.SP_ERR_NULL_PTR
    assert call(meta=None) == sp.SP_ERR_NULL_PTR
    assert call(q=None) == sp.SP_ERR_NULL_PTR
    assert call(sel=None) == sp.SP_ERR_NULL_PTR
    assert call(kn=FAKE + 8) == sp.SP_ERR_MISALIGNED
    assert call(pos=FAKE + 2) == sp.SP_ERR_MISALIGNED
    assert call(slot=FAKE, cap=64) == sp.SP_ERR_BAD_SHAPE
    assert call(k=0) == sp.SP_ERR_BAD_SHAPE
    assert call(n_sink=3, n_recent=2) == sp.SP_ERR_BAD_SHAPE
    assert call(red=2) == sp.SP_ERR_BAD_SHAPE
    assert call(ws=None) == sp.SP_ERR_WORKSPACE
    assert call(nbytes=need - 4) == sp.SP_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == sp.SP_ERR_MISALIGNED


def test_quest_step_validation(lib):
    """sp_quest_decode_step checks the arguments of the append, the selection
    and the attention it stands for, plus its own workspace and block-id
    width; the form query checks its own arguments."""
    d = make_desc()
    need = lib.sp_workspace_bytes(sp.SP_OP_QUEST_STEP, ctypes.byref(d), 4)
    assert need >= lib.sp_workspace_bytes(sp.SP_OP_SELECT_PAGES, ctypes.byref(d), 4)

    def call(desc=d, kn=FAKE, vn=FAKE, meta=FAKE, q=FAKE, k=4, n_sink=0, n_recent=0, red=sp.SP_GROUP_SUM,
             scale=0.1, sel=FAKE, out=FAKE, lse=None, ws=FAKE, nbytes=need):
        return lib.sp_quest_decode_step(ctypes.byref(desc), kn, vn, None, None, 0, meta, q, k, n_sink, n_recent,
                                        red, scale, sel, None, out, lse, ws, nbytes, None)
    assert call(kn=None) == sp.SP_ERR_NULL_PTR            # exactly one of k_new, v_new
    assert call(meta=None) == sp.SP_ERR_NULL_PTR
    assert call(sel=None) == sp.SP_ERR_NULL_PTR
    assert call(out=None) == sp.SP_ERR_NULL_PTR
    assert call(k=0) == sp.SP_ERR_BAD_SHAPE
    assert call(red=2) == sp.SP_ERR_BAD_SHAPE
    assert call(scale=float("nan")) == sp.SP_ERR_BAD_SHAPE
    assert call(kn=FAKE + 8) == sp.SP_ERR_MISALIGNED
    assert call(ws=None) == sp.SP_ERR_WORKSPACE
    assert call(nbytes=need - 4) == sp.SP_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == sp.SP_ERR_MISALIGNED
    wide = make_desc(num_blocks=1 << 25)
    assert call(desc=wide, nbytes=lib.sp_workspace_bytes(sp.SP_OP_QUEST_STEP, ctypes.byref(wide), 4)) \
        == sp.SP_ERR_UNSUPPORTED
    # the error word sits after the counters and epochs: 2 x 3 select counters,
    # 4 attention counters and 4 epochs, each area rounded up to 256 bytes
    assert lib.sp_quest_step_error_offset(ctypes.byref(d)) == 3 * 256
    flag = ctypes.c_int32(-1)
    assert lib.sp_quest_step_single_launch(ctypes.byref(d), sp.SP_GROUP_SUM, None) == sp.SP_ERR_NULL_PTR
    assert lib.sp_quest_step_single_launch(ctypes.byref(d), 2, ctypes.byref(flag)) == sp.SP_ERR_BAD_SHAPE
    assert lib.sp_quest_step_single_launch(None, sp.SP_GROUP_SUM, ctypes.byref(flag)) == sp.SP_ERR_NULL_PTR
    assert flag.value == -1


def test_decode_attn_validation(lib):
    d = make_desc()
    need_sparse = lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(d), 4)
    need_dense = lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(d), 0)
    assert need_sparse > 0 and need_dense > 0

    def call(q=FAKE, sel=FAKE, k=4, scale=0.1, out=FAKE, lse=None, logits=None, cap=0,
             ws=FAKE, nbytes=need_sparse):
        return lib.sp_sparse_decode_attn(ctypes.byref(d), q, sel, k, scale, out, lse, logits,
                                         cap, ws, nbytes, None)
    assert call(out=None) == sp.SP_ERR_NULL_PTR
    assert call(k=0) == sp.SP_ERR_BAD_SHAPE
    assert call(scale=float("nan")) == sp.SP_ERR_BAD_SHAPE
    assert call(logits=FAKE, cap=128) == sp.SP_ERR_UNSUPPORTED       # logits need dense mode
    assert call(sel=None, logits=FAKE, cap=100, nbytes=need_dense) == sp.SP_ERR_BAD_SHAPE
    assert call(nbytes=need_sparse - 4) == sp.SP_ERR_WORKSPACE
    assert call(sel=None, nbytes=need_dense - 4) == sp.SP_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == sp.SP_ERR_MISALIGNED


def test_decode_attn_noalloc_validation(lib):
    """The allocation-free form checks like sp_sparse_decode_attn and rejects
    shapes beyond its scratch array before it looks the array up."""
    d = make_desc()

    def call(desc=d, q=FAKE, sel=FAKE, k=4, scale=0.1, out=FAKE, lse=None, logits=None, cap=0):
        return lib.sp_sparse_decode_attn_noalloc(ctypes.byref(desc), q, sel, k, scale, out, lse, logits,
                                                 cap, None)
    assert call(out=None) == sp.SP_ERR_NULL_PTR
    assert call(q=None) == sp.SP_ERR_NULL_PTR
    assert call(k=0) == sp.SP_ERR_BAD_SHAPE
    assert call(scale=float("inf")) == sp.SP_ERR_BAD_SHAPE
    assert call(logits=FAKE, cap=128) == sp.SP_ERR_UNSUPPORTED       # logits need dense mode
    assert call(q=FAKE + 4) == sp.SP_ERR_MISALIGNED
    # more (sequence, KV head) units than the counter area holds
    big = make_desc(batch=2048, num_q_heads=64, num_kv_heads=16)
    assert call(desc=big, sel=FAKE) == sp.SP_ERR_UNSUPPORTED
    assert b"allocation-free" in lib.sp_last_error()
    # records beyond the array: G = 16, 8 KV heads, 1024 sequences in dense mode
    big2 = make_desc(batch=1024, num_q_heads=128, num_kv_heads=8, max_pages_per_seq=64)
    assert call(desc=big2, sel=None) == sp.SP_ERR_UNSUPPORTED


def test_h2o_validation(lib):
    d = make_desc()
    acc = lambda **kw: lib.sp_h2o_accumulate(
        ctypes.byref(d), kw.get("logits", FAKE), kw.get("lse", FAKE), kw.get("lcap", 128),
        kw.get("n_new", 1), kw.get("scores", FAKE), kw.get("scap", 128), None)
    assert acc(scores=None) == sp.SP_ERR_NULL_PTR
    assert acc(n_new=-1) == sp.SP_ERR_BAD_SHAPE
    assert acc(lcap=64) == sp.SP_ERR_BAD_SHAPE
    assert acc(scap=64) == sp.SP_ERR_BAD_SHAPE
    ev = lambda **kw: lib.sp_h2o_evict_compact(
        ctypes.byref(d), kw.get("scores", FAKE), kw.get("pos", None), kw.get("scap", 128),
        kw.get("budget", 16), kw.get("window", 4), None, 0, None)
    assert ev(scores=None) == sp.SP_ERR_NULL_PTR
    assert ev(budget=0) == sp.SP_ERR_BAD_SHAPE
    assert ev(window=17) == sp.SP_ERR_BAD_SHAPE
    assert ev(window=-1) == sp.SP_ERR_BAD_SHAPE
    assert ev(scap=100) == sp.SP_ERR_BAD_SHAPE
    assert ev(pos=FAKE + 1) == sp.SP_ERR_MISALIGNED
    # up to 8192 slots of capacity the workspace is optional: one counter per
    # sequence (256-byte rounded) fuses the length update into the kernel
    assert lib.sp_workspace_bytes(sp.SP_OP_H2O_EVICT, ctypes.byref(d), 0) == 256
    evs = lambda ws, nbytes: lib.sp_h2o_evict_compact(ctypes.byref(d), FAKE, None, 128, 16, 4, ws, nbytes, None)
    assert evs(FAKE + 8, 256) == sp.SP_ERR_MISALIGNED
    # above 8192 slots of capacity the compaction keeps a list of the kept slots
    big = make_desc(max_pages_per_seq=600)                     # 9600 slots
    need = lib.sp_workspace_bytes(sp.SP_OP_H2O_EVICT, ctypes.byref(big), 1000)
    # per unit: 16-int header, 2048-bin histogram, two counts per 4096-slot
    # slice, the list; then (256-byte aligned) per unit the low moves'
    # scratch for budget rounded up to 64 slots: K rows and V groups of D bf16
    # elements, a score and a position per slot, 256-byte rounded
    per_unit = lambda bud: 16 + 2048 + 2 * 3 + bud
    up = lambda x, a: (x + a - 1) // a * a
    scratch = lambda bud: up(up(bud, 64) * (128 * 2 * 2 + 8), 256)
    assert need == up(2 * 2 * per_unit(1000) * 4, 256) + 2 * 2 * scratch(1000)
    # a budget of the capacity or more is sized as the capacity
    assert lib.sp_workspace_bytes(sp.SP_OP_H2O_EVICT, ctypes.byref(big), 0) == \
        up(2 * 2 * per_unit(9600) * 4, 256) + 2 * 2 * scratch(9600)
    assert lib.sp_workspace_bytes(sp.SP_OP_H2O_EVICT, ctypes.byref(big), 20000) == \
        lib.sp_workspace_bytes(sp.SP_OP_H2O_EVICT, ctypes.byref(big), 9600)
    evb = lambda ws, nbytes: lib.sp_h2o_evict_compact(ctypes.byref(big), FAKE, None, 9600, 1000, 8, ws,
                                                       nbytes, None)
    assert evb(None, 0) == sp.SP_ERR_WORKSPACE
    assert evb(FAKE, need - 4) == sp.SP_ERR_WORKSPACE
    assert evb(FAKE + 8, need) == sp.SP_ERR_MISALIGNED


def test_workspace_bytes_edge_cases(lib):
    d = make_desc()
    assert lib.sp_workspace_bytes(42, ctypes.byref(d), 4) == 0
    assert lib.sp_workspace_bytes(sp.SP_OP_SELECT_PAGES, None, 4) == 0
    bad = make_desc(head_dim=80)
    assert lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(bad), 4) == 0
    # the attention workspace: 256-byte-rounded per-(sequence, KV head) arrival
    # counters, then whole (acc[D], m, l) records for the G heads of a group
    counters = 256
    group_rec = 4 * (128 + 2) * 4
    for top_k in (1, 4, 8):
        n = lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(d), top_k)
        assert n > counters and (n - counters) % group_rec == 0
        # at least one record per unit plus one per workgroup
        assert (n - counters) // group_rec >= 2 * 2 + 1
    dense = lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(d), 0)
    assert dense > counters and (dense - counters) % group_rec == 0


def test_snapkv_scores_validation(lib):
    d = make_desc()                       # 4 query heads per KV head, capacity 128
    need = lib.sp_workspace_bytes(sp.SP_OP_SNAPKV_SCORES, ctypes.byref(d), 32)
    assert need > 0
    assert lib.sp_workspace_bytes(sp.SP_OP_SNAPKV_SCORES, ctypes.byref(d), 0) == 0

    def call(q=FAKE, w=32, scale=0.1, kappa=7, n_sink=0, scores=FAKE, scap=128, ws=FAKE,
             nbytes=need, desc=d):
        return lib.sp_snapkv_scores(ctypes.byref(desc), q, w, scale, kappa, n_sink, scores, scap,
                                    ws, nbytes, None)
    # every call below fails validation
    assert call(q=None) == sp.SP_ERR_NULL_PTR
    assert call(scores=None) == sp.SP_ERR_NULL_PTR
    assert call(desc=make_desc(dtype=sp.SP_F32)) == sp.SP_ERR_UNSUPPORTED
    assert call(w=0) == sp.SP_ERR_BAD_SHAPE
    assert call(w=1025) == sp.SP_ERR_BAD_SHAPE                 # G * w > 4096
    assert call(scale=0.0) == sp.SP_ERR_BAD_SHAPE
    assert call(scale=float("inf")) == sp.SP_ERR_BAD_SHAPE
    assert call(kappa=0) == sp.SP_ERR_BAD_SHAPE
    assert call(kappa=258) == sp.SP_ERR_BAD_SHAPE
    assert call(n_sink=-1) == sp.SP_ERR_BAD_SHAPE
    assert call(scap=127) == sp.SP_ERR_BAD_SHAPE
    assert call(q=FAKE + 8) == sp.SP_ERR_MISALIGNED
    assert call(scores=FAKE + 2) == sp.SP_ERR_MISALIGNED
    assert call(ws=None) == sp.SP_ERR_WORKSPACE
    assert call(nbytes=need - 1) == sp.SP_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == sp.SP_ERR_MISALIGNED
    # more window rows need more per-row state
    assert lib.sp_workspace_bytes(sp.SP_OP_SNAPKV_SCORES, ctypes.byref(d), 128) > need


def test_h2o_prefill_scores_validation(lib):
    d = make_desc()                       # 4 query heads per KV head, capacity 128
    need = lib.sp_workspace_bytes(sp.SP_OP_H2O_PREFILL, ctypes.byref(d), 64)
    assert need > 0
    # a small cache: one pass holds every row, so the workspace grows with n_q
    assert (lib.sp_workspace_bytes(sp.SP_OP_H2O_PREFILL, ctypes.byref(d), 5000)
            > lib.sp_workspace_bytes(sp.SP_OP_H2O_PREFILL, ctypes.byref(d), 1024))
    # a cache whose column sums fill 256 MiB per 16 slabs (2 x 2 units x 2^20
    # slots): passes of 16 slabs (4096 rows, n_q = 1024 at G = 4), so more
    # chunk queries still use one pass's workspace
    wide = make_desc(max_pages_per_seq=1 << 16)
    assert (lib.sp_workspace_bytes(sp.SP_OP_H2O_PREFILL, ctypes.byref(wide), 5000)
            == lib.sp_workspace_bytes(sp.SP_OP_H2O_PREFILL, ctypes.byref(wide), 1024))

    def call(q=FAKE, n=64, scale=0.1, scores=FAKE, scap=128, ws=FAKE, nbytes=need, desc=d):
        return lib.sp_h2o_prefill_scores(ctypes.byref(desc), q, n, scale, scores, scap, ws, nbytes, None)
    assert call(q=None) == sp.SP_ERR_NULL_PTR
    assert call(scores=None) == sp.SP_ERR_NULL_PTR
    assert call(desc=make_desc(dtype=sp.SP_F32)) == sp.SP_ERR_UNSUPPORTED
    assert call(n=0) == sp.SP_ERR_BAD_SHAPE
    assert call(n=65537) == sp.SP_ERR_BAD_SHAPE
    assert call(scale=-1.0) == sp.SP_ERR_BAD_SHAPE
    assert call(scap=100) == sp.SP_ERR_BAD_SHAPE
    assert call(q=FAKE + 4) == sp.SP_ERR_MISALIGNED
    assert call(ws=None) == sp.SP_ERR_WORKSPACE
    assert call(nbytes=need - 16) == sp.SP_ERR_WORKSPACE


def test_omnikv_and_masked_attention_validation(lib):
    d = make_desc()                       # 8 pages of 16 slots, capacity 128
    need = lib.sp_workspace_bytes(sp.SP_OP_OMNIKV_SELECT, ctypes.byref(d), 20)
    assert need > 0

    def sel(q=FAKE, b=20, pages=FAKE, mask=FAKE, kp=8, scores=FAKE, scap=128, ws=FAKE, nbytes=need, desc=d):
        return lib.sp_omnikv_select(ctypes.byref(desc), q, b, pages, mask, kp, scores, scap, ws, nbytes, None)
    assert sel(mask=None) == sp.SP_ERR_NULL_PTR
    assert sel(scores=None) == sp.SP_ERR_NULL_PTR
    assert sel(desc=make_desc(dtype=sp.SP_F32)) == sp.SP_ERR_UNSUPPORTED
    assert sel(desc=make_desc(num_q_heads=256, num_kv_heads=2)) == sp.SP_ERR_UNSUPPORTED
    assert sel(desc=make_desc(num_q_heads=34, num_kv_heads=2)) == sp.SP_ERR_UNSUPPORTED   # 17 per KV head
    assert sel(b=0) == sp.SP_ERR_BAD_SHAPE
    assert sel(b=3, kp=2) == sp.SP_ERR_BAD_SHAPE            # 3 slots may span 3 pages
    assert sel(kp=7) == sp.SP_ERR_BAD_SHAPE                 # min(20, 8 pages) = 8
    assert sel(scap=64) == sp.SP_ERR_BAD_SHAPE
    assert sel(q=FAKE + 2) == sp.SP_ERR_MISALIGNED
    assert sel(ws=None) == sp.SP_ERR_WORKSPACE
    assert sel(nbytes=need - 4) == sp.SP_ERR_WORKSPACE

    need_a = lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(d), 4)

    def att(q=FAKE, pages=FAKE, mask=FAKE, k=4, ws=FAKE, nbytes=need_a):
        return lib.sp_sparse_decode_attn_masked(ctypes.byref(d), q, pages, mask, k, 0.1, FAKE, None, ws,
                                                nbytes, None)
    assert att(mask=None) == sp.SP_ERR_NULL_PTR
    assert att(pages=None) == sp.SP_ERR_NULL_PTR
    assert att(k=0) == sp.SP_ERR_BAD_SHAPE
    assert att(mask=FAKE + 2) == sp.SP_ERR_MISALIGNED
    assert att(nbytes=need_a - 4) == sp.SP_ERR_WORKSPACE


def test_decode_attn_accumulate_argument_checks(lib):
    """The fused dense attention + H2O update checks what its two calls check."""
    d = make_desc()
    ws_need = lib.sp_workspace_bytes(sp.SP_OP_DECODE_ATTN, ctypes.byref(d), 0)
    call = lambda **kw: lib.sp_decode_attn_accumulate(
        ctypes.byref(d), kw.get("q", FAKE), kw.get("scale", 0.1), kw.get("out", FAKE), kw.get("lse", FAKE),
        kw.get("logits", FAKE), kw.get("lcap", 128), kw.get("n_new", 1), kw.get("scores", FAKE),
        kw.get("scap", 128), kw.get("ws", FAKE), kw.get("nbytes", ws_need), None)
    assert call(lse=None) == sp.SP_ERR_NULL_PTR
    assert call(logits=None) == sp.SP_ERR_NULL_PTR
    assert call(scores=None) == sp.SP_ERR_NULL_PTR
    assert call(q=FAKE + 8) == sp.SP_ERR_MISALIGNED
    assert call(scores=FAKE + 2) == sp.SP_ERR_MISALIGNED
    assert call(n_new=-1) == sp.SP_ERR_BAD_SHAPE
    assert call(lcap=64) == sp.SP_ERR_BAD_SHAPE
    assert call(scap=64) == sp.SP_ERR_BAD_SHAPE
    assert call(scale=float("inf")) == sp.SP_ERR_BAD_SHAPE
    assert call(ws=None, nbytes=0) == sp.SP_ERR_WORKSPACE
    assert call(nbytes=ws_need - 4) == sp.SP_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == sp.SP_ERR_MISALIGNED
