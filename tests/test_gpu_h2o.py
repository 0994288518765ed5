"""GPU parity for H2O: dense attention with logits, score accumulation and
eviction with physical compaction, teacher-forced step by step against the
oracle (each step starts from the oracle's state), plus a free-running run
checked by invariants."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import f64, new_cache, bulk_append
from oracle import H2OHeadState, h2o_retain
from oracle.h2o import h2o_append, h2o_attend_accumulate, h2o_evict, h2o_prefill_chunk

pytestmark = pytest.mark.gpu


class H2OCase:
    """A small H2O layer: GPU buffers plus the oracle's per-(b, h) states."""

    def __init__(self, B=2, Hq=8, Hkv=2, D=128, P=16, prompt=300, budget=64, window=8,
                 steps=6, seed=5, dtype="bf16"):
        self.cfg = W.H2OConfig("t", dtype, B, Hq, Hkv, D, prompt, budget, window, steps, page_size=P)
        self.x = W.h2o_inputs(self.cfg, seed, device="cuda")
        self.B, self.Hq, self.Hkv, self.D, self.P, self.G = B, Hq, Hkv, D, P, Hq // Hkv
        self.budget, self.window = budget, window
        self.dt = W.torch_dtype(dtype)
        self.scale = W.default_scale(D)
        self.kv = new_cache(B, Hq, Hkv, D, P, self.x["max_pages"], self.dt, self.x["block_table"],
                            num_blocks=self.x["num_blocks"])
        self.cap = self.kv.capacity
        self.scores = torch.zeros(B, Hkv, self.cap, dtype=torch.float32, device="cuda")
        self.slot_pos = torch.full((B, Hkv, self.cap), -1, dtype=torch.int32, device="cuda")
        self.ws = sp.workspace(sp.SP_OP_H2O_EVICT, self.kv, budget)
        # the prompt's scores: its own queries' causal attention probabilities
        # (one prefill chunk, before any eviction), from the oracle
        empty = H2OHeadState(np.zeros(0, np.int64), np.zeros((0, D)), np.zeros((0, D)), np.zeros(0))
        self.states = [[h2o_prefill_chunk(empty, self.x["q_prompt"][b, :, h * self.G:(h + 1) * self.G].cpu(),
                                          np.arange(prompt), self.x["keys"][b, h].cpu(),
                                          self.x["values"][b, h].cpu(), self.scale)
                        for h in range(Hkv)] for b in range(B)]

    def evict(self, budget=None, window=None):
        budget = self.budget if budget is None else budget
        window = self.window if window is None else window
        sp.sp_h2o_evict_compact(self.kv, self.scores, self.slot_pos, self.cap, budget, window, self.ws)

    def load(self):
        """Teacher forcing: write the oracle states (equal sizes) into the GPU
        cache through the library's append, then set positions and scores."""
        n = len(self.states[0][0])
        self.kv.seq_lens.zero_()
        keys = torch.stack([torch.stack([torch.as_tensor(st.keys) for st in row]) for row in self.states])
        vals = torch.stack([torch.stack([torch.as_tensor(st.values) for st in row]) for row in self.states])
        bulk_append(self.kv, keys.to("cuda", self.dt), vals.to("cuda", self.dt))
        for b in range(self.B):
            for h in range(self.Hkv):
                st = self.states[b][h]
                # the GPU keeps fp32 scores: the oracle continues from the same rounded values
                st.scores = st.scores.astype(np.float32).astype(np.float64)
                self.slot_pos[b, h, :n] = torch.as_tensor(st.positions, dtype=torch.int32)
                self.scores[b, h, :n] = torch.as_tensor(st.scores, dtype=torch.float32)

    def check_retained(self, before, n_after, gpu_scores_before=None):
        """Compare the GPU's retained slots with the oracle under the cutoff rule."""
        torch.cuda.synchronize()
        kept_lens = self.kv.seq_lens.cpu()
        for b in range(self.B):
            assert int(kept_lens[b]) == n_after
            for h in range(self.Hkv):
                st = before[b][h]
                n = len(st)
                pos = self.slot_pos[b, h, :n_after].cpu().numpy()
                assert np.all(np.diff(pos) > 0)
                W_ = self.window
                win = set(st.positions[n - W_:].tolist()) if W_ else set()
                assert win <= set(pos.tolist())
                cand = np.arange(n - W_)
                keep_c = self.budget - W_
                S = st.scores[cand]
                if n > self.budget and keep_c > 0 and len(cand) > keep_c:
                    cut = np.sort(S)[::-1][keep_c - 1]
                    tol = 1e-5 * max(abs(cut), 1.0)
                    must = set(st.positions[cand[S > cut + tol]].tolist())
                    never = set(st.positions[cand[S < cut - tol]].tolist())
                    got = set(pos.tolist()) - win
                    assert must <= got and not (never & got)
                # payload of every retained slot is the token of its position
                kk, vv = sp.read_slots(self.kv, b, h, n_after)
                idx = {int(p): j for j, p in enumerate(st.positions)}
                rows = [idx[int(p)] for p in pos]
                assert np.array_equal(f64(kk), st.keys[rows])
                assert np.array_equal(f64(vv), st.values[rows])
                # scores moved with their slots
                if gpu_scores_before is not None:
                    np.testing.assert_array_equal(self.scores[b, h, :n_after].cpu().numpy(),
                                                  gpu_scores_before[b][h][rows])


# Slot capacities up to 8192 take the LDS-resident eviction path; larger ones
# take the list path (kept-slot list in a workspace, then the entries whose
# sources lie below the budget gathered into a scratch area before any slot
# is written, then every entry moved in parallel).
# In bf16 the recent window's V moves as a shift of 16-byte chunks by
# (prompt - budget) slots: 600 and 603 slots are shifts of 0 and 3 tokens
# within a chunk; P = 32 has four chunks per dim row.  The list-path cases
# cover many low entries (budget 1003, skewed scores; budget 8190 of 8500,
# where each gather and move workgroup takes several passes), a budget that is
# not a multiple of the 16-byte token groups, fp32 and P = 32.
@pytest.mark.parametrize("prompt,B,Hq,D,P,dtype,budget,window", [
    (700, 2, 8, 128, 16, "bf16", 100, 10), (703, 2, 8, 128, 16, "bf16", 100, 10),
    (703, 2, 8, 64, 32, "bf16", 100, 10), (700, 2, 8, 64, 16, "f32", 100, 10),
    (8300, 1, 4, 64, 16, "bf16", 100, 10), (9000, 2, 8, 128, 16, "bf16", 1003, 37),
    (8300, 1, 4, 64, 32, "f32", 700, 64), (8500, 1, 4, 128, 16, "bf16", 8190, 5)])
def test_initial_prompt_compaction_matches_oracle(prompt, B, Hq, D, P, dtype, budget, window):
    c = H2OCase(B=B, Hq=Hq, D=D, P=P, prompt=prompt, budget=budget, window=window, dtype=dtype)
    assert (c.cap <= 8192) == (prompt <= 8192)
    c.load()
    before = [[st.copy() for st in row] for row in c.states]
    gpu_before = c.scores.cpu().numpy()
    c.evict()
    c.check_retained(before, c.budget, gpu_before)
    # exact agreement with the oracle's retained positions (fp32 scores, no ties here)
    for b in range(c.B):
        for h in range(c.Hkv):
            keep = h2o_retain(before[b][h].positions, before[b][h].scores, c.budget, c.window)
            assert c.slot_pos[b, h, :c.budget].cpu().tolist() == before[b][h].positions[keep].tolist()


# Windows up to 128 slots are read ahead while the threshold is found (bf16);
# window 0 and larger windows move with the other kept slots.
@pytest.mark.parametrize("prompt,budget,window", [(200, 64, 0), (200, 64, 8), (200, 64, 64),
                                                  (600, 300, 200)])
def test_teacher_forced_decode_steps(prompt, budget, window):
    c = H2OCase(prompt=prompt, budget=budget, window=window, steps=5)
    for b in range(c.B):
        for h in range(c.Hkv):
            c.states[b][h] = h2o_evict(c.states[b][h], c.budget, c.window)
    G, D = c.G, c.D
    for s in range(c.cfg.steps):
        i = c.cfg.prompt + s
        c.load()
        n0 = len(c.states[0][0])
        pos_new = torch.full((c.B,), i, dtype=torch.int32, device="cuda")
        sp.sp_build_page_meta(c.kv, c.x["k_new"][s][:, None].contiguous(),
                              c.x["v_new"][s][:, None].contiguous(), 1, None, pos_new,
                              c.slot_pos, c.cap)
        q = c.x["q"][s].contiguous()
        out = torch.empty(c.B, c.Hq, D, device="cuda")
        lse = torch.empty(c.B, c.Hq, device="cuda")
        logits = torch.full((c.B, c.Hq, c.cap), float("nan"), device="cuda")
        ws = sp.workspace(sp.SP_OP_DECODE_ATTN, c.kv, 0)
        sp.sp_sparse_decode_attn(c.kv, q, None, 0, c.scale, out, lse, logits, c.cap, ws)
        sp.sp_h2o_accumulate(c.kv, logits, lse, c.cap, 1, c.scores, c.cap)
        torch.cuda.synchronize()
        gpu_acc = c.scores.cpu().numpy().copy()
        appended = [[None] * c.Hkv for _ in range(c.B)]
        for b in range(c.B):
            for h in range(c.Hkv):
                app = h2o_append(c.states[b][h], i, c.x["k_new"][s, b, h].cpu(), c.x["v_new"][s, b, h].cpu())
                acc, o, l, z, _ = h2o_attend_accumulate(app, f64(q[b, h * G:(h + 1) * G]), c.scale)
                np.testing.assert_allclose(f64(out[b, h * G:(h + 1) * G]), o, atol=2e-3)
                np.testing.assert_allclose(f64(lse[b, h * G:(h + 1) * G]), l, atol=2e-3)
                np.testing.assert_allclose(f64(logits[b, h * G:(h + 1) * G, :n0 + 1]), z, atol=1e-4)
                # accumulated scores: fp32 sums of fp32 probabilities
                np.testing.assert_allclose(gpu_acc[b, h, :n0 + 1], acc.scores,
                                           rtol=1e-5, atol=1e-6)
                assert c.slot_pos[b, h, n0].item() == i
                appended[b][h] = acc
        c.evict()
        c.check_retained(appended, min(n0 + 1, c.budget), gpu_acc)
        for b in range(c.B):
            for h in range(c.Hkv):
                c.states[b][h] = h2o_evict(appended[b][h], c.budget, c.window)


def test_free_running_invariants():
    c = H2OCase(prompt=160, budget=48, window=6, steps=24, seed=9)
    c.load()
    c.evict()
    keys_by_pos = {}
    for b in range(c.B):
        for h in range(c.Hkv):
            for p in range(c.cfg.prompt):
                keys_by_pos[(b, h, p)] = c.x["keys"][b, h, p]
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, c.kv, 0)
    for s in range(c.cfg.steps):
        i = c.cfg.prompt + s
        pos_new = torch.full((c.B,), i, dtype=torch.int32, device="cuda")
        sp.sp_build_page_meta(c.kv, c.x["k_new"][s][:, None].contiguous(),
                              c.x["v_new"][s][:, None].contiguous(), 1, None, pos_new,
                              c.slot_pos, c.cap)
        for b in range(c.B):
            for h in range(c.Hkv):
                keys_by_pos[(b, h, i)] = c.x["k_new"][s, b, h]
        before = c.scores[:, :, :c.budget].double().sum(-1)
        out = torch.empty(c.B, c.Hq, c.D, device="cuda")
        lse = torch.empty(c.B, c.Hq, device="cuda")
        logits = torch.empty(c.B, c.Hq, c.cap, device="cuda")
        sp.sp_sparse_decode_attn(c.kv, c.x["q"][s].contiguous(), None, 0, c.scale, out, lse,
                                 logits, c.cap, ws)
        sp.sp_h2o_accumulate(c.kv, logits, lse, c.cap, 1, c.scores, c.cap)
        after = c.scores[:, :, :c.budget + 1].double().sum(-1)
        torch.testing.assert_close(after - before, torch.full_like(after, c.G), rtol=0, atol=1e-3)
        c.evict()
        torch.cuda.synchronize()
        assert bool((c.kv.seq_lens == c.budget).all())
        for b in range(c.B):
            for h in range(c.Hkv):
                pos = c.slot_pos[b, h, :c.budget].cpu()
                assert bool((pos[1:] > pos[:-1]).all())
                assert pos[-c.window:].tolist() == list(range(i - c.window + 1, i + 1))
                kk, _ = sp.read_slots(c.kv, b, h, c.budget)
                for j in (0, c.budget // 2, c.budget - 1):
                    assert torch.equal(kk[j], keys_by_pos[(b, h, int(pos[j]))])


def test_list_path_budget_above_capacity_keeps_everything():
    """A budget above the slot capacity (list path) evicts nothing: lengths,
    positions, scores and payloads are unchanged (the kernels size the list
    areas by the capacity, as the workspace does)."""
    c = H2OCase(B=2, Hq=8, D=128, P=16, prompt=8300, budget=100, window=10)
    assert c.cap > 8192
    c.load()
    pos0, sc0 = c.slot_pos.clone(), c.scores.clone()
    k0, v0 = c.kv.k_pool.clone(), c.kv.v_pool.clone()
    big = 3 * c.cap
    ws = sp.workspace(sp.SP_OP_H2O_EVICT, c.kv, big)
    sp.sp_h2o_evict_compact(c.kv, c.scores, c.slot_pos, c.cap, big, 10, ws)
    torch.cuda.synchronize()
    assert bool((c.kv.seq_lens == 8300).all())
    assert torch.equal(c.slot_pos, pos0) and torch.equal(c.scores, sc0)
    assert torch.equal(c.kv.k_pool, k0) and torch.equal(c.kv.v_pool, v0)


def test_evict_noop_when_within_budget_and_ties_keep_lower_slots():
    c = H2OCase(prompt=50, budget=64, window=4)
    c.load()
    c.evict()
    torch.cuda.synchronize()
    assert bool((c.kv.seq_lens == 50).all())
    assert c.slot_pos[0, 0, :50].tolist() == list(range(50))
    # equal scores everywhere: the lowest candidates survive
    c.scores[:, :, :50] = 1.0
    c.evict(20, 4)
    torch.cuda.synchronize()
    assert c.slot_pos[1, 1, :20].tolist() == list(range(16)) + [46, 47, 48, 49]
    assert bool((c.kv.seq_lens == 20).all())


def test_accumulate_reset_counts():
    """n_new = 0 keeps every old score; n_new = 3 resets the last three first."""
    c = H2OCase(prompt=40, budget=64, window=4)
    c.load()
    out = torch.empty(c.B, c.Hq, c.D, device="cuda")
    lse = torch.empty(c.B, c.Hq, device="cuda")
    logits = torch.empty(c.B, c.Hq, c.cap, device="cuda")
    ws = sp.workspace(sp.SP_OP_DECODE_ATTN, c.kv, 0)
    sp.sp_sparse_decode_attn(c.kv, c.x["q"][0].contiguous(), None, 0, c.scale, out, lse, logits,
                             c.cap, ws)
    base = c.scores.clone()
    probs = torch.exp(logits[:, :, :40] - lse[:, :, None]).reshape(c.B, c.Hkv, c.G, 40).sum(2)
    sp.sp_h2o_accumulate(c.kv, logits, lse, c.cap, 0, c.scores, c.cap)
    torch.cuda.synchronize()
    torch.testing.assert_close(c.scores[:, :, :40], base[:, :, :40] + probs, rtol=1e-6, atol=1e-6)
    c.scores.copy_(base)
    sp.sp_h2o_accumulate(c.kv, logits, lse, c.cap, 3, c.scores, c.cap)
    torch.cuda.synchronize()
    torch.testing.assert_close(c.scores[:, :, 37:40], probs[:, :, 37:], rtol=1e-6, atol=1e-6)
    torch.testing.assert_close(c.scores[:, :, :37], base[:, :, :37] + probs[:, :, :37],
                               rtol=1e-6, atol=1e-6)


def test_evict_length_update_in_kernel_matches_separate_launch():
    """With the optional workspace the last KV head of each evicted sequence
    sets its length inside the eviction kernel; without it a second launch
    does.  Pools, scores, positions and lengths agree bit for bit, on a call
    where one sequence is within the budget and on a second call (the
    counters are left zero)."""
    fused = H2OCase(prompt=300, budget=64, window=8, seed=11)
    plain = H2OCase(prompt=300, budget=64, window=8, seed=11)
    for c in (fused, plain):
        c.load()
        c.kv.seq_lens[1] = 60                       # within the budget: untouched
    for budget, window, lens in ((64, 8, [64, 60]), (40, 4, [40, 40])):
        sp.sp_h2o_evict_compact(fused.kv, fused.scores, fused.slot_pos, fused.cap, budget, window, fused.ws)
        sp.sp_h2o_evict_compact(plain.kv, plain.scores, plain.slot_pos, plain.cap, budget, window)
        torch.cuda.synchronize()
        assert fused.kv.seq_lens.tolist() == lens
        assert torch.equal(fused.kv.seq_lens, plain.kv.seq_lens)
        assert torch.equal(fused.kv.k_pool, plain.kv.k_pool)
        assert torch.equal(fused.kv.v_pool, plain.kv.v_pool)
        assert torch.equal(fused.scores, plain.scores)
        assert torch.equal(fused.slot_pos, plain.slot_pos)
        assert int(fused.ws[:8].view(torch.int32).abs().sum()) == 0   # counters left zero
