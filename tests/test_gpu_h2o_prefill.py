"""GPU parity of the chunk-wise H2O prefill: sp_h2o_prefill_scores against the
oracle's h2o_prefill_chunk (scores of the retained slots and of the chunk's
own slots, causal inside the chunk), then whole prompts prefilled chunk by
chunk with eviction after every chunk (sp_h2o_evict_compact), teacher-forced
from the oracle's state at every chunk.

Score tolerance: 1e-5 relative plus 1e-6 (the largest error observed over
these cases is 6.8e-7 relative, 5.6e-7 on single chunks; 9.1e-7 at the full
8192-token chunk of the H2O workload).  Retained sets: equal to the oracle's
except candidates within 1e-5 * max(|cutoff|, 1) of the cutoff score; none has
differed.  The BAND lines printed under -s record the observed errors."""
import numpy as np
import pytest
import torch

import kv_cache_selection_sp_amd as sp
import workloads as W
from gpu_util import f64
from oracle import H2OHeadState, h2o_prefill_chunk, h2o_retain

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-5, 1e-6
UNTOUCHED = -5.0


def _gen(seed, B, H, Hq, D, n, n_q):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    G = Hq // H
    dirs = torch.randn(B, H, D, generator=g, device="cuda")
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    keys = torch.randn(B, H, n, D, generator=g, device="cuda")
    hot = torch.rand(B, H, n, generator=g, device="cuda") < 0.05      # a few strongly attended keys
    keys = (keys + 6.0 * hot[..., None] * dirs[:, :, None, :]).to(torch.bfloat16)
    values = torch.randn(B, H, n, D, generator=g, device="cuda").to(torch.bfloat16)
    q = (torch.randn(B, n_q, Hq, D, generator=g, device="cuda")
         + 0.5 * D ** 0.5 * dirs.repeat_interleave(G, dim=1)[:, None]).to(torch.bfloat16)
    return keys, values, q


def _cache(B, Hq, H, D, P, n_max, keys, values, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    max_pages = -(-n_max // P) + 1
    bt, nblk = W.random_block_table(B, max_pages, g, "cuda")
    kv = sp.PagedKV.allocate(B, Hq, H, D, P, max_pages, nblk, torch.bfloat16, bt)
    cap = kv.capacity
    slot_pos = torch.zeros(B, H, cap, dtype=torch.int32, device="cuda")
    sp.sp_build_page_meta(kv, keys.permute(0, 2, 1, 3).contiguous(), values.permute(0, 2, 1, 3).contiguous(),
                          keys.shape[2], None, None, slot_pos, cap)
    return kv, slot_pos


# (retained slots per sequence, chunk length, G, D, P, block-table width):
# rows G * n_q from 5 to 4400, the first chunk of a prompt (nothing retained),
# a single query, and a sequence shorter than the chunk (untouched).  With a
# block table of 2^15 pages (the extra entries -1; 2^20 slots of capacity) the
# column sums of 16 row slabs fill the pass budget, so the 4400 rows go in two
# passes of 4096; with the short table they go in one.
@pytest.mark.parametrize("n_r,n_q,G,D,P,wide", [
    ([0, 0], 300, 4, 128, 16, 0), ([500, 233], 200, 4, 128, 16, 0), ([100, 61], 1100, 4, 64, 32, 0),
    ([100, 61], 1100, 4, 64, 32, 1 << 15),
    ([37, 12], 5, 1, 128, 16, 0), ([64, 3], 1, 8, 128, 16, 0), ([40, -1], 70, 2, 128, 16, 0)])
def test_prefill_chunk_scores_match_oracle(n_r, n_q, G, D, P, wide):
    B, H = 2, 2
    Hq = G * H
    n_max = max(n_r) + n_q
    print(f"prefill chunk: retained {n_r} n_q {n_q} G {G} D {D} P {P} table {wide or 'short'}", flush=True)
    keys, values, q = _gen(7 + n_q, B, H, Hq, D, n_max, n_q)
    kv, _ = _cache(B, Hq, H, D, P, n_max, keys, values, 7 + n_q)
    if wide:
        bt = torch.full((B, wide), -1, dtype=torch.int32, device="cuda")
        bt[:, :kv.max_pages] = kv.block_table
        kv = sp.PagedKV(kv.k_pool, kv.v_pool, bt, kv.seq_lens, Hq)
    cap = kv.capacity
    lens = [r + n_q if r >= 0 else n_q - 1 for r in n_r]
    kv.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    old = torch.rand(B, H, cap, device="cuda") * 3
    scores = old.clone()
    for b in range(B):
        scores[b, :, lens[b]:] = UNTOUCHED
    before = scores.clone()
    scale = W.default_scale(D)
    sp.sp_h2o_prefill_scores(kv, q, n_q, scale, scores, cap, sp.workspace(sp.SP_OP_H2O_PREFILL, kv, n_q))
    torch.cuda.synchronize()
    for b in range(B):
        L = lens[b]
        if L < n_q:
            assert torch.equal(scores[b], before[b])
            continue
        for h in range(H):
            st = H2OHeadState(np.arange(L - n_q), f64(keys[b, h, :L - n_q]), f64(values[b, h, :L - n_q]),
                              f64(before[b, h, :L - n_q]))
            ref = h2o_prefill_chunk(st, f64(q[b, :, h * G:(h + 1) * G]), np.arange(L - n_q, L),
                                    keys[b, h, L - n_q:L].cpu(), values[b, h, L - n_q:L].cpu(), scale)
            got = f64(scores[b, h, :L])
            err = np.abs(got - ref.scores)
            print(f"BAND prefill score max_rel {float((err / np.maximum(np.abs(ref.scores), 1e-30)).max()):.3e} "
                  f"max_abs {float(err.max()):.3e}")
            assert bool((err <= RTOL * np.abs(ref.scores) + ATOL).all()), float(err.max())
            assert bool((scores[b, h, L:] == UNTOUCHED).all())


@pytest.mark.parametrize("n,chunk,budget,window,G,D", [(1500, 512, 400, 32, 4, 128), (2300, 1024, 600, 128, 2, 64)])
def test_chunked_prefill_teacher_forced(n, chunk, budget, window, G, D):
    """Every chunk starts from the oracle's retained state (written into the
    cache through the library's append), then scores + evicts on the GPU; the
    retained positions must match the oracle's under the cutoff rule, the
    scores of the kept slots their oracle values."""
    B, H, P = 2, 2, 16
    Hq = G * H
    keys, values, q_all = _gen(11, B, H, Hq, D, n, n)
    scale = W.default_scale(D)
    states = [[H2OHeadState(np.zeros(0, np.int64), np.zeros((0, D)), np.zeros((0, D)), np.zeros(0))
               for _ in range(H)] for _ in range(B)]
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        n_q = c1 - c0
        n_r = len(states[0][0])
        # cache = oracle's retained entries, then the chunk
        kk = torch.stack([torch.stack([torch.cat([torch.as_tensor(states[b][h].keys),
                                                  keys[b, h, c0:c1].cpu().double()])
                                       for h in range(H)]) for b in range(B)]).to("cuda", torch.bfloat16)
        vv = torch.stack([torch.stack([torch.cat([torch.as_tensor(states[b][h].values),
                                                  values[b, h, c0:c1].cpu().double()])
                                       for h in range(H)]) for b in range(B)]).to("cuda", torch.bfloat16)
        kv, slot_pos = _cache(B, Hq, H, D, P, max(n_r + n_q, budget + 1), kk, vv, 11)
        cap = kv.capacity
        for b in range(B):
            for h in range(H):
                slot_pos[b, h, :n_r + n_q] = torch.as_tensor(
                    np.concatenate([states[b][h].positions, np.arange(c0, c1)]), dtype=torch.int32)
        scores = torch.zeros(B, H, cap, device="cuda")
        for b in range(B):
            for h in range(H):
                # the GPU keeps fp32 scores: the oracle continues from the same rounded values
                states[b][h].scores = states[b][h].scores.astype(np.float32).astype(np.float64)
                scores[b, h, :n_r] = torch.as_tensor(states[b][h].scores, dtype=torch.float32)
        qc = q_all[:, c0:c1].contiguous()
        sp.sp_h2o_prefill_scores(kv, qc, n_q, scale, scores, cap, sp.workspace(sp.SP_OP_H2O_PREFILL, kv, n_q))
        acc_gpu = scores.clone()
        sp.sp_h2o_evict_compact(kv, scores, slot_pos, cap, budget, window,
                                sp.workspace(sp.SP_OP_H2O_EVICT, kv, budget))
        torch.cuda.synchronize()
        for b in range(B):
            for h in range(H):
                acc = h2o_prefill_chunk(states[b][h], f64(qc[b, :, h * G:(h + 1) * G]), np.arange(c0, c1),
                                        f64(kk[b, h, n_r:]), f64(vv[b, h, n_r:]), scale)
                got_acc = f64(acc_gpu[b, h, :n_r + n_q])
                e_ = np.abs(got_acc - acc.scores)
                print(f"BAND prefill chunk max_rel {float((e_ / np.maximum(np.abs(acc.scores), 1e-30)).max()):.3e}")
                assert bool((np.abs(got_acc - acc.scores) <= RTOL * np.abs(acc.scores) + ATOL).all())
                keep = h2o_retain(acc.positions, acc.scores, budget, window)
                kept = min(len(acc), budget)
                assert int(kv.seq_lens[b]) == kept
                pos = slot_pos[b, h, :kept].cpu().numpy()
                ref_pos = acc.positions[keep]
                diff = set(pos.tolist()) ^ set(ref_pos.tolist())
                if len(acc) > budget:
                    cs = acc.scores[:len(acc) - window] if window else acc.scores
                    cut_ = np.sort(cs)[::-1][budget - window - 1]
                    print(f"BAND prefill retain in_1e-5_band "
                          f"{int(np.sum(np.abs(cs - cut_) <= 1e-5 * max(abs(cut_), 1.0)))} diff {len(diff)}")
                if diff:
                    cand = acc.positions[:len(acc) - window] if window else acc.positions
                    sc = dict(zip(acc.positions.tolist(), acc.scores.tolist()))
                    cut = np.sort([sc[p_] for p_ in cand.tolist()])[::-1][budget - window - 1]
                    assert all(abs(sc[p_] - cut) <= 1e-5 * max(abs(cut), 1.0) for p_ in diff)
                states[b][h] = H2OHeadState(acc.positions[keep], acc.keys[keep], acc.values[keep],
                                            acc.scores[keep])
