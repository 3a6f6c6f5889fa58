"""Parity at the workloads' full sizes, in the launch configuration the benchmark uses.

The GPU runs every sequence; the oracle recomputes a sample of sequences (its cost is the limit), and properties
that hold at any size are checked on all of them: score rows sum to the number of query rows, the retained sets
match the oracle's modulo near-ties, the compacted cache is the gather of the original by the GPU's own retained
indices, and the free list conserves blocks.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_se_amd as se
import workloads as W
from gpu_util import (DEV, assert_scores_close, assert_sets_match_modulo_ties, assert_token2chunk_of, i32, lists_from,
                      resident_rows, run_h2o_teacher_forced, status_word, storage_tensor, to_device)
from oracle import pipelines as P
from sparse_decode_attention_se_amd import workflows as WF

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def banner(name):
    print(f"\n[case] {name}", flush=True)


def subcache(c: W.CacheState, seqs, spare=2):
    """The sequences `seqs` of a cache as a cache of their own (blocks renumbered in order; `spare` free blocks per
    sequence)."""
    seqs = list(seqs)
    nbs = [int(np.count_nonzero(c.block_table[b] >= 0)) for b in seqs]
    total = sum(nbs)
    out = W.empty_cache(len(seqs), c.n_kv, c.d, c.page, c.max_blocks, total + len(seqs) * spare, c.dtype,
                        slot_cap=c.slot_stack.shape[2], with_meta=c.page_meta is not None,
                        with_cum=c.cum_score is not None)
    nxt = 0
    for i, b in enumerate(seqs):
        for lb in range(nbs[i]):
            out.k_pool[nxt] = c.k_pool[c.block_table[b, lb]]
            out.v_pool[nxt] = c.v_pool[c.block_table[b, lb]]
            out.block_table[i, lb] = nxt
            nxt += 1
        for f in ("pos_map", "ctx_len", "n_slots", "slot_stack", "slot_top"):
            getattr(out, f)[i] = getattr(c, f)[b]
        if c.cum_score is not None:
            out.cum_score[i] = c.cum_score[b]
    spare = np.arange(out.num_blocks - 1, nxt - 1, -1, dtype=np.int32)
    out.free_blocks[:spare.size] = spare
    out.free_top[0] = spare.size
    return out


def test_snapkv_llama8b_full_size():
    banner("SnapKV Llama-8B shape, 8 x 32768 (oracle on sequences 0 and 7)")
    cfg = W.C1
    inp = W.gen_snapkv(cfg, seed=0, threads=16)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    ev = WF.SnapKVEvent(dc, wq=cfg.wq, protect=cfg.protect, keep=cfg.keep, scale=inp["scale"], status=status)
    ev.score(storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]))
    scores = ev.scores.cpu().numpy()
    ev.select()
    keep = lists_from(ev.idx, ev.count)
    ev.compact()
    ev.decode(storage_tensor(inp["q_dec"], "bf16"))
    out = ev.out.cpu().numpy()
    assert se.se_status_read(status) == 0
    r = cfg.hq // cfg.hkv
    np.testing.assert_allclose(scores[:, :, :cfg.N].sum(axis=2), r * cfg.wq, rtol=1e-4)
    dev = dc.to_numpy()
    # every unit: the compacted cache is the gather of the original by the GPU's retained indices
    orig = inp["cache"]
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            idx = keep[b][g]
            assert len(idx) == cfg.keep + cfg.protect and np.all(np.diff(idx) > 0)
            assert idx[-cfg.protect:].tolist() == list(range(cfg.N - cfg.protect, cfg.N))
            new = resident_rows(dev, cfg.page, "k_pool", b, g, len(idx))
            old = resident_rows({"k_pool": orig.k_pool, "block_table": orig.block_table}, cfg.page, "k_pool", b, g,
                                cfg.N)[idx]
            np.testing.assert_array_equal(new, old)
            np.testing.assert_array_equal(dev["pos_map"][b, g, :len(idx)], idx)
    used = dev["block_table"][dev["block_table"] >= 0].tolist()
    free = dev["free_blocks"][:dev["free_top"][0]].tolist()
    assert sorted(used + free) == list(range(orig.num_blocks))
    # sampled sequences against the oracle
    for b in (0, 7):
        sub = dict(inp, cfg=W.scaled(cfg, B=1), cache=subcache(orig, [b]), q_win=inp["q_win"][b:b + 1],
                   q_pos=inp["q_pos"][b:b + 1], q_dec=inp["q_dec"][b:b + 1])
        ref = P.snapkv_event(sub)
        assert_scores_close(scores[b:b + 1, :, :cfg.N], ref["scores"][:, :, :cfg.N], mass=np.full((1, cfg.hkv),
                                                                                                   r * cfg.wq))
        swapped = 0
        for g in range(cfg.hkv):
            swapped += assert_sets_match_modulo_ties(keep[b][g], ref["keep"][0][g], ref["scores"][0, g],
                                                     floor=1e-6 * r * cfg.wq)
        want = ref["out"]
        if swapped:  # near-tie swaps: the oracle decodes over the device's equally valid choice
            want, _ = oracle.decode_attn(oracle.compact_gather(sub["cache"], [keep[b]]), sub["q_dec"], inp["scale"])
        np.testing.assert_allclose(out[b], want[0], atol=2e-3, rtol=0)


def test_quest_128k_full_size():
    banner("Quest, 2 x 131072")
    cfg = W.C3
    inp = W.gen_quest(cfg, seed=0, threads=16)
    ref = P.quest_step(inp)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    qs = WF.QuestStep(dc, top_pages=cfg.top_pages, scale=inp["scale"], status=status)
    qs.build()
    out = qs.run(storage_tensor(inp["q_dec"], "bf16")).cpu().numpy()
    assert se.se_status_read(status) == 0
    meta = dc.page_meta.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(meta, ref["meta"])
    ps = qs.page_scores.cpu().numpy()
    np.testing.assert_allclose(ps, ref["page_scores"], rtol=1e-3, atol=0)
    got = lists_from(qs.pages, qs.count)
    swapped = 0
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            assert len(got[b][g]) == cfg.top_pages + 2 and got[b][g][0] == 0 and got[b][g][-1] == cfg.N // 16 - 1
            swapped += assert_sets_match_modulo_ties(got[b][g], ref["pages"][b][g], ref["page_scores"][b, g])
    want = ref["out"]
    if swapped:  # near-tie swaps: the oracle decodes over the device's equally valid page choice
        want, _ = oracle.decode_attn(ref["cache"], inp["q_dec"], inp["scale"], pages=got)
    np.testing.assert_allclose(out, want, atol=2e-3, rtol=0)


def test_h2o_full_size_teacher_forced():
    """H2O at its full shape (64 sequences from 8192 tokens, budget 8192, recent 256) for 128 steps on the device;
    the oracle follows sequences 0 and 63 step by step on every head: outputs, evictions (teacher-forced at near
    ties), maps, slot stacks and cumulative scores."""
    banner("H2O, 64 x 8192, 128 steps (oracle on sequences 0 and 63, every head, every step)")
    cfg = W.scaled(W.C4, steps=128)
    inp = W.gen_h2o(cfg, seed=0, threads=16)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    seqs = (0, cfg.B - 1)
    st, swaps = run_h2o_teacher_forced(inp, dc, subcache(inp["cache"], seqs), cfg.steps, seqs=seqs, status=status,
                                       check_every=16)
    assert se.se_status_read(status) == 0
    ctx = dc.ctx_len.cpu().numpy()
    n_slots = dc.n_slots.cpu().numpy()
    # one token in, one out every step once over budget: the context stays at the budget, the slots at budget + 1
    assert np.all(ctx == cfg.budget) and np.all(n_slots == cfg.N + 1)
    print(f"near-tie evictions adopted from the device: {swaps}", flush=True)


def test_kara_full_size_event():
    banner("Kara, 128 x 16384: one event + 4 decode steps (oracle on sequences 0 and 127)")
    cfg = W.scaled(W.C2, period=4)
    inp = W.gen_kara(cfg, seed=0, threads=16)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    ev = WF.KaraEvent(dc, window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                      max_gap=cfg.max_gap, scale=inp["scale"], status=status)
    q_win = P.kara_window_queries(inp, inp["cache"])
    ev.run(storage_tensor(q_win, "bf16"))
    scores = ev.scores.cpu().numpy()
    cand = lists_from(ev.cand, ev.cand_count)
    keep = lists_from(ev.keep, ev.keep_count)
    step = WF.DecodeStep(dc, scale=inp["scale"], status=status)
    outs = []
    for s in range(cfg.period):
        pos = np.full((cfg.B,), cfg.N + s, np.int32)
        q = np.ascontiguousarray(inp["q_all"][:, :, cfg.N + s - inp["q_first_pos"]])
        outs.append(step.run(storage_tensor(inp["k_new"][s], "bf16"), storage_tensor(inp["v_new"][s], "bf16"), i32(pos),
                             storage_tensor(q, "bf16")).cpu().numpy())
    assert se.se_status_read(status) == 0
    r = cfg.hq // cfg.hkv
    np.testing.assert_allclose(scores.sum(axis=2), r * cfg.window, rtol=1e-4)
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            assert cfg.n_cand + cfg.protect <= len(keep[b][g]) <= cfg.budget + cfg.protect
    for b in (0, cfg.B - 1):
        sub = dict(inp, cfg=W.scaled(cfg, B=1), cache=subcache(inp["cache"], [b]), q_all=inp["q_all"][b:b + 1],
                   k_new=inp["k_new"][:, b:b + 1], v_new=inp["v_new"][:, b:b + 1])
        ref = P.kara_event(sub, sub["cache"])
        assert_scores_close(scores[b:b + 1], ref["scores"], mass=np.full((1, cfg.hkv), r * cfg.window))
        for g in range(cfg.hkv):
            assert_sets_match_modulo_ties(cand[b][g], ref["cand"][0][g], ref["scores"][0, g],
                                          base=cfg.N - cfg.window, floor=1e-6 * r * cfg.window)
        assert_token2chunk_of([keep[b]], [cand[b]], scores[b:b + 1], sub["cache"], max_gap=cfg.max_gap,
                              budget=cfg.budget, window=cfg.window, protect=cfg.protect)
        if any(keep[b][g].tolist() != ref["keep"][0][g].tolist() for g in range(cfg.hkv)):
            ref = P.kara_event(sub, sub["cache"], keep=[keep[b]])  # a near-tie swap: the device's choice
        st = ref["cache"]
        for s in range(cfg.period):
            st, o_ref = P.kara_decode_step(sub, st, s)
            np.testing.assert_allclose(outs[s][b], o_ref[0], atol=2e-3, rtol=0)


@pytest.mark.parametrize("policy,seqs", [("threshold", (127, 64)), ("periodic", (0,))])
def test_policy_loop_full_size(policy, seqs):
    banner(f"compression policy loop ({policy}), 128 x 16384, one period of 128 steps (oracle on sequences {seqs})")
    cfg = W.C8
    inp = W.gen_kara(cfg, seed=0, threads=16)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    kw = dict(window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget, max_gap=cfg.max_gap,
              scale=inp["scale"])
    loop = WF.CompressionLoop(dc, policy=policy, period=cfg.period, status=status, **kw)
    q0 = inp["q_first_pos"]
    check = set(range(0, cfg.steps, 8)) | {cfg.steps - 1}
    fired, outs = {}, {}
    for t in range(cfg.steps):
        pos = np.full((cfg.B,), cfg.N + t, np.int32)
        q = np.ascontiguousarray(inp["q_all"][:, :, cfg.N + t - q0])
        o, runs = loop.step(t, storage_tensor(inp["k_new"][t], "bf16"), storage_tensor(inp["v_new"][t], "bf16"),
                            i32(pos), storage_tensor(q, "bf16"),
                            lambda b0, b1: storage_tensor(P.kara_recent_window_queries(inp, b0, b1, t), "bf16"))
        for b0, b1 in runs:
            for b in seqs:
                if b0 <= b < b1:
                    fired[b] = t
        if t in check:
            outs[t] = o[list(seqs)].cpu().numpy()
    assert se.se_status_read(status) == 0
    dev = dc.to_numpy()
    cand = lists_from(loop.cand, loop.cand_count)
    keep = lists_from(loop.keep, loop.keep_count)
    scores = loop.scores.cpu().numpy()
    r = cfg.hq // cfg.hkv
    for i, b in enumerate(seqs):
        # each sampled sequence is compressed once, when the schedule says
        assert fired[b] == [t for t in range(cfg.steps) if b in P.policy_due(policy, t, cfg.B, cfg.period)][0]
        sub = dict(inp, cfg=W.scaled(cfg, B=1), q_all=inp["q_all"][b:b + 1], k_new=inp["k_new"][:, b:b + 1],
                   v_new=inp["v_new"][:, b:b + 1])
        st = subcache(inp["cache"], [b], spare=16)
        for t in range(cfg.steps):
            st, _ = oracle.cache_append(st, sub["k_new"][t], sub["v_new"][t], np.full((1,), cfg.N + t, np.int32))
            if t in check:
                o_ref, _ = oracle.decode_attn(st, np.ascontiguousarray(sub["q_all"][:, :, cfg.N + t - q0]), inp["scale"])
                np.testing.assert_allclose(outs[t][i], o_ref[0], atol=2e-3, rtol=0)
            if t == fired[b]:
                qw = P.kara_recent_window_queries(sub, 0, 1, t)
                ref = P.kara_event_range(st, qw, 0, 1, **kw)
                assert_scores_close(scores[b:b + 1], ref["scores"], mass=np.full((1, cfg.hkv), r * cfg.window))
                for g in range(cfg.hkv):
                    assert_sets_match_modulo_ties(cand[b][g], ref["cand"][0][g], ref["scores"][0, g],
                                                  base=int(st.n_slots[0, g]) - cfg.window, floor=1e-6 * r * cfg.window)
                assert_token2chunk_of([keep[b]], [cand[b]], scores[b:b + 1], st, max_gap=cfg.max_gap,
                                      budget=cfg.budget, window=cfg.window, protect=cfg.protect)
                if any(keep[b][g].tolist() != ref["keep"][0][g].tolist() for g in range(cfg.hkv)):
                    # a near-tie swap: continue the oracle from the device's equally valid choice
                    ref = P.kara_event_range(st, qw, 0, 1, keep=[keep[b]], **kw)
                st = ref["cache"]
        ora = {"k_pool": st.k_pool, "v_pool": st.v_pool, "block_table": st.block_table}
        for g in range(cfg.hkv):
            n = int(st.n_slots[0, g])
            assert int(dev["n_slots"][b, g]) == n and int(dev["ctx_len"][b, g]) == int(st.ctx_len[0, g])
            np.testing.assert_array_equal(dev["pos_map"][b, g, :n], st.pos_map[0, g, :n])
            for which in ("k_pool", "v_pool"):
                np.testing.assert_array_equal(resident_rows(dev, cfg.page, which, b, g, n),
                                              resident_rows(ora, cfg.page, which, 0, g, n))


def test_window_scores_repeat_bitwise_at_full_size():
    """Every kernel of the path is deterministic, so repeated runs must agree bit for bit; a missing wait or barrier
    shows up here as a difference between runs (the full-size shapes exercise every chunk-end case)."""
    banner("window scores repeated 4x: Llama-8B SnapKV 8 x 32768 and Kara 128 x 16384")
    cfg = W.C1
    inp = W.gen_snapkv(cfg, seed=1, threads=16)
    dc = to_device(inp["cache"], cfg.hq)
    ev = WF.SnapKVEvent(dc, wq=cfg.wq, protect=cfg.protect, keep=cfg.keep, scale=inp["scale"])
    q_win, q_pos = storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"])
    runs = []
    for _ in range(4):
        ev.score(q_win, q_pos)
        runs.append(ev.scores.clone())
    for r in runs[1:]:
        assert torch.equal(r, runs[0])
    del dc, ev, runs
    cfg = W.scaled(W.C2, period=1, events=1)
    inp = W.gen_kara(cfg, seed=1, threads=16)
    dc = to_device(inp["cache"], cfg.hq)
    ke = WF.KaraEvent(dc, window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                      max_gap=cfg.max_gap, scale=inp["scale"])
    qk = storage_tensor(np.ascontiguousarray(inp["q_all"][:, :, :cfg.window]), "bf16")
    runs = []
    for _ in range(4):
        se.se_window_score(dc, qk, None, ke.scores, scale=ke.scale, mode=se.SE_SCORE_BIDIR, n_query=cfg.window,
                           window=cfg.window, protect=cfg.protect)
        runs.append(ke.scores.clone())
    r = cfg.hq // cfg.hkv
    np.testing.assert_allclose(runs[0].sum(dim=2).cpu().numpy(), r * cfg.window, rtol=1e-4)
    for x in runs[1:]:
        assert torch.equal(x, runs[0])


def _fields(dc):
    """Every tensor of a device cache, cloned."""
    return {f: getattr(dc, f).clone() for f in se.DeviceCache.FIELDS if getattr(dc, f) is not None}


def _assert_same(a: dict, b: dict, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs between two identical runs"


def test_every_call_repeats_bitwise_at_full_size():
    """Each call of the path, run twice on identical state at the workloads' full sizes, gives identical bits:
    window scores, top-K, Token2Chunk, in-place compaction (whole and trailing), append, decode (split and
    accumulating), page bounds (build and score). A missing wait or barrier, or an order-dependent reduction,
    shows up as a difference between the runs."""
    banner("double runs: Llama-8B SnapKV 8 x 32768, Kara 128 x 16384, Quest 2 x 131072, H2O 64 x 8192")
    # SnapKV: scores, top-K, whole-cache compaction, decode over the compacted cache
    cfg = W.C1
    inp = W.gen_snapkv(cfg, seed=2, threads=16)
    q_win, q_pos, q_dec = storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]), storage_tensor(inp["q_dec"], "bf16")
    base = to_device(inp["cache"], cfg.hq)
    runs = []
    for _ in range(2):
        dc = base.clone()
        status = status_word()
        ev = WF.SnapKVEvent(dc, wq=cfg.wq, protect=cfg.protect, keep=cfg.keep, scale=inp["scale"], status=status)
        ev.run(q_win, q_pos, q_dec)
        assert se.se_status_read(status) == 0
        runs.append(dict(_fields(dc), scores=ev.scores.clone(), idx=ev.idx.clone(), count=ev.count.clone(),
                         out=ev.out.clone()))
        del dc, ev
    _assert_same(runs[0], runs[1], "SnapKV event")
    del base, runs, inp
    torch.cuda.empty_cache()
    # Kara: bidirectional scores, candidates, Token2Chunk, trailing compaction, append, decode
    cfg = W.scaled(W.C2, period=1, events=1)
    inp = W.gen_kara(cfg, seed=2, threads=16)
    q_win = storage_tensor(np.ascontiguousarray(inp["q_all"][:, :, :cfg.window]), "bf16")
    k_new, v_new = storage_tensor(inp["k_new"][0], "bf16"), storage_tensor(inp["v_new"][0], "bf16")
    q = storage_tensor(np.ascontiguousarray(inp["q_all"][:, :, cfg.N - inp["q_first_pos"]]), "bf16")
    pos = i32(np.full((cfg.B,), cfg.N, np.int32))
    base = to_device(inp["cache"], cfg.hq)
    del inp
    runs = []
    for _ in range(2):
        dc = base.clone()
        status = status_word()
        ev = WF.KaraEvent(dc, window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                          max_gap=cfg.max_gap, scale=cfg.d ** -0.5, status=status)
        ev.run(q_win)
        step = WF.DecodeStep(dc, scale=cfg.d ** -0.5, status=status)
        step.run(k_new, v_new, pos, q)
        assert se.se_status_read(status) == 0
        runs.append(dict(_fields(dc), scores=ev.scores.clone(), cand=ev.cand.clone(), keep=ev.keep.clone(),
                         keep_count=ev.keep_count.clone(), out=step.out.clone()))
        del dc, ev, step
    _assert_same(runs[0], runs[1], "Kara event and decode step")
    del base, runs
    torch.cuda.empty_cache()
    # Quest: page bounds build and score, page choice, decode over the pages (the cache itself is not changed)
    cfg = W.C3
    inp = W.gen_quest(cfg, seed=2, threads=16)
    q = storage_tensor(inp["q_dec"], "bf16")
    base = to_device(inp["cache"], cfg.hq)
    runs = []
    for _ in range(2):
        dc = base.clone()
        qs = WF.QuestStep(dc, top_pages=cfg.top_pages, scale=inp["scale"])
        qs.build()
        qs.run(q)
        runs.append(dict(meta=dc.page_meta.clone(), ps=qs.page_scores.clone(), pages=qs.pages.clone(),
                         out=qs.out.clone()))
        del dc, qs
    _assert_same(runs[0], runs[1], "Quest step")
    del base, runs, inp
    torch.cuda.empty_cache()
    # H2O: eight steps of append, accumulating decode, bottom-1, slot eviction
    cfg = W.scaled(W.C4, steps=8)
    inp = W.gen_h2o(cfg, seed=2, threads=16)
    base = to_device(inp["cache"], cfg.hq)
    runs = []
    for _ in range(2):
        dc = base.clone()
        status = status_word()
        h2o = WF.H2OStep(dc, scale=inp["scale"], budget=cfg.budget, recent=cfg.recent, status=status)
        outs = []
        for s in range(cfg.steps):
            h2o.run(storage_tensor(inp["k_new"][s], "bf16"), storage_tensor(inp["v_new"][s], "bf16"),
                    i32(np.full((cfg.B,), cfg.N + s, np.int32)), storage_tensor(inp["q_steps"][s], "bf16"))
            outs.append(h2o.out.clone())
        assert se.se_status_read(status) == 0
        runs.append(dict(_fields(dc), out=torch.stack(outs)))
        del dc, h2o
    _assert_same(runs[0], runs[1], "H2O steps")


def test_h2o_graph_of_1024_steps_replays_like_eager_and_the_oracle():
    """The H2O workload's whole loop (64 sequences from 8192 tokens, budget 8192, recent 256, 1024 steps) captured
    as one HIP graph. Each of two replays, on the restored cache with eager work and synchronisations between them,
    gives bit for bit what the eager loop gives: every step's evicted slots, the recorded sequence's outputs, the
    final maps, stacks and cumulative scores. The oracle then follows the replay on that sequence (teacher-forced on
    the replay's recorded evictions) for its first 384 steps: outputs within 2e-3 and every eviction the oracle's
    choice or a near tie of it."""
    banner("H2O graph: 64 x 8192, 1024 steps, two replays against eager; oracle on sequence 37, 384 steps")
    cfg = W.C4
    seq, checked = 37, 384
    inp = W.gen_h2o(cfg, seed=5, threads=16)
    k_new = [storage_tensor(inp["k_new"][s], "bf16") for s in range(cfg.steps)]
    v_new = [storage_tensor(inp["v_new"][s], "bf16") for s in range(cfg.steps)]
    q = [storage_tensor(inp["q_steps"][s], "bf16") for s in range(cfg.steps)]
    pos = [i32(np.full((cfg.B,), cfg.N + s, np.int32)) for s in range(cfg.steps)]
    pristine = to_device(inp["cache"], cfg.hq)
    status = status_word()
    # eager
    eager = pristine.clone()
    h2o = WF.H2OStep(eager, scale=inp["scale"], budget=cfg.budget, recent=cfg.recent, status=status)
    ev_e, cnt_e, out_e = [], [], []
    for s in range(cfg.steps):
        h2o.run(k_new[s], v_new[s], pos[s], q[s])
        ev_e.append(h2o.evict[:, :, 0].clone())
        cnt_e.append(h2o.evict_count.clone())
        out_e.append(h2o.out[seq].clone())
    assert se.se_status_read(status) == 0
    ev_e, cnt_e, out_e = torch.stack(ev_e), torch.stack(cnt_e), torch.stack(out_e)
    final_e = _fields(eager)
    del eager, h2o
    # graph: captured once, replayed twice on the restored cache
    work = pristine.clone()
    graph = WF.H2OGraph(work, k_new, v_new, pos, q, scale=inp["scale"], budget=cfg.budget, recent=cfg.recent,
                        record=[seq], status=status)
    for r in range(2):
        for f, x in _fields(pristine).items():
            getattr(work, f).copy_(x)
        graph.evict.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert se.se_status_read(status) == 0
        assert torch.equal(graph.evict, ev_e) and torch.equal(graph.evict_count, cnt_e), r
        assert torch.equal(graph.out[:, 0], out_e), r
        _assert_same(final_e, _fields(work), f"replay {r}")
    assert bool((cnt_e == 1).all())  # over budget at every step: one eviction per (sequence, head)
    # the oracle along the replay on the sampled sequence
    ev = graph.evict[:, seq].cpu().numpy()
    outs = graph.out[:, 0].cpu().numpy()
    sub = dict(inp, cfg=W.scaled(cfg, B=1), k_new=inp["k_new"][:, seq:seq + 1], v_new=inp["v_new"][:, seq:seq + 1],
               q_steps=inp["q_steps"][:, seq:seq + 1])
    st = subcache(inp["cache"], [seq])
    r_ = cfg.hq // cfg.hkv
    swaps = 0
    for s in range(checked):
        forced = [[np.array([ev[s, g]], np.int32) for g in range(cfg.hkv)]]
        st, info = P.h2o_step(sub, st, s, evict=forced)
        np.testing.assert_allclose(outs[s], info["out"][0], atol=2e-3, rtol=0)
        for g in range(cfg.hkv):
            swaps += assert_sets_match_modulo_ties(forced[0][g], info["evict"][0][g], info["cum"][0, g],
                                                   floor=1e-6 * r_ * (s + 1))
    print(f"near-tie evictions adopted from the replay: {swaps}", flush=True)
