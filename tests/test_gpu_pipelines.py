"""End-to-end parity of the four workflows against the oracle pipelines on the same seeded inputs.

Retained sets must equal the oracle's except for swaps inside the near-tie tolerance (oracle scores within
1e-3 relative). Where a unit's set equals the oracle's, its compacted cache is compared bit for bit and its
decode output within 2e-3; where a permitted swap happened, the compacted cache is checked to be the gather of
the original cache by the GPU's own retained indices (a property that holds at any size) instead.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_se_amd as se
import workloads as W
from gpu_util import (DEV, assert_scores_close, assert_sets_match_modulo_ties, assert_token2chunk_of, compare_cache,
                      i32, lists_from, resident_rows, run_h2o_teacher_forced, status_word, storage_tensor,
                      to_device)
from oracle import pipelines as P
from sparse_decode_attention_se_amd import workflows as WF

pytestmark = pytest.mark.gpu


def banner(name):
    print(f"\n[case] {name}", flush=True)


def check_gather_property(dev_arrays, original: W.CacheState, keep_lists, page, window=0):
    B, G = original.n_slots.shape
    for b in range(B):
        for g in range(G):
            idx = np.asarray(keep_lists[b][g])
            w0 = original.n_slots[b, g] - window if window else 0
            assert dev_arrays["n_slots"][b, g] == w0 + len(idx)
            new = resident_rows(dev_arrays, page, "k_pool", b, g, w0 + len(idx))[w0:]
            old = resident_rows({"k_pool": original.k_pool, "block_table": original.block_table}, page, "k_pool", b, g,
                                int(original.n_slots[b, g]))[idx]
            np.testing.assert_array_equal(new, old)
            np.testing.assert_array_equal(dev_arrays["pos_map"][b, g, w0:w0 + len(idx)], original.pos_map[b, g, idx])


def run_snapkv(cfg, seed):
    inp = W.gen_snapkv(cfg, seed=seed, threads=8)
    ref = P.snapkv_event(inp)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    ev = WF.SnapKVEvent(dc, wq=cfg.wq, protect=cfg.protect, keep=cfg.keep, scale=inp["scale"], status=status)
    ev.score(storage_tensor(inp["q_win"], cfg.dtype), i32(inp["q_pos"]))
    got_scores = ev.scores.cpu().numpy()
    ev.select()
    got_keep = lists_from(ev.idx, ev.count)
    ev.compact()
    ev.decode(storage_tensor(inp["q_dec"], cfg.dtype))
    assert se.se_status_read(status) == 0
    N = cfg.N
    r = cfg.hq // cfg.hkv
    assert_scores_close(got_scores[:, :, :N], ref["scores"][:, :, :N], mass=np.full((cfg.B, cfg.hkv), r * cfg.wq))
    swapped = 0
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            swapped += assert_sets_match_modulo_ties(got_keep[b][g], ref["keep"][b][g], ref["scores"][b, g],
                                                     floor=1e-6 * r * cfg.wq)
    dev = ev.cache.to_numpy()
    check_gather_property(dev, inp["cache"], got_keep, cfg.page)
    st, want = ref["cache"], ref["out"]
    if swapped:  # near-tie swaps: the oracle continues from the device's equally valid choice
        st = oracle.compact_gather(inp["cache"], got_keep)
        want, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"])
    compare_cache(dev, st)
    np.testing.assert_allclose(ev.out.cpu().numpy(), want, atol=2e-3, rtol=0)
    return swapped


def test_pipeline_tiny_snapkv_full_size():
    banner("pipeline tiny fp32 SnapKV (full size)")
    run_snapkv(W.C0, 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_pipeline_snapkv_llama_shape(seed):
    banner(f"pipeline SnapKV Llama-8B shape, 2 seqs x 4096, seed {seed}")
    cfg = W.scaled(W.C1, B=2, N=4096, keep=448)
    run_snapkv(cfg, seed)


def test_pipeline_quest_small():
    banner("pipeline Quest, 2 seqs x 8192")
    cfg = W.scaled(W.C3, N=8192, top_pages=48)
    inp = W.gen_quest(cfg, seed=0, threads=8)
    ref = P.quest_step(inp)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    qs = WF.QuestStep(dc, top_pages=cfg.top_pages, scale=inp["scale"], status=status)
    qs.build()
    q = storage_tensor(inp["q_dec"], "bf16")
    out = qs.run(q).cpu().numpy()
    assert se.se_status_read(status) == 0
    meta = dc.page_meta.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(meta, ref["meta"])
    n_pages = cfg.N // 16
    ps = qs.page_scores.cpu().numpy()
    np.testing.assert_allclose(ps[:, :, :n_pages], ref["page_scores"][:, :, :n_pages], rtol=1e-3, atol=0)
    got = lists_from(qs.pages, qs.count)
    swapped = 0
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            swapped += assert_sets_match_modulo_ties(got[b][g], ref["pages"][b][g], ref["page_scores"][b, g])
    want = ref["out"]
    if swapped:  # near-tie swaps: the oracle decodes over the device's equally valid page choice
        want, _ = oracle.decode_attn(ref["cache"], inp["q_dec"], inp["scale"], pages=got)
    np.testing.assert_allclose(out, want, atol=2e-3, rtol=0)


def test_pipeline_kara_small():
    banner("pipeline Kara, 4 seqs x 2048, one event + 16 decode steps")
    cfg = W.scaled(W.C2, B=4, N=2048, period=16)
    inp = W.gen_kara(cfg, seed=0, threads=8)
    ref = P.kara_event(inp, inp["cache"])
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    ev = WF.KaraEvent(dc, window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                      max_gap=cfg.max_gap, scale=inp["scale"], status=status)
    ev.run(storage_tensor(ref["q_win"], "bf16"))
    assert se.se_status_read(status) == 0
    r = cfg.hq // cfg.hkv
    gpu_scores = ev.scores.cpu().numpy()
    assert_scores_close(gpu_scores, ref["scores"], mass=np.full((cfg.B, cfg.hkv), r * cfg.window))
    cand = lists_from(ev.cand, ev.cand_count)
    keep = lists_from(ev.keep, ev.keep_count)
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            base = cfg.N - cfg.window
            assert_sets_match_modulo_ties(cand[b][g], ref["cand"][b][g], ref["scores"][b, g], base=base,
                                          floor=1e-6 * r * cfg.window)
    # the kept lists are Token2Chunk of the device's own candidates and scores, exactly
    assert_token2chunk_of(keep, cand, gpu_scores, inp["cache"], max_gap=cfg.max_gap, budget=cfg.budget,
                          window=cfg.window, protect=cfg.protect)
    if any(keep[b][g].tolist() != ref["keep"][b][g].tolist() for b in range(cfg.B) for g in range(cfg.hkv)):
        ref = P.kara_event(inp, inp["cache"], keep=keep)  # a near-tie swap: continue from the device's choice
    dev = dc.to_numpy()
    check_gather_property(dev, inp["cache"], keep, cfg.page, window=cfg.window)
    compare_cache(dev, ref["cache"])
    # decode steps after the event: append then attend
    step = WF.DecodeStep(dc, scale=inp["scale"], status=status)
    st = ref["cache"]
    for s in range(cfg.period):
        st, o_ref = P.kara_decode_step(inp, st, s)
        pos = np.full((cfg.B,), cfg.N + s, np.int32)
        q = np.ascontiguousarray(inp["q_all"][:, :, cfg.N + s - inp["q_first_pos"]])
        o = step.run(storage_tensor(inp["k_new"][s], "bf16"), storage_tensor(inp["v_new"][s], "bf16"), i32(pos),
                     storage_tensor(q, "bf16"))
        np.testing.assert_allclose(o.cpu().numpy(), o_ref, atol=2e-3, rtol=0)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), st)


def test_pipeline_h2o_small():
    banner("pipeline H2O, 4 seqs, 48 steps, teacher-forced on every head")
    cfg = W.scaled(W.C4, B=4, N=1024, budget=1024, recent=64, steps=48)
    inp = W.gen_h2o(cfg, seed=0, threads=8)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    st, _ = run_h2o_teacher_forced(inp, dc, inp["cache"], cfg.steps, status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), st, cum_exact=False, cum_mass=np.full((cfg.B, cfg.hkv), 4.0 * cfg.steps))


def test_pipeline_quest_with_append_small():
    """Quest decode steps that first append a token: the refreshed metadata equals a rebuild of the appended cache
    after every step, and page choice and decode follow the oracle."""
    banner("pipeline Quest with appends, 2 seqs x 8192, 3 steps")
    cfg = W.scaled(W.C5, N=8192, top_pages=48, steps=3)
    inp = W.gen_quest(cfg, seed=1, threads=8)
    st = inp["cache"]
    dc = to_device(st, cfg.hq)
    status = status_word()
    qs = WF.QuestStep(dc, top_pages=cfg.top_pages, scale=inp["scale"], status=status)
    qs.build()
    q = storage_tensor(inp["q_dec"], "bf16")
    r = cfg.hq // cfg.hkv
    for s in range(cfg.steps):
        pos = np.full((cfg.B,), cfg.N + s, np.int32)
        st, _ = oracle.cache_append(st, inp["k_new"][s], inp["v_new"][s], pos)
        se.se_cache_append(dc, storage_tensor(inp["k_new"][s], "bf16"), storage_tensor(inp["v_new"][s], "bf16"),
                           i32(pos), status=status)
        qs.refresh_last_page()
        out = qs.run(q).cpu().numpy()
        assert se.se_status_read(status) == 0
        ref = P.quest_step(inp, st)
        meta = dc.page_meta.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(meta, ref["meta"])
        n_pages = -(-(cfg.N + s + 1) // 16)
        ps = qs.page_scores.cpu().numpy()
        np.testing.assert_allclose(ps[:, :, :n_pages], ref["page_scores"][:, :, :n_pages], rtol=1e-3, atol=0)
        got = lists_from(qs.pages, qs.count)
        swapped = 0
        for b in range(cfg.B):
            for g in range(cfg.hkv):
                assert n_pages - 1 in got[b][g]  # the page holding the new token is always read
                swapped += assert_sets_match_modulo_ties(got[b][g], ref["pages"][b][g], ref["page_scores"][b, g])
        want = ref["out"]
        if swapped:  # near-tie swaps: the oracle decodes over the device's equally valid page choice
            want, _ = oracle.decode_attn(ref["cache"], inp["q_dec"], inp["scale"], pages=got)
        np.testing.assert_allclose(out, want, atol=2e-3, rtol=0)


def test_pipeline_prune_range_then_decode():
    """Range pruning at the Llama-8B head shape on 2 x 4096 tokens: the GPU's window scores drive both the GPU and
    the oracle selection (the scores themselves are compared to the oracle's), the pruned cache equals the
    oracle's bit for bit, and a decode step over it matches."""
    banner("pipeline range pruning, 2 seqs x 4096")
    cfg = W.SnapKV("prune", B=2, hq=32, hkv=8, d=128, N=4096, wq=64, protect=0, keep=0, dtype="bf16",
                   spike_frac=0.04, spike_std=3.0)
    inp = W.gen_snapkv(cfg, seed=5, threads=8)
    st = inp["cache"]
    stack = np.full((2, 8, 4096), -1, np.int32)
    stack[:, :, :st.slot_stack.shape[2]] = st.slot_stack
    st.slot_stack = stack
    rs = np.random.default_rng(5)
    refs = (rs.random(st.num_blocks) < 0.2).astype(np.int32)
    lo, hi, keep = 512, 3584, 600
    dc = to_device(st, cfg.hq)
    status = status_word()
    pr = WF.PruneRange(dc, wq=cfg.wq, scale=inp["scale"], status=status)
    pr.score(storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]))
    gpu_scores = pr.scores.cpu().numpy()
    ora_scores = oracle.window_score_causal(st, inp["q_win"], inp["q_pos"], inp["scale"])
    mass = np.full((2, 8), float(cfg.hq // cfg.hkv * cfg.wq))
    for b in range(2):
        assert_scores_close(gpu_scores[b, :, :4096], ora_scores[b, :, :4096], mass[b])
    pr.select(lo, hi, keep, i32(refs))
    pr.evict()
    assert se.se_status_read(status) == 0
    dropped = oracle.topk_largest(gpu_scores, st, keep, prune_range=(lo, hi), block_refs=refs, emit="dropped")
    assert [len(x) for row in lists_from(pr.drop, pr.count) for x in row] == [len(x) for row in dropped for x in row]
    ref = oracle.evict_slots(st, dropped)
    compare_cache(dc.to_numpy(), ref)
    out = torch.empty((2, cfg.hq, 128), dtype=torch.float32, device=DEV)
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], status=status)
    want, _ = oracle.decode_attn(ref, inp["q_dec"], inp["scale"])
    assert se.se_status_read(status) == 0
    np.testing.assert_allclose(out.cpu().numpy(), want, atol=2e-3, rtol=0)


def test_pipeline_h2o_prefill_chunks():
    """H2O's chunked-prefill eviction, 2 seqs x 1536 tokens in chunks of 512 with a budget of 700: each chunk is
    appended, cumulative scores and kept sets follow the oracle chunk by chunk on every head (sets modulo near ties,
    after which the oracle continues from the device's choice), and the context ends at the budget."""
    banner("pipeline H2O prefill, 2 seqs x 1536, 3 chunks, teacher-forced")
    cfg = W.scaled(W.C7, B=2, N=1536, budget=700, recent=64)
    inp = W.gen_h2o_prefill(cfg, seed=3, threads=4)
    st = inp["cache"]
    dc = to_device(st, cfg.hq)
    status = status_word()
    pf = WF.H2OPrefillChunk(dc, chunk=cfg.chunk, budget=cfg.budget, recent=cfg.recent, scale=inp["scale"],
                            status=status)
    r = cfg.hq // cfg.hkv
    for c in range(cfg.N // cfg.chunk):
        lo, hi = c * cfg.chunk, (c + 1) * cfg.chunk
        q_pos = np.broadcast_to(np.arange(lo, hi, dtype=np.int32), (cfg.B, cfg.chunk)).copy()
        if c > 0:  # the first chunk is already in the cache
            pf.append(storage_tensor(np.ascontiguousarray(inp["k_all"][:, :, lo:hi]), "bf16"),
                      storage_tensor(np.ascontiguousarray(inp["v_all"][:, :, lo:hi]), "bf16"),
                      i32(np.full((cfg.B,), lo, np.int32)))
        pf.score(storage_tensor(np.ascontiguousarray(inp["q_all"][:, :, lo:hi]), "bf16"), i32(q_pos))
        cum_dev = dc.cum_score.cpu().numpy()
        pf.select()
        got = lists_from(pf.keep, pf.count)
        pf.compact()
        assert se.se_status_read(status) == 0
        st, info = P.h2o_prefill_chunk(inp, st, c, keep=got)
        mass = float(r * hi)
        for b in range(cfg.B):
            for g in range(cfg.hkv):
                assert_sets_match_modulo_ties(got[b][g], info["keep"][b][g], info["cum"][b, g], floor=1e-6 * mass)
        # the cumulative scores the selection ran on, on every slot of every head (the cache is dense: the budget's
        # survivors, then the chunk)
        n = min(lo, cfg.budget) + cfg.chunk
        for b in range(cfg.B):
            for g in range(cfg.hkv):
                assert_scores_close(cum_dev[b, g, :n][None], info["cum"][b, g, :n][None].astype(np.float64),
                                    mass=np.array([mass]))
        d = dc.to_numpy()
        compare_cache(d, st, cum_exact=False, cum_mass=np.full((cfg.B, cfg.hkv), mass))
    d = dc.to_numpy()
    assert np.all(d["ctx_len"] == cfg.budget) and np.all(d["n_slots"] == cfg.budget)


def test_mixed_cache_operations_stay_bit_exact():
    """A seeded sequence of single and chunk appends, slot evictions and whole-cache compactions, each followed by a
    page-metadata refresh, on the GPU and the oracle in lockstep: maps, stacks, free list, K/V, cumulative scores
    and page metadata match bit for bit after every operation, and an accumulating decode at the end matches."""
    banner("mixed cache operations, 2 seqs, 14 operations")
    cfg = W.H2O("t", B=2, hq=8, hkv=2, d=128, N=150, budget=1000, recent=4, steps=200, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=21, threads=2)
    st = inp["cache"]
    stack = np.full((2, 2, 64), -1, np.int32)
    stack[:, :, :st.slot_stack.shape[2]] = st.slot_stack
    st.slot_stack = stack
    rs = np.random.default_rng(22)
    st.cum_score[:] = rs.random(st.cum_score.shape).astype(np.float32)
    st.page_meta = oracle.page_bounds_build(st)
    dc = to_device(st, 8)
    status = status_word()
    tok, pos_next = 0, 150
    ops = ["append", "chunk", "evict", "compact"] * 3 + ["append", "evict"]
    rs.shuffle(ops)
    for step, op in enumerate(ops):
        if op == "append":
            pos = np.full((2,), pos_next, np.int32)
            st, _ = oracle.cache_append(st, inp["k_new"][tok], inp["v_new"][tok], pos)
            se.se_cache_append(dc, storage_tensor(inp["k_new"][tok], "bf16"),
                               storage_tensor(inp["v_new"][tok], "bf16"), i32(pos), status=status)
            tok, pos_next = tok + 1, pos_next + 1
        elif op == "chunk":
            T = int(rs.integers(1, 40))
            kc = np.ascontiguousarray(inp["k_new"][tok:tok + T].transpose(1, 2, 0, 3))
            vc = np.ascontiguousarray(inp["v_new"][tok:tok + T].transpose(1, 2, 0, 3))
            pos0 = np.full((2,), pos_next, np.int32)
            st = oracle.cache_append_chunk(st, kc, vc, pos0)
            se.se_cache_append_chunk(dc, storage_tensor(kc, "bf16"), storage_tensor(vc, "bf16"), i32(pos0),
                                     status=status)
            tok, pos_next = tok + T, pos_next + T
        elif op == "evict":
            ev = [[np.sort(rs.choice(np.where(st.pos_map[b, g, :st.n_slots[b, g]] >= 0)[0], size=1 + (b + g) % 3,
                                     replace=False)).astype(np.int32) for g in range(2)] for b in range(2)]
            st = oracle.evict_slots(st, ev)
            idx, cnt = W.pack_lists(ev, 3)
            se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_EVICT_SLOTS, status=status)
        else:
            keep = []
            for b in range(2):
                row = []
                for g in range(2):
                    res = np.where(st.pos_map[b, g, :st.n_slots[b, g]] >= 0)[0]
                    row.append(np.sort(rs.choice(res, size=int(0.7 * res.size), replace=False)).astype(np.int32))
                keep.append(row)
            st = oracle.compact_gather(st, keep)
            idx, cnt = W.pack_lists(keep, int(st.pos_map.shape[2]))
            se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, status=status)
        # an append may reuse a freed slot in any page, a compaction rewrites the prefix: refresh every used page
        st.page_meta = oracle.page_bounds_refresh(st, st.page_meta, "from")
        se.se_page_bounds_refresh(dc, se.SE_REFRESH_FROM_PAGE, status=status)
        assert se.se_status_read(status) == 0, (step, op)
        d = dc.to_numpy()
        compare_cache(d, st)
        meta = dc.page_meta.view(torch.int16).cpu().numpy().view(np.uint16)
        for b in range(2):
            for g in range(2):
                n_pages = -(-int(st.n_slots[b, g]) // 16)
                np.testing.assert_array_equal(meta[b, g, :n_pages], st.page_meta[b, g, :n_pages], err_msg=op)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    q = inp["q_steps"][0]
    se.se_sparse_decode_attn(dc, storage_tensor(q, "bf16"), out, scale=inp["scale"], accumulate=True, status=status)
    ref_out, ref_cum = oracle.decode_attn(st, q, inp["scale"], accumulate=True)
    assert se.se_status_read(status) == 0
    np.testing.assert_allclose(out.cpu().numpy(), ref_out, atol=2e-3, rtol=0)
    st.cum_score = ref_cum.astype(np.float32)
    compare_cache(dc.to_numpy(), st, cum_exact=False, cum_mass=np.full((2, 2), 4.0))


def test_chain_cache_resume_suffix_and_lru_reclaim():
    """Two sessions end their prompts with SnapKV's eviction and are parked. A request that extends session A
    resumes in A's slot and appends only its suffix; its decode matches attention over the retained prefix plus the
    suffix. A new request with no matching chain and no free slot reclaims the least recently used chain (B), whose
    blocks return to the free stack, and its prompt goes into that slot. The cache matches the oracle bit for bit
    after every step."""
    banner("chain cache: resume with a suffix, LRU reclaim")
    cfg = W.SnapKV("chain", B=2, hq=8, hkv=2, d=128, N=600, wq=32, protect=16, keep=100, dtype="bf16",
                   spike_frac=0.04)
    inp = W.gen_snapkv(cfg, seed=13, threads=4)
    st = inp["cache"]
    dc = to_device(st, cfg.hq)
    status = status_word()
    ev = WF.SnapKVEvent(dc, wq=cfg.wq, protect=cfg.protect, keep=cfg.keep, scale=inp["scale"], status=status)
    ev.score(storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]))
    ev.select()
    ev.compact()
    st = oracle.compact_gather(st, lists_from(ev.idx, ev.count))  # the GPU's choice, replayed on the oracle
    compare_cache(dc.to_numpy(), st)
    chains = WF.ChainCacheIndex(dc, status=status)
    prompt = {"A": [("A", i) for i in range(600)], "B": [("B", i) for i in range(600)]}
    chains.park("A", 0, prompt["A"])
    chains.park("B", 1, prompt["B"])
    rs = np.random.default_rng(14)

    def chunk(T):
        return W.to_storage(rs.standard_normal((2, 2, T, 128)), "bf16")

    # A's session continues: 48 new tokens, appended to slot 0 alone
    request = prompt["A"] + [("A", 600 + i) for i in range(48)]
    assert chains.acquire(request) == (0, 600, "A")
    ks, vs = chunk(48), chunk(48)
    counts, pos0 = np.array([48, 0], np.int32), np.array([600, 0], np.int32)
    st = oracle.cache_append_chunk(st, ks, vs, pos0, counts=counts)
    se.se_cache_append_chunk(dc, storage_tensor(ks, "bf16"), storage_tensor(vs, "bf16"), i32(pos0),
                             counts=i32(counts), status=status)
    out = torch.empty((2, cfg.hq, 128), dtype=torch.float32, device=DEV)
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], status=status)
    want, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"])
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), st)
    np.testing.assert_allclose(out.cpu().numpy(), want, atol=2e-3, rtol=0)
    chains.park("A", 0, request)
    # an unrelated request: B, least recently used, is reclaimed and slot 1 takes the new prompt
    top0 = int(st.free_top[0])
    assert chains.acquire([("C", i) for i in range(100)]) == (1, 0, None)
    # the reclaim is a gather that keeps nothing, on the victim's sequence alone
    victim = oracle.compact_gather(oracle.sequence_range(st, 1, 2), [[np.zeros(0, np.int32)] * 2])
    st_other = st
    st = oracle.put_sequence_range(st, victim, 1)
    assert st.n_slots[1].tolist() == [0, 0] and int(st.free_top[0]) > top0
    np.testing.assert_array_equal(st.pos_map[0], st_other.pos_map[0])
    compare_cache(dc.to_numpy(), st)
    kc, vc = chunk(100), chunk(100)
    counts, pos0 = np.array([0, 100], np.int32), np.array([0, 0], np.int32)
    st = oracle.cache_append_chunk(st, kc, vc, pos0, counts=counts)
    se.se_cache_append_chunk(dc, storage_tensor(kc, "bf16"), storage_tensor(vc, "bf16"), i32(pos0),
                             counts=i32(counts), status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), st)
    assert chains.acquire(request + [("A", 648)]) == (0, 648, "A")  # A is still parked


@pytest.mark.parametrize("policy", ["periodic", "threshold"])
def test_compression_policy_loop(policy):
    # 12 sequences, period 8: the threshold policy's tails start at 0, 0, 1, 2, 2, 3, 4, 4, 5, 6, 6, 7 tokens, so
    # its events cover one or two consecutive sequences at every step; the periodic policy's cover all twelve
    banner(f"compression policy loop ({policy}), 12 seqs x 700, window 128, period 8, 24 steps")
    cfg = W.scaled(W.C2, B=12, N=700, window=128, protect=16, period=8, events=3)
    inp = W.gen_kara(cfg, seed=5, threads=8)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    kw = dict(window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget, max_gap=cfg.max_gap,
              scale=inp["scale"])
    loop = WF.CompressionLoop(dc, policy=policy, period=cfg.period, status=status, **kw)
    r = cfg.hq // cfg.hkv
    st = inp["cache"]
    n_runs = resynced = 0
    for t in range(cfg.steps):
        st, o_ref = P.kara_decode_step(inp, st, t)
        pos = np.full((cfg.B,), cfg.N + t, np.int32)
        q = np.ascontiguousarray(inp["q_all"][:, :, cfg.N + t - inp["q_first_pos"]])
        o, runs = loop.step(t, storage_tensor(inp["k_new"][t], "bf16"), storage_tensor(inp["v_new"][t], "bf16"),
                            i32(pos), storage_tensor(q, "bf16"),
                            lambda b0, b1: storage_tensor(P.kara_recent_window_queries(inp, b0, b1, t), "bf16"))
        np.testing.assert_allclose(o.cpu().numpy(), o_ref, atol=2e-3, rtol=0)
        assert runs == P.runs_of(P.policy_due(policy, t, cfg.B, cfg.period))
        for b0, b1 in runs:
            qw = P.kara_recent_window_queries(inp, b0, b1, t)
            ref = P.kara_event_range(st, qw, b0, b1, **kw)
            dev_scores = loop.scores[b0:b1].cpu().numpy()
            assert_scores_close(dev_scores, ref["scores"], mass=np.full((b1 - b0, cfg.hkv), r * cfg.window))
            cand = lists_from(loop.cand[b0:b1], loop.cand_count[b0:b1])
            keep = lists_from(loop.keep[b0:b1], loop.keep_count[b0:b1])
            same = True
            for i in range(b1 - b0):
                for g in range(cfg.hkv):
                    base = int(st.n_slots[b0 + i, g]) - cfg.window
                    assert_sets_match_modulo_ties(cand[i][g], ref["cand"][i][g], ref["scores"][i, g], base=base,
                                                  floor=1e-6 * r * cfg.window)
                    same &= keep[i][g].tolist() == ref["keep"][i][g].tolist()
            assert_token2chunk_of(keep, cand, dev_scores, oracle.sequence_range(st, b0, b1), max_gap=cfg.max_gap,
                                  budget=cfg.budget, window=cfg.window, protect=cfg.protect)
            if not same:
                # a near-tie swap among the candidates: continue the oracle from the device's equally valid choice
                ref = P.kara_event_range(st, qw, b0, b1, keep=keep, **kw)
                resynced += 1
            st = ref["cache"]
            n_runs += 1
        assert se.se_status_read(status) == 0
        compare_cache(dc.to_numpy(), st)
    want_runs = sum(len(P.runs_of(P.policy_due(policy, t, cfg.B, cfg.period))) for t in range(cfg.steps))
    assert n_runs == want_runs > 0 and resynced <= 1


def test_events_on_disjoint_sequence_views_share_the_free_stack():
    # two runs compressed one after the other in the same step: each frees blocks onto the one shared stack, and
    # the sequences between and after them are not touched
    banner("Kara events on sequence views [0, 2) and [5, 7) of 8 sequences")
    cfg = W.scaled(W.C2, B=8, N=640, window=128, protect=16, period=8, events=1)
    inp = W.gen_kara(cfg, seed=9, threads=8)
    dc = to_device(inp["cache"], cfg.hq)
    status = status_word()
    kw = dict(window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget, max_gap=cfg.max_gap,
              scale=inp["scale"])
    loop = WF.CompressionLoop(dc, policy="threshold", period=cfg.period, status=status, **kw)
    st = inp["cache"]
    r = cfg.hq // cfg.hkv
    for b0, b1 in ((0, 2), (5, 7)):
        qw = P.kara_recent_window_queries(inp, b0, b1, -1)
        loop.compress(b0, b1, storage_tensor(qw, "bf16"))
        dev_scores = loop.scores[b0:b1].cpu().numpy()
        cand = lists_from(loop.cand[b0:b1], loop.cand_count[b0:b1])
        keep = lists_from(loop.keep[b0:b1], loop.keep_count[b0:b1])
        ref = P.kara_event_range(st, qw, b0, b1, **kw)
        # the device's scores and candidates against the oracle's, and its kept lists exactly Token2Chunk of its
        # own candidates and scores, before its choice is adopted where a near tie allowed another
        assert_scores_close(dev_scores, ref["scores"], mass=np.full((b1 - b0, cfg.hkv), r * cfg.window))
        for i in range(b1 - b0):
            for g in range(cfg.hkv):
                assert_sets_match_modulo_ties(cand[i][g], ref["cand"][i][g], ref["scores"][i, g],
                                              base=int(st.n_slots[b0 + i, g]) - cfg.window,
                                              floor=1e-6 * r * cfg.window)
        assert_token2chunk_of(keep, cand, dev_scores, oracle.sequence_range(st, b0, b1), max_gap=cfg.max_gap,
                              budget=cfg.budget, window=cfg.window, protect=cfg.protect)
        if any(keep[i][g].tolist() != ref["keep"][i][g].tolist() for i in range(b1 - b0) for g in range(cfg.hkv)):
            ref = P.kara_event_range(st, qw, b0, b1, keep=keep, **kw)  # a near-tie swap: the device's choice
        st = ref["cache"]
        assert se.se_status_read(status) == 0
        compare_cache(dc.to_numpy(), st)
    assert int(st.free_top[0]) > int(inp["cache"].free_top[0])
    np.testing.assert_array_equal(st.pos_map[2:5], inp["cache"].pos_map[2:5])
    np.testing.assert_array_equal(st.pos_map[7], inp["cache"].pos_map[7])
