"""Oracle against what the pages and the mathematics fix: closed forms, invariants, special cases that reduce to
a library routine, and brute force on tiny inputs. Each test is chosen so that a plausible slip in the oracle
(a dropped term, a wrong mask or index, a transposed operand, a wrong GQA map, a reversed tie-break) fails it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import pipelines as P


def tiny_snapkv(B=1, hq=4, hkv=2, d=8, N=40, wq=6, protect=3, keep=10, dtype="f32", seed=1):
    cfg = W.SnapKV("tiny", B=B, hq=hq, hkv=hkv, d=d, N=N, wq=wq, protect=protect, keep=keep, dtype=dtype,
                   page=4)
    return W.gen_snapkv(cfg, seed=seed, threads=1)


def set_keys(cache, b, g, slots, rows):
    for s, row in zip(slots, rows):
        blk = cache.block_table[b, s // cache.page]
        cache.k_pool[blk, g, s % cache.page] = W.to_storage(np.asarray(row, np.float64), cache.dtype)


# ------------------------------------------------------------------ causal window scores ------------------------
def test_causal_rows_sum_to_one_per_query():
    inp = tiny_snapkv(B=2)
    s = oracle.window_score_causal(inp["cache"], inp["q_win"], inp["q_pos"], inp["scale"])
    r = inp["q_win"].shape[1] // inp["cache"].n_kv
    np.testing.assert_allclose(s.sum(axis=2), r * inp["q_win"].shape[2], rtol=0, atol=1e-12)


def test_causal_zero_queries_closed_form():
    # q = 0 -> each query spreads its mass uniformly over the keys it sees: score_j = r * sum_{t >= pos_j} 1/(t+1)
    inp = tiny_snapkv()
    q = np.zeros_like(inp["q_win"])
    s = oracle.window_score_causal(inp["cache"], q, inp["q_pos"], inp["scale"])
    N, wq, r = 40, 6, 2
    for j in range(N):
        expect = r * sum(1.0 / (t + 1) for t in range(N - wq, N) if t >= j)
        assert abs(s[0, 0, j] - expect) < 1e-12
        assert abs(s[0, 1, j] - expect) < 1e-12


def test_causal_single_query_matches_library_softmax():
    # one query, one head per group: the score row is exactly softmax(scale * K q) over the visible keys
    from scipy.special import softmax

    inp = tiny_snapkv(hq=2, hkv=2, wq=1)
    c = inp["cache"]
    s = oracle.window_score_causal(c, inp["q_win"], inp["q_pos"], inp["scale"])
    K = W.gather_contiguous(c, "k").astype(np.float64)
    for g in range(2):
        z = inp["scale"] * (K[0, g, :40] @ inp["q_win"][0, g, 0].astype(np.float64))
        np.testing.assert_allclose(s[0, g, :40], softmax(z), rtol=1e-13, atol=1e-16)


def test_causal_mask_uses_positions_not_slots():
    # permute the slot order (and pos_map with it): scores follow the tokens
    inp = tiny_snapkv()
    c = inp["cache"]
    base = oracle.window_score_causal(c, inp["q_win"], inp["q_pos"], inp["scale"])
    perm = np.random.default_rng(3).permutation(40)
    c2 = c.copy()
    Kc = W.gather_contiguous(c, "k")
    for g in range(2):
        c2.pos_map[0, g, :40] = perm
        set_keys(c2, 0, g, range(40), Kc[0, g, perm].astype(np.float64))
    s2 = oracle.window_score_causal(c2, inp["q_win"], inp["q_pos"], inp["scale"])
    np.testing.assert_allclose(s2[0, :, :40], base[0, :, perm].T, rtol=1e-12, atol=1e-15)


def test_causal_query_sees_only_earlier_keys():
    # a huge key at the last position is invisible to every query except the last one
    inp = tiny_snapkv(hq=2, hkv=2, wq=2)
    c = inp["cache"]
    q = np.zeros_like(inp["q_win"])
    q[0, :, :, 0] = 1.0
    set_keys(c, 0, 0, [39], [[1000.0] + [0.0] * 7])
    s = oracle.window_score_causal(c, q, inp["q_pos"], inp["scale"])
    # query at position 38 cannot see slot 39: its mass (1) is spread over 0..38; query 39 puts ~1 on slot 39
    assert abs(s[0, 0, 39] - 1.0) < 1e-12
    assert abs(s[0, 0, :39].sum() - 1.0) < 1e-12


def test_causal_gqa_group_map():
    # head h belongs to KV head h // r: only head 3 (group 1 when r = 2) gets a query aligned with key 5
    inp = tiny_snapkv(hq=4, hkv=2, wq=1)
    c = inp["cache"]
    e0 = np.zeros(8)
    e0[0] = 10.0
    set_keys(c, 0, 1, [5], [e0])
    q = np.zeros_like(inp["q_win"])
    q[0, 3, 0, :] = e0
    s = oracle.window_score_causal(c, q, inp["q_pos"], inp["scale"])
    # group 1 = heads 2 (uniform, 1/40 each) and 3 (nearly one-hot on slot 5); group 0 heads are both uniform
    assert s[0, 1, 5] > 1.0 + 1.0 / 40 - 1e-6
    np.testing.assert_allclose(s[0, 0], 2.0 / 40, rtol=0, atol=1e-14)


def test_causal_brute_force_loops():
    inp = tiny_snapkv(B=2, hq=4, hkv=2, d=3, N=9, wq=3, protect=1, keep=2, seed=7)
    c = inp["cache"]
    s = oracle.window_score_causal(c, inp["q_win"], inp["q_pos"], inp["scale"])
    K = W.gather_contiguous(c, "k").astype(np.float64)
    for b in range(2):
        for h in range(4):
            g = h // 2
            for t in range(3):
                qp = int(inp["q_pos"][b, t])
                logits = [sum(float(inp["q_win"][b, h, t, i]) * K[b, g, j, i] for i in range(3)) * inp["scale"]
                          for j in range(qp + 1)]
                mx = max(logits)
                den = sum(math.exp(x - mx) for x in logits)
                for j in range(qp + 1):
                    s[b, g, j] -= math.exp(logits[j] - mx) / den
    assert np.abs(s).max() < 1e-12


# ------------------------------------------------------------------ bidirectional window scores -----------------
def tiny_kara(B=1, N=48, window=16, protect=4, hq=4, hkv=2, d=8, seed=2):
    cfg = W.Kara("tiny", B=B, hq=hq, hkv=hkv, d=d, N=N, window=window, protect=protect, cand_frac=0.25,
                 budget_frac=0.5, max_gap=3, period=2, events=1, rho=0.9, dtype="f32", page=4)
    return W.gen_kara(cfg, seed=seed, threads=1)


def test_bidir_conservation_and_uniform():
    inp = tiny_kara()
    c = inp["cache"]
    qw = P.kara_window_queries(inp, c)
    s = oracle.window_score_bidir(c, qw, inp["scale"], 16, 4)
    np.testing.assert_allclose(s.sum(axis=2), 2 * 16, atol=1e-12)
    s0 = oracle.window_score_bidir(c, np.zeros_like(qw), inp["scale"], 16, 4)
    np.testing.assert_allclose(s0, 2 * 16 / 12, atol=1e-13)


def test_bidir_ignores_keys_outside_region():
    inp = tiny_kara()
    c = inp["cache"]
    qw = P.kara_window_queries(inp, c)
    base = oracle.window_score_bidir(c, qw, inp["scale"], 16, 4)
    c2 = c.copy()
    big = [[100.0] * 8]
    for g in range(2):
        set_keys(c2, 0, g, [47], big)   # protected tail
        set_keys(c2, 0, g, [31], big)   # just before the window
    s2 = oracle.window_score_bidir(c2, qw, inp["scale"], 16, 4)
    np.testing.assert_array_equal(s2, base)
    c3 = c.copy()
    set_keys(c3, 0, 0, [32], big)       # first region slot does matter
    assert not np.allclose(oracle.window_score_bidir(c3, qw, inp["scale"], 16, 4)[0, 0], base[0, 0])


def test_bidir_brute_force_loops():
    inp = tiny_kara(d=3, window=6, protect=2, N=10)
    c = inp["cache"]
    qw = P.kara_window_queries(inp, c)
    s = oracle.window_score_bidir(c, qw, inp["scale"], 6, 2)
    K = W.gather_contiguous(c, "k").astype(np.float64)
    for h in range(4):
        g = h // 2
        for t in range(6):
            logits = [inp["scale"] * sum(float(qw[0, h, t, i]) * K[0, g, 4 + j, i] for i in range(3))
                      for j in range(4)]
            mx = max(logits)
            den = sum(math.exp(x - mx) for x in logits)
            for j in range(4):
                s[0, g, j] -= math.exp(logits[j] - mx) / den
    assert np.abs(s).max() < 1e-12


# ------------------------------------------------------------------ top-K ------------------------------------------
def test_topk_matches_lexsort_and_edge_cases():
    rs = np.random.default_rng(5)
    c = W.empty_cache(2, 3, 2, 16, 8, 16, "f32")
    W.layout_initial(c, 100)
    scores = W.gen_scores(9, (2, 3, 128), levels=7)  # many exact ties
    for k in (0, 1, 13, 97, 200):
        out = oracle.topk_largest(scores, c, k, protect=3)
        for b in range(2):
            for g in range(3):
                region = np.arange(97)
                order = np.lexsort((region, -scores[b, g, :97].astype(np.float64)))
                exp = sorted(order[:min(k, 97)].tolist() + [97, 98, 99])
                assert out[b][g].tolist() == exp
    # k = region size keeps everything; all-equal scores keep the lowest positions
    full = oracle.topk_largest(scores, c, 97, protect=3)
    assert all(x.tolist() == list(range(100)) for row in full for x in row)
    flat = oracle.topk_largest(np.ones_like(scores), c, 10, protect=3)
    assert all(x.tolist() == list(range(10)) + [97, 98, 99] for row in flat for x in row)


def test_topk_window_base():
    c = W.empty_cache(1, 1, 2, 16, 8, 8, "f32")
    W.layout_initial(c, 100)
    scores = np.zeros((1, 1, 20), np.float32)
    scores[0, 0, [3, 7]] = 1.0  # window of 24 starting at slot 76, region 20
    out = oracle.topk_largest(scores, c, 2, window=24, protect=4)
    assert out[0][0].tolist() == [79, 83, 96, 97, 98, 99]


def test_smallest_matches_lexsort():
    c = W.empty_cache(1, 2, 2, 16, 8, 8, "f32")
    W.layout_initial(c, 100)
    c.pos_map[0, 1, 10] = -1
    c.ctx_len[0, 1] = 99
    cum = W.gen_scores(3, (1, 2, 128), levels=5)
    out = oracle.topk_smallest(cum, c, 1, budget=50, recent=20)
    for g in range(2):
        pos = c.pos_map[0, g, :100]
        elig = np.where((pos >= 0) & (pos <= 99 - 20))[0]
        order = np.lexsort((-pos[elig], cum[0, g, elig]))
        assert out[0][g].tolist() == [int(elig[order[0]])]


# ------------------------------------------------------------------ Token2Chunk ------------------------------------
def test_token2chunk_identities_and_invariants():
    inp = tiny_kara(N=80, window=40, protect=4)
    c = inp["cache"]
    rs = np.random.default_rng(11)
    scores = rs.random((1, 2, 36)).astype(np.float32)
    cand = oracle.topk_largest(scores, c, 9, window=40, protect=4)
    m = [len(x) - 4 for x in cand[0]]
    same = oracle.token2chunk(cand, scores, c, max_gap=8, budget=min(m), window=40, protect=4)
    assert all(a.tolist() == b.tolist() for a, b in zip(same[0], cand[0]))
    nogap = oracle.token2chunk(cand, scores, c, max_gap=0, budget=1000, window=40, protect=4)
    assert all(a.tolist() == b.tolist() for a, b in zip(nogap[0], cand[0]))
    full = oracle.token2chunk(cand, scores, c, max_gap=3, budget=1000, window=40, protect=4)
    for g in range(2):
        cs = [s for s in cand[0][g].tolist() if s < 76]
        exp = set(cs)
        for a, b in zip(cs, cs[1:]):
            if 1 <= b - a - 1 <= 3:
                exp.update(range(a + 1, b))
        assert full[0][g].tolist() == sorted(exp) + [76, 77, 78, 79]
    for budget in range(9, 30):
        out = oracle.token2chunk(cand, scores, c, max_gap=4, budget=budget, window=40, protect=4)
        for g in range(2):
            o = out[0][g].tolist()
            assert o == sorted(set(o)) and set(cand[0][g].tolist()) <= set(o)
            assert len(o) - 4 <= max(budget, m[g])
            cs = [s for s in cand[0][g].tolist() if s < 76]
            for a, b in zip(cs, cs[1:]):
                if b - a - 1 > 4:
                    assert not any(a < s < b for s in o)


# ------------------------------------------------------------------ compaction / append ----------------------------
def test_compaction_is_a_gather_and_conserves_blocks():
    inp = tiny_snapkv(B=3, N=37, dtype="bf16")
    c = inp["cache"]
    c = c.copy()
    # more pool than needed so spare blocks exist
    counts = np.array([[5, 9], [0, 37], [13, 1]], np.int32)
    keep = W.gen_keep_sets(4, c.n_slots, counts)
    out = oracle.compact_gather(c, keep)
    K0 = W.gather_contiguous(c, "k")
    V0 = W.gather_contiguous(c, "v")
    K1 = W.gather_contiguous(out, "k")
    V1 = W.gather_contiguous(out, "v")
    for b in range(3):
        for g in range(2):
            n = counts[b, g]
            np.testing.assert_array_equal(K1[b, g, :n], K0[b, g, keep[b][g]])
            np.testing.assert_array_equal(V1[b, g, :n], V0[b, g, keep[b][g]])
            assert out.pos_map[b, g, :n].tolist() == keep[b][g].tolist()
    used = out.block_table[out.block_table >= 0].tolist()
    free = out.free_blocks[:out.free_top[0]].tolist()
    assert sorted(used + free) == list(range(out.num_blocks))
    ident = oracle.compact_gather(c, [[np.arange(37, dtype=np.int32)] * 2] * 3)
    np.testing.assert_array_equal(ident.k_pool, c.k_pool)
    assert ident.free_top[0] == c.free_top[0]


def test_evict_then_append_reuses_slot_and_keeps_counts():
    c = W.empty_cache(1, 1, 2, 4, 4, 4, "f32", with_cum=True)
    W.layout_initial(c, 10)
    c.cum_score[0, 0, :10] = np.arange(10)
    c = oracle.evict_slots(c, [[np.array([4], np.int32)]])
    assert c.cum_score[0, 0, 4] == 0 and c.ctx_len[0, 0] == 9
    c, slots = oracle.cache_append(c, np.ones((1, 1, 2), np.float32), np.ones((1, 1, 2), np.float32),
                                   np.array([10], np.int32))
    assert slots.tolist() == [[4]] and c.pos_map[0, 0, 4] == 10 and c.n_slots[0, 0] == 10


# ------------------------------------------------------------------ range-restricted pruning ----------------------
def _prune_case(seed=3, N=90, busy_frac=0.3):
    inp = tiny_snapkv(B=2, hq=4, hkv=2, d=8, N=N, dtype="f32", seed=seed)
    c = inp["cache"]
    c.slot_stack = np.zeros((2, 2, N), np.int32)  # room for every eviction
    rs = np.random.default_rng(seed)
    c.pos_map[0, 1, [5, 40, 41]] = -1  # a few holes
    refs = (rs.random(c.num_blocks) < busy_frac).astype(np.int32)
    scores = rs.random((2, 2, N)).round(2)  # coarse values: many ties
    return c, refs, scores


def _brute_kept_positions(c, refs, scores, b, g, k, lo, hi):
    """R' = (R minus T) plus I, straight from the definition on one (b, g)."""
    n = int(c.n_slots[b, g])
    res = [s for s in range(n) if c.pos_map[b, g, s] >= 0]
    T = [s for s in res if lo <= c.pos_map[b, g, s] < hi and refs[c.block_table[b, s // c.page]] == 0]
    order = np.lexsort((np.array([c.pos_map[b, g, s] for s in T]), -np.array([scores[b, g, s] for s in T])))
    I = [T[i] for i in order[:k]]
    return sorted(int(c.pos_map[b, g, s]) for s in set(res) - set(T) | set(I))


@pytest.mark.parametrize("k", [0, 7, 1000])
def test_range_pruning_keeps_outside_busy_and_top_k(k):
    c, refs, scores = _prune_case()
    lo, hi = 20, 70
    kept = oracle.topk_largest(scores, c, k, prune_range=(lo, hi), block_refs=refs)
    dropped = oracle.topk_largest(scores, c, k, prune_range=(lo, hi), block_refs=refs, emit="dropped")
    after = oracle.evict_slots(c, dropped)
    for b in range(2):
        for g in range(2):
            n = int(c.n_slots[b, g])
            res = {s for s in range(n) if c.pos_map[b, g, s] >= 0}
            assert set(kept[b][g]) | set(dropped[b][g]) == res and not set(kept[b][g]) & set(dropped[b][g])
            want = _brute_kept_positions(c, refs, scores, b, g, k, lo, hi)
            now = sorted(int(x) for x in after.pos_map[b, g, :n] if x >= 0)
            assert now == want
            assert [int(c.pos_map[b, g, s]) for s in kept[b][g]] == want
            # busy blocks and positions outside the range lose nothing
            for s in res:
                p = c.pos_map[b, g, s]
                if not lo <= p < hi or refs[c.block_table[b, s // c.page]] > 0:
                    assert s in set(kept[b][g])
            if k == 0:
                assert all(lo <= c.pos_map[b, g, s] < hi for s in dropped[b][g])
            if k == 1000:
                assert len(dropped[b][g]) == 0


def test_range_pruning_without_refs_or_with_full_range_is_plain_top_k():
    c, refs, scores = _prune_case(busy_frac=0.0)
    plain = oracle.topk_largest(scores, c, 11)
    ranged = oracle.topk_largest(scores, c, 11, prune_range=(0, 1 << 30), block_refs=np.zeros_like(refs))
    for b in range(2):
        for g in range(2):
            assert plain[b][g].tolist() == ranged[b][g].tolist()


# ------------------------------------------------------------------ H2O chunked prefill -----------------------------
def test_h2o_prefill_chunks_match_brute_force():
    """Three prefill chunks on a tiny cache against a loop written from the rule: every chunk query's softmax over
    the resident keys it may see is added to the keys' cumulative scores, then while ctx > budget the lowest score
    among positions <= newest - recent is evicted (ties to the higher position). Compared by position: the
    resident set and the cumulative scores."""
    cfg = W.H2OPrefill("tiny", B=1, hq=4, hkv=2, d=8, N=24, chunk=8, budget=10, recent=3, dtype="f32", page=4)
    inp = W.gen_h2o_prefill(cfg, seed=4, threads=1)
    st = inp["cache"]
    K = inp["k_all"].astype(np.float64)  # [B][hkv][N][d] by position
    q = inp["q_all"].astype(np.float64)
    cum = np.zeros((2, 24))
    alive = np.ones((2, 24), bool)
    for c in range(3):
        st, info = P.h2o_prefill_chunk(inp, st, c)
        hi = 8 * (c + 1)
        for g in range(2):
            for h in (2 * g, 2 * g + 1):
                for t in range(8 * c, hi):
                    vis = [j for j in range(t + 1) if alive[g, j]]
                    x = np.array([q[0, h, t] @ K[0, g, j] for j in vis]) * inp["scale"]
                    p = np.exp(x - x.max())
                    cum[g, vis] += p / p.sum()
            while alive[g, :hi].sum() > cfg.budget:
                newest = max(j for j in range(hi) if alive[g, j])
                elig = [j for j in range(hi) if alive[g, j] and j <= newest - cfg.recent]
                worst = min(elig, key=lambda j: (np.float32(cum[g, j]), -j))
                alive[g, worst] = False
                cum[g, worst] = 0.0
            n = int(st.n_slots[0, g])
            pos = st.pos_map[0, g, :n]
            assert sorted(pos.tolist()) == [j for j in range(hi) if alive[g, j]], (c, g)
            np.testing.assert_allclose(st.cum_score[0, g, :n], cum[g, pos], rtol=1e-6)
        assert st.ctx_len[0].tolist() == [min(hi, cfg.budget)] * 2


def _h2o_tiny(N, T, seed=6):
    cfg = W.H2O("tiny", B=2, hq=4, hkv=2, d=4, N=N, budget=N + T, recent=2, steps=T, zipf=1.1, dtype="f32", page=4)
    return W.gen_h2o(cfg, seed=seed, threads=1)


@pytest.mark.parametrize("N,T", [(8, 9), (10, 3), (11, 1)])
def test_chunk_append_equals_single_appends_by_position(N, T):
    """A chunk of T tokens gives, position by position, the cache T single-token appends give (no free slots to
    reuse): same K/V per position, maps, counts; the blocks taken are the same set."""
    inp = _h2o_tiny(N, T)
    c = inp["cache"]
    kc = np.ascontiguousarray(inp["k_new"].transpose(1, 2, 0, 3))  # [B][n_kv][T][d]
    vc = np.ascontiguousarray(inp["v_new"].transpose(1, 2, 0, 3))
    one = c
    for t in range(T):
        one, _ = oracle.cache_append(one, inp["k_new"][t], inp["v_new"][t], np.full((2,), N + t, np.int32))
    chunk = oracle.cache_append_chunk(c, kc, vc, np.full((2,), N, np.int32))
    for f in ("n_slots", "ctx_len", "pos_map", "free_top"):
        np.testing.assert_array_equal(getattr(chunk, f), getattr(one, f))
    np.testing.assert_array_equal(W.gather_contiguous(chunk, "k"), W.gather_contiguous(one, "k"))
    np.testing.assert_array_equal(W.gather_contiguous(chunk, "v"), W.gather_contiguous(one, "v"))
    used = lambda x: sorted(int(v) for v in x.block_table.ravel() if v >= 0)
    assert used(chunk) == used(one)
    top = int(chunk.free_top[0])
    assert sorted(used(chunk) + [int(x) for x in chunk.free_blocks[:top]]) == list(range(c.num_blocks))


def test_chunk_append_with_counts_equals_per_sequence_appends():
    """Counts per sequence (one of them 0) give each sequence what a chunk of its own count would."""
    inp = _h2o_tiny(10, 7)
    c = inp["cache"]
    kc = np.ascontiguousarray(inp["k_new"].transpose(1, 2, 0, 3))
    vc = np.ascontiguousarray(inp["v_new"].transpose(1, 2, 0, 3))
    both = oracle.cache_append_chunk(c, kc, vc, np.full((2,), 10, np.int32), counts=np.array([5, 0]))
    assert both.n_slots.tolist() == [[15, 15], [10, 10]]
    alone = oracle.cache_append_chunk(c, kc[:, :, :5], vc[:, :, :5], np.full((2,), 10, np.int32),
                                      counts=np.array([5, 0]))
    np.testing.assert_array_equal(W.gather_contiguous(both, "k"), W.gather_contiguous(alone, "k"))
    full5 = oracle.cache_append_chunk(c, kc[:, :, :5], vc[:, :, :5], np.full((2,), 10, np.int32))
    np.testing.assert_array_equal(W.gather_contiguous(both, "k")[0], W.gather_contiguous(full5, "k")[0])
    np.testing.assert_array_equal(both.pos_map[1], c.pos_map[1])


def test_chunk_append_pops_in_sequence_then_block_order_and_is_all_or_nothing():
    inp = _h2o_tiny(8, 9)  # each sequence needs logical blocks 2, 3 and 4
    c = inp["cache"]
    kc = np.ascontiguousarray(inp["k_new"].transpose(1, 2, 0, 3))
    vc = np.ascontiguousarray(inp["v_new"].transpose(1, 2, 0, 3))
    top = int(c.free_top[0])
    out = oracle.cache_append_chunk(c, kc, vc, np.full((2,), 8, np.int32))
    popped = [int(c.free_blocks[top - 1 - i]) for i in range(6)]
    assert [int(out.block_table[b, lb]) for b in range(2) for lb in (2, 3, 4)] == popped
    short = c.copy()
    short.free_top[0] = 5  # one block short
    with pytest.raises(oracle.cache_ops.CapacityError):
        oracle.cache_append_chunk(short, kc, vc, np.full((2,), 8, np.int32))
    np.testing.assert_array_equal(short.n_slots, c.n_slots)


# ------------------------------------------------------------------ page bounds -----------------------------------
def test_page_bound_is_an_upper_bound_and_tight_for_equal_keys():
    cfg = W.Quest("tiny", B=2, hq=4, hkv=2, d=16, N=100, top_pages=2, shift_frac=0.1, shift=2.0)
    inp = W.gen_quest(cfg, seed=3, threads=1)
    c = inp["cache"]
    meta = oracle.page_bounds_build(c)
    u = oracle.page_bounds_score(c, meta, inp["q_dec"])
    K = W.gather_contiguous(c, "k")
    Kf = W.bf16_bits_to_f32(K).astype(np.float64)
    q = W.bf16_bits_to_f32(inp["q_dec"]).astype(np.float64)
    for b in range(2):
        for g in range(2):
            for p in range(7):
                rows = Kf[b, g, p * 16:min(p * 16 + 16, 100)]
                best = max((rows @ q[b, h]).max() for h in (2 * g, 2 * g + 1))
                assert u[b, g, p] >= best - 1e-9
    # a page whose keys are all equal: bound equals the exact maximum
    c2 = c.copy()
    for s in range(16, 32):
        set_keys(c2, 0, 0, [s], [Kf[0, 0, 16]])
    meta2 = oracle.page_bounds_build(c2)
    u2 = oracle.page_bounds_score(c2, meta2, inp["q_dec"])
    exact = max(Kf[0, 0, 16] @ q[0, h] for h in (0, 1))
    assert abs(u2[0, 0, 1] - exact) < 1e-9


@pytest.mark.parametrize("N", [32, 37])
def test_refresh_last_page_after_append_equals_rebuild(N):
    # N = 32: the append opens a new page (a spare block is popped); N = 37: it lands in the partly filled last page
    cfg = W.H2O("tiny", B=2, hq=4, hkv=2, d=8, N=N, budget=N, recent=4, steps=2, zipf=1.1, dtype="f32")
    inp = W.gen_h2o(cfg, seed=2, threads=1)
    c0 = inp["cache"]
    meta0 = oracle.page_bounds_build(c0)
    c1, slots = oracle.cache_append(c0, inp["k_new"][0], inp["v_new"][0], np.full((2,), N, np.int32))
    assert (slots == N).all()
    got = oracle.page_bounds_refresh(c1, meta0, "last")
    want = oracle.page_bounds_build(c1)
    np.testing.assert_array_equal(got, want)
    assert not np.array_equal(meta0, want)  # the append did change the metadata
    # an empty range changes nothing
    n_pages = -(-(N + 1) // 16)
    same = oracle.page_bounds_refresh(c1, meta0, "from", page_lo=np.full((2, 2), n_pages))
    np.testing.assert_array_equal(same, meta0)


@pytest.mark.parametrize("window", [0, 27])
def test_refresh_from_page_after_compaction_equals_rebuild(window):
    # window 27 of 61 slots (page 4): w0 = 34 is not page-aligned, so page 8 holds both untouched and moved slots
    inp = tiny_snapkv(B=2, hq=4, hkv=2, d=8, N=61, dtype="f32")
    c = inp["cache"]
    page = c.page
    meta = oracle.page_bounds_build(c)
    rs = np.random.default_rng(4)
    w0 = 61 - window if window else 0
    keep = [[np.sort(rs.choice(np.arange(w0, 61), size=12, replace=False)).astype(np.int32) for g in range(2)]
            for b in range(2)]
    c2 = oracle.compact_gather(c, keep, window=window)
    lo = np.full((2, 2), w0 // page)
    got = oracle.page_bounds_refresh(c2, meta, "from", page_lo=lo)
    want = oracle.page_bounds_build(c2)
    for b in range(2):
        for g in range(2):
            n_pages = -(-int(c2.n_slots[b, g]) // page)
            np.testing.assert_array_equal(got[b, g, :n_pages], want[b, g, :n_pages])
            np.testing.assert_array_equal(got[b, g, n_pages:], meta[b, g, n_pages:])


# ------------------------------------------------------------------ decode -------------------------------------------
def test_decode_matches_library_attention():
    inp = tiny_snapkv(B=2, hq=4, hkv=2, d=8, N=40)
    c = inp["cache"]
    out, _ = oracle.decode_attn(c, inp["q_dec"], inp["scale"])
    K = torch.from_numpy(W.gather_contiguous(c, "k")[:, :, :40].astype(np.float64))
    V = torch.from_numpy(W.gather_contiguous(c, "v")[:, :, :40].astype(np.float64))
    q = torch.from_numpy(inp["q_dec"].astype(np.float64))[:, :, None, :]  # [B, hq, 1, d]
    Kr = K.repeat_interleave(2, dim=1)
    Vr = V.repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, Kr, Vr, scale=inp["scale"])[:, :, 0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_decode_special_views():
    inp = tiny_snapkv(B=1, hq=4, hkv=2, d=8, N=40)
    c = inp["cache"]
    pages = [[[3], [3]]]
    c1 = c.copy()
    c1.pos_map[0, :, 12:15] = -1  # page 3 keeps only slot 15
    out, _ = oracle.decode_attn(c1, inp["q_dec"], inp["scale"], pages=pages)
    V = W.gather_contiguous(c, "v").astype(np.float64)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], V[0, h // 2, 15])
    c2 = c.copy()
    K = W.gather_contiguous(c, "k").astype(np.float64)
    for g in range(2):
        set_keys(c2, 0, g, range(40), [K[0, g, 0]] * 40)
    out2, _ = oracle.decode_attn(c2, inp["q_dec"], inp["scale"])
    for h in range(4):
        np.testing.assert_allclose(out2[0, h], V[0, h // 2, :40].mean(axis=0), atol=1e-13)
    allp = [[list(range(10)), list(range(10))]]
    o_all, _ = oracle.decode_attn(c, inp["q_dec"], inp["scale"], pages=allp)
    o_dense, _ = oracle.decode_attn(c, inp["q_dec"], inp["scale"])
    np.testing.assert_allclose(o_all, o_dense, atol=1e-14)


def test_decode_cumulative_mass_is_group_size():
    cfg = W.H2O("tiny", B=2, hq=8, hkv=2, d=8, N=30, budget=28, recent=4, steps=3, zipf=1.1, page=4)
    inp = W.gen_h2o(cfg, seed=1, threads=1)
    c = inp["cache"]
    _, cum = oracle.decode_attn(c, inp["q_steps"][0], inp["scale"], accumulate=True)
    np.testing.assert_allclose(cum.sum(axis=2), 4.0, rtol=1e-6)
    assert cum.dtype == np.float32


# ------------------------------------------------------------------ pipelines --------------------------------------
def test_h2o_loop_invariants_brute_force():
    cfg = W.H2O("tiny", B=1, hq=4, hkv=2, d=8, N=48, budget=48, recent=8, steps=24, zipf=1.1, page=4)
    inp = W.gen_h2o(cfg, seed=2, threads=1)
    c = inp["cache"]
    # brute-force sequential simulation with plain dicts: position -> (k, v, cum)
    K = {g: {p: W.bf16_bits_to_f32(c.k_pool[c.block_table[0, p // 4], g, p % 4]).astype(np.float64)
             for p in range(48)} for g in range(2)}
    V = {g: {p: W.bf16_bits_to_f32(c.v_pool[c.block_table[0, p // 4], g, p % 4]).astype(np.float64)
             for p in range(48)} for g in range(2)}
    cum = {g: {p: np.float32(0) for p in range(48)} for g in range(2)}
    for step in range(24):
        c, info = P.h2o_step(inp, c, step)
        pnew = 48 + step
        for g in range(2):
            K[g][pnew] = W.bf16_bits_to_f32(inp["k_new"][step, 0, g]).astype(np.float64)
            V[g][pnew] = W.bf16_bits_to_f32(inp["v_new"][step, 0, g]).astype(np.float64)
            cum[g][pnew] = np.float32(0)
            ps = sorted(K[g])
            mass = {p: 0.0 for p in ps}
            for h in (2 * g, 2 * g + 1):
                q = W.bf16_bits_to_f32(inp["q_steps"][step, 0, h]).astype(np.float64)
                z = {p: inp["scale"] * float(K[g][p] @ q) for p in ps}
                mx = max(z.values())
                den = sum(math.exp(z[p] - mx) for p in ps)
                o = sum(math.exp(z[p] - mx) / den * V[g][p] for p in ps)
                np.testing.assert_allclose(info["out"][0, h], o, atol=1e-12)
                for p in ps:
                    mass[p] += math.exp(z[p] - mx) / den
            for p in ps:
                cum[g][p] = np.float32(float(cum[g][p]) + mass[p])
            # evict: lowest cum among pos <= pnew - 8, ties to higher pos
            elig = [p for p in ps if p <= pnew - 8]
            victim = min(elig, key=lambda p: (cum[g][p], -p))
            ev = info["evict"][0][g].tolist()
            assert len(ev) == 1
            assert int(np.where(c.slot_stack[0, g, :c.slot_top[0, g]] == ev[0])[0].size) == 1
            assert info["slots"][0, g] >= 0
            pos_evicted = [p for p in ps if p == victim][0]
            assert pos_evicted <= pnew - 8
            del K[g][victim], V[g][victim], cum[g][victim]
            res = set(int(x) for x in c.pos_map[0, g] if x >= 0)
            assert res == set(K[g]) and len(res) == 48 and c.ctx_len[0, g] == 48


def test_append_into_a_slot_with_a_stale_score_starts_it_at_zero():
    """H2O's cumulative score of a token is the attention it has received since it was written (SparseEngine page,
    "What it is": continuous scores during generation). A freed slot may still carry an old score (a caller that
    freed it without clearing, or stale values past the high-water mark). After one H2O step appends into such a
    slot, the new token's score must be exactly this step's group weight on it, formed here by an explicit softmax,
    and every older token's score its old value plus its weight; a new chunk's high-water slots start at zero."""
    cfg = W.H2O("tiny", B=1, hq=4, hkv=2, d=8, N=20, budget=100, recent=2, steps=1, zipf=1.1, page=4)
    inp = W.gen_h2o(cfg, seed=4, threads=1)
    c = inp["cache"]
    c.cum_score[:] = 3.0  # every slot, resident or not, holds a score of 3
    for g in range(2):  # free slot 5 the way a careless caller might: its score stays behind
        c.pos_map[0, g, 5] = -1
        c.slot_stack[0, g, c.slot_top[0, g]] = 5
        c.slot_top[0, g] += 1
        c.ctx_len[0, g] -= 1
    out, info = P.h2o_step(inp, c, 0)
    assert info["slots"].tolist() == [[5, 5]]
    for g in range(2):
        res = [s for s in range(20) if s == 5 or c.pos_map[0, g, s] >= 0]
        K = {s: W.bf16_bits_to_f32(inp["k_new"][0, 0, g] if s == 5 else
                                   c.k_pool[c.block_table[0, s // 4], g, s % 4]).astype(np.float64) for s in res}
        mass = dict.fromkeys(res, 0.0)
        for h in (2 * g, 2 * g + 1):
            q = W.bf16_bits_to_f32(inp["q_steps"][0, 0, h]).astype(np.float64)
            z = {s: inp["scale"] * float(K[s] @ q) for s in res}
            den = sum(math.exp(v) for v in z.values())
            for s in res:
                mass[s] += math.exp(z[s]) / den
        assert out.cum_score[0, g, 5] == np.float32(mass[5])
        for s in res:
            if s != 5:
                assert out.cum_score[0, g, s] == np.float32(3.0 + mass[s])
    # a chunk at the high-water mark: slots 20.. held stale scores of 3 and start at 0
    kc = np.zeros((1, 2, 3, 8), c.k_pool.dtype)
    after = oracle.cache_append_chunk(c, kc, kc, np.array([20], np.int32))
    assert np.all(after.cum_score[0, :, 20:23] == 0) and np.all(after.cum_score[0, :, :5] == 3.0)


# ------------------------------------------------------------------ compression policy loop --------------------
def tiny_kara_loop(B=5, period=8, events=2, cand_frac=0.2, budget_frac=0.2, seed=3):
    cfg = W.scaled(W.C2, B=B, hq=4, hkv=2, d=16, N=300, window=64, protect=8, period=period, events=events,
                   cand_frac=cand_frac, budget_frac=budget_frac, dtype="f32", page=4)
    return W.gen_kara(cfg, seed=seed, threads=1)


def event_kw(inp):
    cfg = inp["cfg"]
    return dict(scale=inp["scale"], window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                max_gap=cfg.max_gap)


def assert_same_state(a, b, seqs):
    """Per-sequence state and the resident K/V rows of the given sequences are identical."""
    Ka, Kb = W.gather_contiguous(a, "k"), W.gather_contiguous(b, "k")
    Va, Vb = W.gather_contiguous(a, "v"), W.gather_contiguous(b, "v")
    for s in seqs:
        np.testing.assert_array_equal(a.pos_map[s], b.pos_map[s])
        np.testing.assert_array_equal(a.n_slots[s], b.n_slots[s])
        np.testing.assert_array_equal(a.ctx_len[s], b.ctx_len[s])
        res = a.pos_map[s] >= 0
        np.testing.assert_array_equal(Ka[s][res], Kb[s][res])
        np.testing.assert_array_equal(Va[s][res], Vb[s][res])


def test_event_on_a_sequence_range_acts_on_those_sequences_alone():
    inp = tiny_kara_loop()
    cfg, c = inp["cfg"], inp["cache"]
    q = P.kara_recent_window_queries(inp, 0, cfg.B, -1)
    full = P.kara_event_range(c, q, 0, cfg.B, **event_kw(inp))
    # the whole batch as one range is the event over the batch (before any step the most recent tokens are the
    # window's slots, whose queries the plain event looks up by position)
    plain = P.kara_event(inp, c)
    assert_same_state(full["cache"], plain["cache"], range(cfg.B))
    assert full["cache"].free_top[0] == plain["cache"].free_top[0] > c.free_top[0]
    part = P.kara_event_range(c, q[1:3], 1, 3, **event_kw(inp))
    out = part["cache"]
    # sequences 1 and 2 end as the batch-wide event leaves them, the others as they were
    assert_same_state(out, full["cache"], [1, 2])
    assert_same_state(out, c, [0, 3, 4])
    np.testing.assert_array_equal(out.block_table[[0, 3, 4]], c.block_table[[0, 3, 4]])
    # the freed blocks are those the batch-wide event freed from sequences 1 and 2, in the same order
    top0 = int(c.free_top[0])
    owned = set(c.block_table[1:3].ravel().tolist()) - {-1}
    pushed_full = full["cache"].free_blocks[top0:full["cache"].free_top[0]].tolist()
    pushed = out.free_blocks[top0:out.free_top[0]].tolist()
    assert pushed == [x for x in pushed_full if x in owned] and len(pushed) > 0
    used = out.block_table[out.block_table >= 0].tolist()
    assert sorted(used + out.free_blocks[:out.free_top[0]].tolist()) == list(range(out.num_blocks))


@pytest.mark.parametrize("B,period", [(6, 8), (128, 128), (20, 4), (3, 16)])
def test_policy_schedules(B, period):
    T = 3 * period
    for policy in ("periodic", "threshold"):
        fired = {b: [] for b in range(B)}
        per_step = []
        for t in range(T):
            due = P.policy_due(policy, t, B, period)
            assert due == sorted(set(due))
            per_step.append(len(due))
            for b in due:
                fired[b].append(t)
        for b in range(B):
            # one compression per `period` decode steps under either policy
            assert len(fired[b]) == 3 and np.all(np.diff(fired[b]) == period)
            if policy == "periodic":
                assert fired[b][0] == period - 1
            else:
                assert fired[b][0] == period - 1 - (b * period) // B
        if policy == "threshold":
            # the staggered tails spread the events: no step holds more than ceil(B / period)
            assert max(per_step) == -(-B // period)
        else:
            assert max(per_step) == B and per_step.count(B) == 3
    assert P.runs_of([0, 1, 2, 4, 5, 9]) == [(0, 3), (4, 6), (9, 10)]
    assert P.runs_of([]) == []


@pytest.mark.parametrize("policy", ["periodic", "threshold"])
def test_policy_loop_with_full_budget_is_plain_decode(policy):
    # budget and candidates covering the whole window keep every slot: each event is the identity, so the loop
    # equals plain decode steps (append, then attend)
    inp = tiny_kara_loop(cand_frac=1.0, budget_frac=1.0)
    cfg = inp["cfg"]
    assert cfg.n_cand == cfg.window - cfg.protect and cfg.budget == cfg.window
    cache, outs, events = P.kara_policy_loop(inp, inp["cache"], policy, cfg.steps)
    want = [(t, b0, b1) for t in range(cfg.steps) for b0, b1 in P.runs_of(P.policy_due(policy, t, cfg.B, cfg.period))]
    assert events == want and len(events) > 0
    st = inp["cache"]
    for t in range(cfg.steps):
        st, o = P.kara_decode_step(inp, st, t)
        np.testing.assert_array_equal(outs[t], o)
    assert_same_state(cache, st, range(cfg.B))
    assert cache.free_top[0] == st.free_top[0]


@pytest.mark.parametrize("policy", ["periodic", "threshold"])
def test_policy_loop_invariants(policy):
    inp = tiny_kara_loop()
    cfg = inp["cfg"]
    cache, outs, events = P.kara_policy_loop(inp, inp["cache"], policy, cfg.steps)
    assert len(events) > 0
    T = cfg.N + cfg.steps
    for b in range(cfg.B):
        for g in range(cfg.hkv):
            n = int(cache.n_slots[b, g])
            pos = cache.pos_map[b, g, :n]
            # dense, in position order, every position at most once, the newest token kept; each event's window
            # reaches back at most one region past what earlier events removed, so the prefix before that stays
            assert np.all(pos >= 0) and np.all(np.diff(pos) > 0) and pos[-1] == T - 1
            assert int(cache.ctx_len[b, g]) == n < T
            n_ev = sum(1 for _, b0, b1 in events if b0 <= b < b1)
            keep0 = cfg.N - cfg.window - n_ev * (cfg.window - cfg.protect)
            assert n_ev == cfg.events and keep0 > 0
            np.testing.assert_array_equal(pos[:keep0], np.arange(keep0))
    used = cache.block_table[cache.block_table >= 0].tolist()
    assert sorted(used + cache.free_blocks[:cache.free_top[0]].tolist()) == list(range(cache.num_blocks))


def test_recent_window_queries_are_those_of_the_latest_positions():
    inp = tiny_kara_loop()
    cfg = inp["cfg"]
    for t in (-1, 0, 5, cfg.steps - 1):
        q = P.kara_recent_window_queries(inp, 1, 4, t)
        last = cfg.N + t  # position of the token step t appended (t = -1: the prompt's last)
        for j, p in enumerate(range(last - cfg.window + 1, last + 1)):
            np.testing.assert_array_equal(q[:, :, j], inp["q_all"][1:4, :, p - inp["q_first_pos"]])
    with pytest.raises(ValueError):
        P.kara_recent_window_queries(inp, 0, 1, -2)
