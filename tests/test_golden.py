"""Oracle against hand-worked examples (tests/golden/*.json, each citing the passage it follows)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle.cache_ops import CapacityError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def small_cache(B, n_kv, page, N, max_blocks, num_blocks, d=2, dtype="f32", fill="ids", with_cum=False):
    c = W.empty_cache(B, n_kv, d, page, max_blocks, num_blocks, dtype, slot_cap=4, with_cum=with_cum)
    nb = W.layout_initial(c, N)
    for b in range(B):
        x = np.zeros((n_kv, N, d), np.float32)
        for g in range(n_kv):
            for s in range(N):
                x[g, s, :] = 1000 * b + 100 * g + s  # identifies (b, g, original slot)
        W.write_sequence(c.k_pool, nb, b, W.to_storage(x, dtype), page)
        W.write_sequence(c.v_pool, nb, b, W.to_storage(-x, dtype), page)
    return c


# ---------------------------------------------------------------------------------------------------------------
def test_token2chunk_golden():
    fx = load("token2chunk_small.json")
    for case in fx["cases"]:
        c = W.empty_cache(1, 1, 2, 16, 2, 2, "f32")
        c.n_slots[:] = fx["n_slots"]
        c.ctx_len[:] = fx["n_slots"]
        c.pos_map[0, 0, :fx["n_slots"]] = np.arange(fx["n_slots"])
        scores = np.zeros((1, 1, fx["window"] - fx["protect"]), np.float32)
        for k, v in case["scores"].items():
            scores[0, 0, int(k)] = v
        sel = case["candidates"] + list(range(fx["n_slots"] - fx["protect"], fx["n_slots"]))
        out = oracle.token2chunk([[np.array(sel, np.int32)]], scores, c, max_gap=fx["max_gap"],
                                 budget=case["budget"], window=fx["window"], protect=fx["protect"])
        assert out[0][0].tolist() == case["expected"], case["why"]


def test_topk_largest_slots_golden():
    fx = load("topk_small.json")
    for case in fx["largest_slots"]:
        n = len(case["scores"])
        c = W.empty_cache(1, 1, 2, 16, 1, 1, "f32")
        c.n_slots[:] = n
        c.pos_map[0, 0, :n] = case["pos"]
        c.ctx_len[:] = sum(p >= 0 for p in case["pos"])
        scores = np.zeros((1, 1, 16), np.float32)
        scores[0, 0, :n] = case["scores"]
        out = oracle.topk_largest(scores, c, case["k"], protect=case["protect"])
        assert out[0][0].tolist() == case["expected"], case["why"]


def test_topk_largest_pages_golden():
    fx = load("topk_small.json")
    for case in fx["largest_pages"]:
        c = W.empty_cache(1, 1, 2, 16, 8, 8, "f32")
        c.n_slots[:] = case["n_slots"]
        scores = np.full((1, 1, 8), -np.inf, np.float32)
        scores[0, 0, :len(case["scores"])] = case["scores"]
        out = oracle.topk_largest(scores, c, case["k"], unit="page", forced_ends=True)
        assert out[0][0].tolist() == case["expected"], case["why"]


def test_topk_smallest_golden():
    fx = load("topk_small.json")
    for case in fx["smallest"]:
        n = len(case["cum"])
        c = W.empty_cache(1, 1, 2, 16, 1, 1, "f32")
        c.n_slots[:] = n
        c.ctx_len[:] = n
        c.pos_map[0, 0, :n] = np.arange(n)
        cum = np.zeros((1, 1, 16), np.float32)
        cum[0, 0, :n] = case["cum"]
        out = oracle.topk_smallest(cum, c, 1, budget=case["budget"], recent=case["recent"])
        assert out[0][0].tolist() == case["expected"], case["why"]


def test_compact_whole_golden():
    fx = load("cache_ops_small.json")["compact_whole"]
    c = small_cache(fx["B"], fx["n_kv"], fx["page"], fx["N"], fx["max_blocks"], fx["num_blocks"])
    assert c.free_blocks[:c.free_top[0]].tolist() == [9, 8]
    keep = [[np.array(x, np.int32) for x in row] for row in fx["keep"]]
    out = oracle.compact_gather(c, keep)
    assert out.block_table.tolist() == fx["expected_block_table"]
    assert out.free_blocks[:out.free_top[0]].tolist() == fx["expected_free"]
    assert out.n_slots.tolist() == fx["expected_n_slots"]
    assert out.ctx_len.tolist() == fx["expected_ctx"]
    for b in range(fx["B"]):
        for g in range(fx["n_kv"]):
            exp = fx["expected_pos_prefix"][b][g]
            n = len(exp)
            assert out.pos_map[b, g, :n].tolist() == exp
            assert np.all(out.pos_map[b, g, n:] == -1)
            for j, s in enumerate(exp):  # K/V rows carry their original (b, g, slot) id
                blk = out.block_table[b, j // fx["page"]]
                assert out.k_pool[blk, g, j % fx["page"], 0] == 1000 * b + 100 * g + s
                assert out.v_pool[blk, g, j % fx["page"], 1] == -(1000 * b + 100 * g + s)


def test_compact_trailing_golden():
    fx = load("cache_ops_small.json")["compact_trailing"]
    c = small_cache(fx["B"], fx["n_kv"], fx["page"], fx["N"], fx["max_blocks"], fx["num_blocks"])
    keep = [[np.array(x, np.int32) for x in row] for row in fx["keep"]]
    out = oracle.compact_gather(c, keep, window=fx["window"])
    assert out.block_table.tolist() == fx["expected_block_table"]
    assert out.free_blocks[:out.free_top[0]].tolist() == fx["expected_free"]
    assert out.n_slots.tolist() == fx["expected_n_slots"]
    assert out.ctx_len.tolist() == fx["expected_ctx"]
    exp = fx["expected_pos_prefix"][0][0]
    assert out.pos_map[0, 0, :len(exp)].tolist() == exp
    for j, s in enumerate(exp):
        blk = out.block_table[0, j // fx["page"]]
        assert out.k_pool[blk, 0, j % fx["page"], 0] == s


def test_evict_append_golden():
    fx = load("cache_ops_small.json")["evict_append"]
    c = small_cache(fx["B"], fx["n_kv"], fx["page"], fx["N"], fx["max_blocks"], fx["num_blocks"])
    assert c.free_blocks[:c.free_top[0]].tolist() == [3, 2]
    c = oracle.evict_slots(c, [[np.array(x, np.int32) for x in row] for row in fx["evict"]])
    assert c.slot_top.tolist() == [[1, 0]] and c.ctx_len.tolist() == [[7, 8]]
    for step, p in enumerate(fx["appends"]):
        k = np.full((fx["B"], fx["n_kv"], 2), 50.0 + step, np.float32)
        c, slots = oracle.cache_append(c, k, -k, np.array([p], np.int32))
        assert slots.tolist() == fx["expected_slots"][step]
    assert c.block_table.tolist() == fx["expected_block_table"]
    assert int(c.free_top[0]) == fx["expected_free_top"]
    assert c.n_slots.tolist() == fx["expected_n_slots"]
    assert c.ctx_len.tolist() == fx["expected_ctx"]
    assert c.pos_map.tolist() == fx["expected_pos"]
    assert c.k_pool[0, 0, 3, 0] == 50.0 and c.k_pool[2, 1, 0, 0] == 50.0 and c.k_pool[2, 1, 1, 0] == 51.0


def test_append_capacity_all_or_nothing():
    fx = load("cache_ops_small.json")["evict_append"]
    c = small_cache(1, 1, 4, 8, 3, 2)  # no spare blocks at all
    assert int(c.free_top[0]) == 0
    with pytest.raises(CapacityError):
        oracle.cache_append(c, np.zeros((1, 1, 2), np.float32), np.zeros((1, 1, 2), np.float32),
                            np.array([8], np.int32))


def test_page_bounds_golden():
    fx = load("page_bounds_small.json")
    c = W.empty_cache(1, 1, 2, 2, 2, 2, "f32")
    W.layout_initial(c, 4)
    c.pos_map[0, 0, :4] = fx["pos"]
    c.ctx_len[:] = 3
    keys = np.array(fx["keys"], np.float32)
    W.write_sequence(c.k_pool, 2, 0, keys[None], 2)
    meta = oracle.page_bounds_build(c)
    assert meta[0, 0, :, 0].tolist() == fx["expected_min"]
    assert meta[0, 0, :, 1].tolist() == fx["expected_max"]
    q = np.array(fx["q"], np.float32)[None]  # hq = 2 over one KV head: a group of 2
    u = oracle.page_bounds_score(c, meta, q)
    assert u[0, 0, :2].tolist() == fx["expected_scores"]
