"""Helpers of the GPU parity tests: move workload state to the device and compare results with the oracle."""
import numpy as np
import torch

import oracle
import sparse_decode_attention_se_amd as se
import workloads as W
from oracle import pipelines as P
from sparse_decode_attention_se_amd import workflows as WF

DEV = "cuda:0"


def to_device(state: W.CacheState, n_q: int) -> se.DeviceCache:
    arrays = {f: getattr(state, f) for f in se.DeviceCache.FIELDS if getattr(state, f, None) is not None}
    return se.DeviceCache.from_arrays(n_q, state.dtype, DEV, **arrays)


def storage_tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def i32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)


def status_word() -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def lists_from(idx: torch.Tensor, count: torch.Tensor):
    idx = idx.cpu().numpy()
    count = count.cpu().numpy()
    B, G = count.shape
    return [[idx[b, g, :count[b, g]].copy() for g in range(G)] for b in range(B)]


def assert_scores_close(gpu: np.ndarray, ora: np.ndarray, mass: np.ndarray, rtol=1e-3, floor=1e-6):
    """|gpu - ora| <= rtol |ora| for every score. A pair where both values are below floor * row mass counts as a
    tie at zero (float32 exponentials underflow and flush where float64 ones do not); no other slack."""
    g = gpu.astype(np.float64)
    tie = (np.abs(g) <= floor * mass[..., None]) & (np.abs(ora) <= floor * mass[..., None])
    bad = (np.abs(g - ora) > rtol * np.abs(ora)) & ~tie
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} scores differ, first at {tuple(i)}: gpu {gpu[tuple(i)]} oracle "
                             f"{ora[tuple(i)]}")


def assert_sets_match_modulo_ties(gpu_list, ora_list, ora_scores_row, base=0, rtol=1e-3, floor=0.0):
    """Retained sets equal except for swaps whose oracle scores are within rtol (relative) or below floor."""
    G, O = set(int(x) for x in gpu_list), set(int(x) for x in ora_list)
    assert len(G) == len(O), (len(G), len(O))
    for x in G - O:
        for y in O - G:
            sx, sy = float(ora_scores_row[x - base]), float(ora_scores_row[y - base])
            if max(abs(sx), abs(sy)) <= floor:
                continue
            assert abs(sx - sy) <= rtol * max(abs(sx), abs(sy)), (x, y, sx, sy)
    return len(G - O)


def assert_token2chunk_of(keep_lists, cand_lists, scores32, cache, *, max_gap, budget, window, protect):
    """Where several results are correct: the device's kept lists must be exactly the oracle's Token2Chunk of the
    device's own candidates and float32 scores (the fill is a deterministic function of those two)."""
    want = oracle.token2chunk(cand_lists, scores32, cache, max_gap=max_gap, budget=budget, window=window,
                              protect=protect)
    for b, row in enumerate(want):
        for g, w in enumerate(row):
            assert np.asarray(keep_lists[b][g]).tolist() == w.tolist(), (b, g)


def resident_rows(arrays: dict, page: int, which: str, b: int, g: int, n: int):
    """[n][d] rows of slots 0..n-1 of (b, g) read through the block table (bit patterns)."""
    pool = arrays[which]
    bt = arrays["block_table"][b]
    s = np.arange(n)
    return pool[bt[s // page], g, s % page]


def compare_cache(dev: dict, ora: W.CacheState, data=True, cum_exact=True, cum_mass=None):
    """Bit-exact comparison of everything the cache defines (slots below n_slots; stack entries below top). With
    cum_exact False the cumulative scores are compared as scores: 1e-3 relative, values below 1e-6 of the per-unit
    mass ``cum_mass`` [B][n_kv] on both sides counting as ties at zero."""
    np.testing.assert_array_equal(dev["n_slots"], ora.n_slots)
    np.testing.assert_array_equal(dev["ctx_len"], ora.ctx_len)
    np.testing.assert_array_equal(dev["block_table"], ora.block_table)
    assert int(dev["free_top"][0]) == int(ora.free_top[0])
    top = int(ora.free_top[0])
    np.testing.assert_array_equal(dev["free_blocks"][:top], ora.free_blocks[:top])
    np.testing.assert_array_equal(dev["slot_top"], ora.slot_top)
    B, G = ora.n_slots.shape
    for b in range(B):
        for g in range(G):
            n = int(ora.n_slots[b, g])
            np.testing.assert_array_equal(dev["pos_map"][b, g, :n], ora.pos_map[b, g, :n])
            t = int(ora.slot_top[b, g])
            np.testing.assert_array_equal(dev["slot_stack"][b, g, :t], ora.slot_stack[b, g, :t])
            if data and n:
                res = ora.pos_map[b, g, :n] >= 0
                for which in ("k_pool", "v_pool"):
                    dr = resident_rows(dev, ora.page, which, b, g, n)[res]
                    orr = resident_rows({which: getattr(ora, which), "block_table": ora.block_table}, ora.page,
                                        which, b, g, n)[res]
                    np.testing.assert_array_equal(dr, orr)
            if ora.cum_score is not None and n:
                if cum_exact:
                    np.testing.assert_array_equal(dev["cum_score"][b, g, :n], ora.cum_score[b, g, :n])
                else:
                    assert cum_mass is not None, "inexact cumulative scores need the unit's mass"
                    assert_scores_close(dev["cum_score"][b, g, :n][None], ora.cum_score[b, g, :n][None].astype(
                        np.float64), mass=np.array([cum_mass[b, g]], np.float64))


def run_h2o_teacher_forced(inp, dc, st, steps, seqs=None, status=None, check_every=1):
    """H2O decode steps on the device (every sequence of dc) and on the oracle (the sequences ``seqs`` of the
    device's batch, held in ``st`` as a cache of their own; all when None), in lock-step. At every step and every
    sampled head: the decode output within 2e-3, and the device's evicted slot equal to the oracle's or a near tie
    of it by the oracle's cumulative scores, after which the oracle continues from the device's eviction (teacher
    forcing). Every ``check_every`` steps the sampled sequences' maps, stacks and cumulative scores are compared."""
    cfg = inp["cfg"]
    B_dev = int(dc.pos_map.shape[0])
    seqs = list(range(B_dev)) if seqs is None else list(seqs)
    r = cfg.hq // cfg.hkv
    step = WF.H2OStep(dc, scale=inp["scale"], budget=cfg.budget, recent=cfg.recent, status=status)
    swaps = 0
    for s in range(steps):
        pos = np.full((B_dev,), cfg.N + s, np.int32)
        o = step.run(storage_tensor(inp["k_new"][s], "bf16"), storage_tensor(inp["v_new"][s], "bf16"), i32(pos),
                     storage_tensor(inp["q_steps"][s], "bf16")).cpu().numpy()
        ev_all = lists_from(step.evict, step.evict_count)
        ev = [ev_all[b] for b in seqs]
        sub = dict(inp, cfg=W.scaled(cfg, B=len(seqs)), k_new=inp["k_new"][:, seqs], v_new=inp["v_new"][:, seqs],
                   q_steps=inp["q_steps"][:, seqs])
        st, info = P.h2o_step(sub, st, s, evict=ev)
        mass = r * (s + 1)
        for i, b in enumerate(seqs):
            np.testing.assert_allclose(o[b], info["out"][i], atol=2e-3, rtol=0)
            for g in range(cfg.hkv):
                swaps += assert_sets_match_modulo_ties(ev[i][g], info["evict"][i][g], info["cum"][i, g],
                                                       floor=1e-6 * mass)
        if (s + 1) % check_every == 0 or s == steps - 1:
            d = {f: getattr(dc, f).cpu().numpy() for f in ("n_slots", "ctx_len", "pos_map", "slot_top", "slot_stack",
                                                          "cum_score")}
            for i, b in enumerate(seqs):
                for g in range(cfg.hkv):
                    n = int(st.n_slots[i, g])
                    assert int(d["n_slots"][b, g]) == n and int(d["ctx_len"][b, g]) == int(st.ctx_len[i, g])
                    np.testing.assert_array_equal(d["pos_map"][b, g, :n], st.pos_map[i, g, :n])
                    t = int(st.slot_top[i, g])
                    assert int(d["slot_top"][b, g]) == t
                    np.testing.assert_array_equal(d["slot_stack"][b, g, :t], st.slot_stack[i, g, :t])
                    assert_scores_close(d["cum_score"][b, g, :n][None], st.cum_score[i, g, :n][None].astype(
                        np.float64), mass=np.array([float(mass)]))
    return st, swaps
