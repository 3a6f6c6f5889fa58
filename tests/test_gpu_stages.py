"""Stage-isolated parity: each libse call against the oracle on the same seeded inputs (small sizes that still
span several tiles and a ragged tail). Index, map and list results are bit-exact; floats within the stated
tolerances (scores 1e-3 relative with a 1e-6 row-mass floor, decode outputs 2e-3 absolute)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_se_amd as se
import workloads as W
from gpu_util import (DEV, assert_scores_close, assert_sets_match_modulo_ties, compare_cache, i32, lists_from,
                      status_word, storage_tensor, to_device)
from sparse_decode_attention_se_amd import workflows as WF

pytestmark = pytest.mark.gpu


def banner(name):
    print(f"\n[case] {name}", flush=True)


def snap_inputs(B=2, hq=8, hkv=2, d=128, N=1500, wq=64, protect=64, keep=200, dtype="bf16", seed=0, spikes=0.04,
                page=16):
    cfg = W.SnapKV("t", B=B, hq=hq, hkv=hkv, d=d, N=N, wq=wq, protect=protect, keep=keep, dtype=dtype,
                   spike_frac=spikes, page=page)
    return W.gen_snapkv(cfg, seed=seed, threads=4)


def punch_holes(state, frac, seed, slot_cap=8):
    """Evict a few slots (oracle semantics) so the cache has free slots on its slot stacks."""
    rs = np.random.default_rng(seed)
    B, G = state.n_slots.shape
    ev = [[np.sort(rs.choice(int(state.n_slots[b, g]), size=min(slot_cap, max(1, int(frac * state.n_slots[b, g]))),
                             replace=False)).astype(np.int32) for g in range(G)] for b in range(B)]
    return oracle.evict_slots(state, ev)


# ------------------------------------------------------------------ decode --------------------------------------
@pytest.mark.parametrize("dtype,d,N", [("bf16", 128, 777), ("f32", 64, 777), ("bf16", 128, 40), ("f32", 64, 40)])
def test_decode_all_slots(dtype, d, N):
    # N = 40: the whole view is one chunk, whose workgroup writes the output without partials
    banner(f"decode all slots {dtype} N={N}")
    inp = snap_inputs(d=d, dtype=dtype, N=N, wq=8, protect=8, keep=16)
    st = punch_holes(inp["cache"], 0.01, 1)
    ref, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"])
    dc = to_device(st, 8)
    out = torch.empty((2, 8, d), dtype=torch.float32, device=DEV)
    status = status_word()
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], dtype), out, scale=inp["scale"], status=status)
    assert se.se_status_read(status) == 0
    np.testing.assert_allclose(out.cpu().numpy(), ref, atol=2e-3, rtol=0)


def test_decode_many_units_256_row_chunks():
    # 64 units of 2100 slots: 256-row chunks (all four steps of a wave in flight), ragged last chunk
    banner("decode 64 units x 2100 slots")
    inp = snap_inputs(B=8, hq=32, hkv=8, N=2100, wq=8, protect=8, keep=16, seed=4)
    st = punch_holes(inp["cache"], 0.01, 5)
    ref, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"])
    dc = to_device(st, 32)
    out = torch.empty((8, 32, 128), dtype=torch.float32, device=DEV)
    status = status_word()
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], status=status)
    assert se.se_status_read(status) == 0
    np.testing.assert_allclose(out.cpu().numpy(), ref, atol=2e-3, rtol=0)


def test_decode_max_slots_bound_and_pages():
    banner("decode page lists")
    inp = snap_inputs(N=1000)
    st = inp["cache"]
    rs = np.random.default_rng(3)
    n_pages = -(-1000 // 16)
    pages = [[np.sort(rs.choice(n_pages, size=int(rs.integers(1, 20)), replace=False)).astype(np.int32)
              for g in range(2)] for b in range(2)]
    pages[0][0] = np.array([n_pages - 1], np.int32)  # ragged last page only
    ref, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"], pages=pages)
    sel, cnt = W.pack_lists(pages, 24)
    dc = to_device(st, 8)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    status = status_word()
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], sel_pages=i32(sel),
                             sel_count=i32(cnt), status=status)
    assert se.se_status_read(status) == 0
    np.testing.assert_allclose(out.cpu().numpy(), ref, atol=2e-3, rtol=0)
    # all pages selected == dense attention
    allp = [[np.arange(n_pages, dtype=np.int32)] * 2] * 2
    sel, cnt = W.pack_lists(allp, n_pages)
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], sel_pages=i32(sel),
                             sel_count=i32(cnt), status=status)
    dense, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"])
    np.testing.assert_allclose(out.cpu().numpy(), dense, atol=2e-3, rtol=0)
    # an n_slots bound below the real size is reported
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], max_slots=512,
                             status=status)
    assert se.se_status_read(status) & se.SE_DEV_CAPACITY


@pytest.mark.parametrize("B,N", [(3, 900), (3, 40), (1, 12000)])
def test_decode_accumulates_cumulative_scores(B, N):
    banner(f"decode cum B={B} N={N}")
    cfg = W.H2O("t", B=B, hq=8, hkv=2, d=128, N=N, budget=N, recent=min(32, N // 2), steps=2, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=5, threads=4)
    st = punch_holes(inp["cache"], 0.005, 2)
    st.cum_score[:] = np.random.default_rng(0).random(st.cum_score.shape).astype(np.float32)
    ref_out, ref_cum = oracle.decode_attn(st, inp["q_steps"][0], inp["scale"], accumulate=True)
    dc = to_device(st, 8)
    out = torch.empty((B, 8, 128), dtype=torch.float32, device=DEV)
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_steps"][0], "bf16"), out, scale=inp["scale"],
                             accumulate=True)
    np.testing.assert_allclose(out.cpu().numpy(), ref_out, atol=2e-3, rtol=0)
    cum = dc.cum_score.cpu().numpy()
    for b in range(B):
        for g in range(2):
            n = int(st.n_slots[b, g])
            res = st.pos_map[b, g, :n] >= 0
            np.testing.assert_allclose(cum[b, g, :n][res], ref_cum[b, g, :n][res], rtol=1e-5, atol=1e-7)
            np.testing.assert_array_equal(cum[b, g, :n][~res], st.cum_score[b, g, :n][~res])


def test_decode_workspace_needs_no_clearing():
    """The merge's arrival counters live in the workspace: garbage there, reuse across calls of other shapes and
    repeated calls all give the same outputs."""
    banner("decode workspace reuse")
    inp = snap_inputs(N=1000)
    st = inp["cache"]
    dc = to_device(st, 8)
    q = storage_tensor(inp["q_dec"], "bf16")
    ref, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"])
    ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
        se.se_sparse_decode_attn(dc, q, out, scale=inp["scale"], ws=ws)
        outs.append(out.cpu().numpy())
    np.testing.assert_allclose(outs[0], ref, atol=2e-3, rtol=0)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # a page-selected call of another size on the same workspace, then the dense one again
    n_pages = -(-1000 // 16)
    pages = [[np.arange(0, n_pages, 3, dtype=np.int32)] * 2] * 2
    sel, cnt = W.pack_lists(pages, n_pages)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    se.se_sparse_decode_attn(dc, q, out, scale=inp["scale"], sel_pages=i32(sel), sel_count=i32(cnt), ws=ws)
    ref_sel, _ = oracle.decode_attn(st, inp["q_dec"], inp["scale"], pages=pages)
    np.testing.assert_allclose(out.cpu().numpy(), ref_sel, atol=2e-3, rtol=0)
    se.se_sparse_decode_attn(dc, q, out, scale=inp["scale"], ws=ws)
    assert np.array_equal(out.cpu().numpy(), outs[0])


# ------------------------------------------------------------------ window scores -------------------------------
@pytest.mark.parametrize("N,page", [(1500, 16), (700, 16), (1500, 12), (300, 12)])
def test_window_score_causal_bf16(N, page):
    """Two-kernel path (1500 and 700 slots) and single-kernel path (a unit's keys in one chunk: 300 slots); page
    12 takes the addressing without power-of-two shifts."""
    banner(f"window causal bf16 N={N} page={page}")
    inp = snap_inputs(N=N, page=page)
    st = punch_holes(inp["cache"], 0.002, 4)
    ref = oracle.window_score_causal(st, inp["q_win"], inp["q_pos"], inp["scale"])
    dc = to_device(st, 8)
    S = st.pos_map.shape[2]
    scores = torch.zeros((2, 2, S), dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]), scores, scale=inp["scale"],
                       mode=se.SE_SCORE_CAUSAL, n_query=64)
    got = scores.cpu().numpy()
    assert_scores_close(got[:, :, :N], ref[:, :, :N], mass=np.full((2, 2), 4 * 64.0))
    np.testing.assert_allclose(got.sum(axis=2), 256.0, rtol=1e-5)


@pytest.mark.parametrize("case,wq", [("overflow", 64), ("underflow", 64), ("overflow", 128), ("underflow", 128)])
def test_window_score_causal_extreme_logits(case, wq):
    """Logits whose row sums of exp2(s c) leave [2^-80, 2^80]: the reference-free first pass must hand those chunks
    to the exact (running-max) pass. "overflow": the first 600 slots' keys scaled by 30, so only the chunks that
    hold them overflow (the others stay reference-free); "underflow": every key shifted along one direction and the
    queries against it, so every logit is near -900 and every row sum near 2^-104. wq = 128 gives two row groups
    (the other step width of the streaming kernels)."""
    banner(f"window causal bf16 extreme logits: {case} wq={wq}")
    inp = snap_inputs(N=1500, wq=wq)
    st = inp["cache"].copy()
    k = W.bf16_bits_to_f32(st.k_pool).reshape(st.k_pool.shape).astype(np.float64)
    q = W.bf16_bits_to_f32(inp["q_win"]).reshape(inp["q_win"].shape).astype(np.float64)
    if case == "overflow":
        page = st.page
        for b in range(2):
            for slot in range(600):
                k[st.block_table[b, slot // page], :, slot % page, :] *= 30.0
    else:
        u = np.random.default_rng(11).standard_normal(128)
        u /= np.linalg.norm(u)
        k += 30.0 * u
        q -= 30.0 * u
    st.k_pool = W.to_storage(k, "bf16").reshape(st.k_pool.shape)
    q_win = W.to_storage(q, "bf16").reshape(inp["q_win"].shape)
    ref = oracle.window_score_causal(st, q_win, inp["q_pos"], inp["scale"])
    dc = to_device(st, 8)
    S = st.pos_map.shape[2]
    scores = torch.zeros((2, 2, S), dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(q_win, "bf16"), i32(inp["q_pos"]), scores, scale=inp["scale"],
                       mode=se.SE_SCORE_CAUSAL, n_query=wq)
    got = scores.cpu().numpy()
    assert np.isfinite(got).all()
    assert_scores_close(got[:, :, :1500], ref[:, :, :1500], mass=np.full((2, 2), 4.0 * wq))
    np.testing.assert_allclose(got.sum(axis=2), 4.0 * wq, rtol=1e-5)


def test_window_score_causal_f32_c0():
    banner("window causal f32 (tiny workload, full size)")
    inp = W.gen_snapkv(W.C0, seed=0, threads=1)
    st = inp["cache"]
    ref = oracle.window_score_causal(st, inp["q_win"], inp["q_pos"], inp["scale"])
    dc = to_device(st, 8)
    scores = torch.zeros((1, 2, 1024), dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(inp["q_win"], "f32"), i32(inp["q_pos"]), scores, scale=inp["scale"],
                       mode=se.SE_SCORE_CAUSAL, n_query=32)
    assert_scores_close(scores.cpu().numpy(), ref, mass=np.full((1, 2), 4 * 32.0))


def test_window_score_bidir():
    banner("window bidir")
    cfg = W.Kara("t", B=2, hq=8, hkv=2, d=128, N=700, window=512, protect=64, cand_frac=0.2, budget_frac=0.2,
                 max_gap=8, period=4, events=1, rho=0.9)
    inp = W.gen_kara(cfg, seed=3, threads=4)
    st = inp["cache"]
    from oracle.pipelines import kara_window_queries

    qw = kara_window_queries(inp, st)
    ref = oracle.window_score_bidir(st, qw, inp["scale"], 512, 64)
    dc = to_device(st, 8)
    scores = torch.zeros((2, 2, 448), dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(qw, "bf16"), None, scores, scale=inp["scale"], mode=se.SE_SCORE_BIDIR,
                       n_query=512, window=512, protect=64)
    got = scores.cpu().numpy()
    assert_scores_close(got, ref, mass=np.full((2, 2), 4 * 512.0))
    np.testing.assert_allclose(got.sum(axis=2), 2048.0, rtol=1e-5)


@pytest.mark.parametrize("window,protect,holes", [(40, 8, 0.0), (512, 0, 0.0), (300, 17, 0.02)])
def test_window_score_bidir_shapes(window, protect, holes):
    """Region sizes the register-resident kernel handles differently: 32 keys (one tile per wave; two waves hold
    none), 512 keys (eight tiles per wave), and 283 keys (a partial last tile) with free slots in the region (the
    masked path). Two sequences x two KV heads: each unit's query rows are split over several workgroups."""
    banner(f"window bidir window={window} protect={protect} holes={holes}")
    cfg = W.Kara("t", B=2, hq=8, hkv=2, d=128, N=window + 200, window=window, protect=protect, cand_frac=0.2,
                 budget_frac=0.2, max_gap=8, period=4, events=1, rho=0.9)
    inp = W.gen_kara(cfg, seed=11, threads=4)
    st = inp["cache"]
    if holes:
        st = punch_holes(st, holes, 12)
    qw = W.to_storage(np.random.default_rng(13).standard_normal((2, 8, window, 128)), "bf16")
    ref = oracle.window_score_bidir(st, qw, inp["scale"], window, protect)
    dc = to_device(st, 8)
    R = window - protect
    scores = torch.full((2, 2, R), 7.0, dtype=torch.float32, device=DEV)
    status = status_word()
    se.se_window_score(dc, storage_tensor(qw, "bf16"), None, scores, scale=inp["scale"], mode=se.SE_SCORE_BIDIR,
                       n_query=window, window=window, protect=protect, status=status)
    assert se.se_status_read(status) == 0
    got = scores.cpu().numpy()
    assert_scores_close(got, ref, mass=np.full((2, 2), 4.0 * window))
    # every query row that sees a resident key gives it mass 1 per head
    for b in range(2):
        for g in range(2):
            n = int(st.n_slots[b, g])
            seen = np.any(st.pos_map[b, g, n - window:n - protect] >= 0)
            np.testing.assert_allclose(got[b, g].sum(), 4.0 * window * seen, rtol=1e-5)


@pytest.mark.parametrize("wq,N", [(128, 900), (20, 1300)])
def test_window_score_causal_row_groups(wq, N):
    """512 query rows per unit (two row groups, whose partial column sums a last kernel adds up) and 80 rows (a row
    count that is not a multiple of 16)."""
    banner(f"window causal bf16 wq={wq} N={N}")
    inp = snap_inputs(N=N, wq=wq)
    st = punch_holes(inp["cache"], 0.002, 5)
    ref = oracle.window_score_causal(st, inp["q_win"], inp["q_pos"], inp["scale"])
    dc = to_device(st, 8)
    S = st.pos_map.shape[2]
    scores = torch.zeros((2, 2, S), dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]), scores, scale=inp["scale"],
                       mode=se.SE_SCORE_CAUSAL, n_query=wq)
    got = scores.cpu().numpy()
    assert_scores_close(got[:, :, :N], ref[:, :, :N], mass=np.full((2, 2), 4.0 * wq))
    np.testing.assert_allclose(got.sum(axis=2), 4.0 * wq, rtol=1e-5)


def test_window_score_bidir_long_window():
    """A 1024-token window (960 region keys): the two-kernel path in bidirectional mode."""
    banner("window bidir, window 1024")
    cfg = W.Kara("t", B=2, hq=8, hkv=2, d=128, N=1500, window=1024, protect=64, cand_frac=0.2, budget_frac=0.2,
                 max_gap=8, period=4, events=1, rho=0.9)
    inp = W.gen_kara(cfg, seed=4, threads=4)
    st = inp["cache"]
    from oracle.pipelines import kara_window_queries

    qw = kara_window_queries(inp, st)
    ref = oracle.window_score_bidir(st, qw, inp["scale"], 1024, 64)
    dc = to_device(st, 8)
    scores = torch.zeros((2, 2, 960), dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(qw, "bf16"), None, scores, scale=inp["scale"], mode=se.SE_SCORE_BIDIR,
                       n_query=1024, window=1024, protect=64)
    got = scores.cpu().numpy()
    assert_scores_close(got, ref, mass=np.full((2, 2), 4 * 1024.0))
    np.testing.assert_allclose(got.sum(axis=2), 4096.0, rtol=1e-5)


# ------------------------------------------------------------------ top-K -----------------------------------------
def _topk_cache(B=2, G=3, N=3000, page=16):
    c = W.empty_cache(B, G, 128, page, -(-N // page), B * -(-N // page), "bf16")
    W.layout_initial(c, N)
    return c


@pytest.mark.parametrize("levels,k,protect", [(0, 300, 64), (50, 300, 64), (7, 1000, 0), (0, 2936, 64),
                                              (0, 0, 16)])
def test_topk_largest_slots_exact(levels, k, protect):
    banner(f"topk slots levels={levels} k={k}")
    c = _topk_cache()
    c.n_slots[1, 2] = 2500  # ragged
    c.ctx_len[1, 2] = 2500
    c.pos_map[0, 1, 100:110] = -1
    scores = W.gen_scores(7, (2, 3, c.pos_map.shape[2]), levels=levels, tie_frac=0.05)
    ref = oracle.topk_largest(scores, c, k, protect=protect)
    dc = to_device(c, 12)
    idx = torch.full((2, 3, 3000), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    se.se_topk_select(dc, torch.from_numpy(scores).to(DEV), idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT,
                      k=k, protect=protect)
    got = lists_from(idx, cnt)
    for b in range(2):
        for g in range(3):
            assert got[b][g].tolist() == ref[b][g].tolist(), (b, g)


def test_topk_window_and_pages_and_smallest_exact():
    banner("topk window/pages/smallest")
    c = _topk_cache(N=2000)
    scores = W.gen_scores(8, (2, 3, 448), levels=100)
    ref = oracle.topk_largest(scores, c, 89, window=512, protect=64)
    dc = to_device(c, 12)
    idx = torch.zeros((2, 3, 160), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    se.se_topk_select(dc, torch.from_numpy(scores).to(DEV), idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT,
                      k=89, window=512, protect=64)
    assert [x.tolist() for r in lists_from(idx, cnt) for x in r] == [x.tolist() for r in ref for x in r]
    # pages with forced ends
    pscores = W.gen_scores(9, (2, 3, c.max_blocks), levels=30)
    ref = oracle.topk_largest(pscores, c, 40, unit="page", forced_ends=True)
    idx = torch.zeros((2, 3, 42), dtype=torch.int32, device=DEV)
    se.se_topk_select(dc, torch.from_numpy(pscores).to(DEV), idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_PAGE,
                      k=40, forced_ends=1)
    assert [x.tolist() for r in lists_from(idx, cnt) for x in r] == [x.tolist() for r in ref for x in r]
    # smallest with holes, ties and the recent window
    c2 = punch_holes(c, 0.001, 9)
    cum = W.gen_scores(10, (2, 3, c2.pos_map.shape[2]), levels=20)
    for budget in (1990, 1000, 5000):
        ref = oracle.topk_smallest(cum, c2, 3, budget=budget, recent=256)
        dc2 = to_device(c2, 12)
        idx = torch.zeros((2, 3, 3), dtype=torch.int32, device=DEV)
        se.se_topk_select(dc2, torch.from_numpy(cum).to(DEV), idx, cnt, mode=se.SE_TOPK_SMALLEST,
                          unit=se.SE_UNIT_SLOT, k=3, budget=budget, recent=256)
        assert [x.tolist() for r in lists_from(idx, cnt) for x in r] == [x.tolist() for r in ref for x in r]


@pytest.mark.parametrize("levels", [0, 3])
def test_topk_single_item_exact(levels):
    """k = 1 takes its own arg-max path: largest slots, pages with forced ends and smallest, with heavy ties."""
    banner(f"topk k=1 levels={levels}")
    c = punch_holes(_topk_cache(N=2000), 0.002, 11)
    dc = to_device(c, 12)
    cnt = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    scores = W.gen_scores(12, (2, 3, c.pos_map.shape[2]), levels=levels)
    for protect in (0, 64):
        ref = oracle.topk_largest(scores, c, 1, protect=protect)
        idx = torch.zeros((2, 3, 65), dtype=torch.int32, device=DEV)
        se.se_topk_select(dc, torch.from_numpy(scores).to(DEV), idx, cnt, mode=se.SE_TOPK_LARGEST,
                          unit=se.SE_UNIT_SLOT, k=1, protect=protect)
        assert [x.tolist() for r in lists_from(idx, cnt) for x in r] == [x.tolist() for r in ref for x in r]
    pscores = W.gen_scores(13, (2, 3, c.max_blocks), levels=levels)
    ref = oracle.topk_largest(pscores, c, 1, unit="page", forced_ends=True)
    idx = torch.zeros((2, 3, 3), dtype=torch.int32, device=DEV)
    se.se_topk_select(dc, torch.from_numpy(pscores).to(DEV), idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_PAGE,
                      k=1, forced_ends=1)
    assert [x.tolist() for r in lists_from(idx, cnt) for x in r] == [x.tolist() for r in ref for x in r]
    for budget in (1990, 1000):
        ref = oracle.topk_smallest(scores, c, 1, budget=budget, recent=256)
        idx = torch.zeros((2, 3, 1), dtype=torch.int32, device=DEV)
        se.se_topk_select(dc, torch.from_numpy(scores).to(DEV), idx, cnt, mode=se.SE_TOPK_SMALLEST,
                          unit=se.SE_UNIT_SLOT, k=1, budget=budget, recent=256)
        assert [x.tolist() for r in lists_from(idx, cnt) for x in r] == [x.tolist() for r in ref for x in r]


# ------------------------------------------------------------------ Token2Chunk -----------------------------------
def test_token2chunk_exact():
    banner("token2chunk")
    c = _topk_cache(B=4, G=2, N=1200)
    scores = W.gen_scores(11, (4, 2, 448), levels=64)  # coarse levels -> tied priorities
    cand = oracle.topk_largest(scores, c, 89, window=512, protect=64)
    for budget in (89, 102, 140, 400):
        ref = oracle.token2chunk(cand, scores, c, max_gap=8, budget=budget, window=512, protect=64)
        dc = to_device(c, 8)
        idx, cnt = W.pack_lists(cand, 160)
        out = torch.full((4, 2, 470), -1, dtype=torch.int32, device=DEV)
        ocnt = torch.zeros((4, 2), dtype=torch.int32, device=DEV)
        status = status_word()
        se.se_token2chunk(dc, i32(idx), i32(cnt), torch.from_numpy(scores).to(DEV), out, ocnt, max_gap=8,
                          budget=budget, window=512, protect=64, status=status)
        assert se.se_status_read(status) == 0
        got = lists_from(out, ocnt)
        for b in range(4):
            for g in range(2):
                assert got[b][g].tolist() == ref[b][g].tolist(), (budget, b, g)


# ------------------------------------------------------------------ compaction / append ---------------------------
@pytest.mark.parametrize("pattern", ["random", "prefix", "shift1", "tail"])
def test_compact_gather_whole_bit_exact(pattern):
    banner(f"compact whole {pattern}")
    inp = snap_inputs(B=3, N=1337, d=128)
    st = inp["cache"]
    counts = np.array([[200, 1000], [0, 64], [1300, 17]], np.int32)
    keep = W.gen_keep_sets(5, st.n_slots, counts, pattern=pattern)
    ref = oracle.compact_gather(st, keep)
    dc = to_device(st, 8)
    idx, cnt = W.pack_lists(keep, 1337)
    status = status_word()
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref)


def test_compact_gather_trailing_with_holes_and_cum():
    banner("compact trailing")
    cfg = W.H2O("t", B=2, hq=8, hkv=2, d=128, N=1100, budget=2000, recent=8, steps=1, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=2, threads=4)
    st = inp["cache"]
    st.cum_score[:] = np.random.default_rng(1).random(st.cum_score.shape).astype(np.float32)
    st = punch_holes(st, 0.004, 3)  # some holes inside and before the window
    lo = st.n_slots - 512
    keep = []
    for b in range(2):
        row = []
        for g in range(2):
            n = int(st.n_slots[b, g])
            res = [s for s in range(n - 512, n) if st.pos_map[b, g, s] >= 0]
            rs = np.random.default_rng(b * 2 + g)
            row.append(np.sort(rs.choice(res, size=166, replace=False)).astype(np.int32))
        keep.append(row)
    ref = oracle.compact_gather(st, keep, window=512)
    dc = to_device(st, 8)
    idx, cnt = W.pack_lists(keep, 170)
    status = status_word()
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, window=512, status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref)


def test_evict_append_sequence_bit_exact():
    banner("evict/append")
    cfg = W.H2O("t", B=3, hq=8, hkv=2, d=128, N=47, budget=100, recent=4, steps=40, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=4, threads=2)
    st = inp["cache"]
    ref = st.copy()
    dc = to_device(st, 8)
    status = status_word()
    rs = np.random.default_rng(8)
    for step in range(40):
        if step % 3 == 0:  # evict one or two resident slots per head
            ev = []
            for b in range(3):
                row = []
                for g in range(2):
                    res = np.where(ref.pos_map[b, g, :ref.n_slots[b, g]] >= 0)[0]
                    row.append(np.sort(rs.choice(res, size=1 + (b + g + step) % 2, replace=False)).astype(np.int32))
                ev.append(row)
            ref = oracle.evict_slots(ref, ev)
            idx, cnt = W.pack_lists(ev, 2)
            se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_EVICT_SLOTS, status=status)
        pos = np.full((3,), 47 + step, np.int32)
        ref, _ = oracle.cache_append(ref, inp["k_new"][step], inp["v_new"][step], pos)
        se.se_cache_append(dc, storage_tensor(inp["k_new"][step], "bf16"), storage_tensor(inp["v_new"][step], "bf16"),
                           i32(pos), status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref)


def test_append_capacity_is_all_or_nothing():
    banner("append capacity")
    c = W.empty_cache(2, 2, 128, 16, 4, 8, "bf16")
    W.layout_initial(c, 64)  # 4 blocks each: no spare block
    dc = to_device(c, 8)
    before = dc.to_numpy()
    status = status_word()
    z = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device=DEV)
    se.se_cache_append(dc, z, z, i32([64, 64]), status=status)
    assert se.se_status_read(status) & se.SE_DEV_CAPACITY
    after = dc.to_numpy()
    for f in before:
        np.testing.assert_array_equal(after[f], before[f])


def test_compact_rejects_bad_indices():
    banner("compact bad indices")
    inp = snap_inputs(B=1, N=300)
    dc = to_device(inp["cache"], 8)
    idx, cnt = W.pack_lists([[np.array([5, 3, 9], np.int32), np.array([1, 400], np.int32)]], 4)
    status = status_word()
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, status=status)
    assert se.se_status_read(status) & se.SE_DEV_INDEX


@pytest.mark.parametrize("stride", [4, 300])
def test_compact_rejects_a_free_slot_moved_through_the_hazard_list(stride):
    """Kept list [1, 3, 10, 11] of a unit: outputs 0 and 1 read slots 1 and 3 before those slots are overwritten,
    so with a list stride of 300 (the tiled path) output 3 (destination slot 3) is moved with the ordered hazard
    tiles; with a stride of 4 the whole unit is one read-then-write workgroup. Its source, slot 11, is a hole: the
    oracle rejects the list, and the device must flag an index error instead of copying the free slot."""
    banner(f"compact: free slot at a hazard destination, list stride {stride}")
    inp = snap_inputs(B=1, N=300)
    st = inp["cache"]
    st.pos_map[0, 0, 11] = -1
    st.ctx_len[0, 0] -= 1
    keep = [[np.array([1, 3, 10, 11], np.int32), np.array([1, 3, 10, 12], np.int32)]]
    with pytest.raises(IndexError):
        oracle.compact_gather(st, keep)
    dc = to_device(st, 8)
    idx, cnt = W.pack_lists(keep, stride)
    status = status_word()
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, status=status)
    assert se.se_status_read(status) & se.SE_DEV_INDEX


# ------------------------------------------------------------------ page bounds -----------------------------------
def test_page_bounds_build_exact_and_score():
    banner("page bounds")
    cfg = W.Quest("t", B=2, hq=8, hkv=2, d=128, N=2000, top_pages=16, shift_frac=0.05, shift=2.0)
    inp = W.gen_quest(cfg, seed=6, threads=4)
    st = punch_holes(inp["cache"], 0.003, 5)
    meta = oracle.page_bounds_build(st)
    dc = to_device(st, 8)
    se.se_page_bounds(dc, se.SE_PAGES_BUILD)
    got = dc.page_meta.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, meta)
    u = oracle.page_bounds_score(st, meta, inp["q_dec"])
    ps = torch.full((2, 2, st.max_blocks), 7.0, dtype=torch.float32, device=DEV)
    se.se_page_bounds(dc, se.SE_PAGES_SCORE, storage_tensor(inp["q_dec"], "bf16"), ps)
    n_pages = -(-2000 // 16)
    g = ps.cpu().numpy()[:, :, :n_pages]
    r = u[:, :, :n_pages]
    assert np.all(np.isfinite(r))
    np.testing.assert_allclose(g, r, rtol=1e-3, atol=0)


# ------------------------------------------------------------------ page metadata refresh -------------------------
def meta_bits(dc):
    return dc.page_meta.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("N", [32, 37, 1000])
def test_page_bounds_refresh_last_page_after_append(N):
    # N = 32: the append opens a page (a block is popped); 37 and 1000: it lands in the partly filled last page
    banner(f"refresh last page after append N={N}")
    cfg = W.H2O("t", B=3, hq=8, hkv=2, d=128, N=N, budget=N, recent=4, steps=1, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=7, threads=2)
    st = inp["cache"]
    st.page_meta = oracle.page_bounds_build(st)
    pos = np.full((3,), N, np.int32)
    ref, _ = oracle.cache_append(st, inp["k_new"][0], inp["v_new"][0], pos)
    want = oracle.page_bounds_build(ref)
    assert not np.array_equal(want, st.page_meta)
    dc = to_device(st, 8)
    status = status_word()
    se.se_cache_append(dc, storage_tensor(inp["k_new"][0], "bf16"), storage_tensor(inp["v_new"][0], "bf16"), i32(pos),
                       status=status)
    se.se_page_bounds_refresh(dc, se.SE_REFRESH_LAST_PAGE, status=status)
    assert se.se_status_read(status) == 0
    np.testing.assert_array_equal(meta_bits(dc), want)


@pytest.mark.parametrize("window", [0, 300])
def test_page_bounds_refresh_after_compaction_and_quest_over_evicted_cache(window):
    """Physical eviction, then logical selection on the evicted cache: the metadata of the compacted pages is
    refreshed, page scores and the page choice follow the oracle, and decode over every page equals dense decode
    over the retained slots."""
    banner(f"refresh after compaction, Quest over the evicted cache, window={window}")
    from types import SimpleNamespace
    from oracle import pipelines as P

    inp = snap_inputs(B=2, N=1337, seed=9)
    st = inp["cache"]
    st.page_meta = oracle.page_bounds_build(st)
    n = 1337
    w0 = n - window if window else 0  # w0 = 1037 is not page-aligned
    rs = np.random.default_rng(9)
    keep = [[np.sort(rs.choice(np.arange(w0, n), size=100 + 37 * (b + g), replace=False)).astype(np.int32)
             for g in range(2)] for b in range(2)]
    ref = oracle.compact_gather(st, keep, window=window)
    dc = to_device(st, 8)
    idx, cnt = W.pack_lists(keep, 200)
    status = status_word()
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, window=window, status=status)
    lo = np.full((2, 2), w0 // 16, np.int32)
    se.se_page_bounds_refresh(dc, se.SE_REFRESH_FROM_PAGE, i32(lo), status=status)
    assert se.se_status_read(status) == 0
    got, want = meta_bits(dc), oracle.page_bounds_build(ref)
    for b in range(2):
        for g in range(2):
            n_pages = -(-int(ref.n_slots[b, g]) // 16)
            np.testing.assert_array_equal(got[b, g, :n_pages], want[b, g, :n_pages])
            np.testing.assert_array_equal(got[b, g, n_pages:], st.page_meta[b, g, n_pages:])

    # Quest page selection and decode over the evicted cache
    top = 3
    qref = P.quest_step(dict(cfg=SimpleNamespace(top_pages=top), q_dec=inp["q_dec"], scale=inp["scale"]), ref)
    qs = WF.QuestStep(dc, top_pages=top, scale=inp["scale"], status=status)
    out = qs.run(storage_tensor(inp["q_dec"], "bf16")).cpu().numpy()
    assert se.se_status_read(status) == 0
    ps = qs.page_scores.cpu().numpy()
    sel = lists_from(qs.pages, qs.count)
    for b in range(2):
        for g in range(2):
            n_pages = -(-int(ref.n_slots[b, g]) // 16)
            np.testing.assert_allclose(ps[b, g, :n_pages], qref["page_scores"][b, g, :n_pages], rtol=1e-3, atol=0)
            if not assert_sets_match_modulo_ties(sel[b][g], qref["pages"][b][g], qref["page_scores"][b, g]):
                np.testing.assert_allclose(out[b, 4 * g:4 * g + 4], qref["out"][b, 4 * g:4 * g + 4], atol=2e-3, rtol=0)
    # every page selected: dense decode over the retained slots
    n_pages_max = int(-(-ref.n_slots.max() // 16))
    allp = [[np.arange(-(-int(ref.n_slots[b, g]) // 16), dtype=np.int32) for g in range(2)] for b in range(2)]
    sel_all, cnt_all = W.pack_lists(allp, n_pages_max)
    out_all = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out_all, scale=inp["scale"],
                             sel_pages=i32(sel_all), sel_count=i32(cnt_all), status=status)
    dense, _ = oracle.decode_attn(ref, inp["q_dec"], inp["scale"])
    assert se.se_status_read(status) == 0
    np.testing.assert_allclose(out_all.cpu().numpy(), dense, atol=2e-3, rtol=0)


# ------------------------------------------------------------------ range-restricted pruning ----------------------
@pytest.mark.parametrize("k", [0, 60, 5000])
def test_topk_range_pruning_and_parallel_slot_eviction_exact(k):
    """Kept and dropped lists for a position range with busy blocks equal the oracle's on the same fp32 scores
    (coarse values: many ties), and evicting the dropped slots gives the oracle's cache state bit for bit."""
    banner(f"range pruning k={k}")
    inp = snap_inputs(B=2, N=1500, seed=11)
    st = punch_holes(inp["cache"], 0.004, 6)
    stack = np.full((2, 2, 1500), -1, np.int32)  # room for every eviction
    stack[:, :, :st.slot_stack.shape[2]] = st.slot_stack
    st.slot_stack = stack
    rs = np.random.default_rng(12)
    refs = (rs.random(st.num_blocks) < 0.25).astype(np.int32)
    scores = (rs.random((2, 2, st.pos_map.shape[2])) * 50).round().astype(np.float32)
    lo, hi = 200, 1300
    kept = oracle.topk_largest(scores, st, k, prune_range=(lo, hi), block_refs=refs)
    dropped = oracle.topk_largest(scores, st, k, prune_range=(lo, hi), block_refs=refs, emit="dropped")
    dc = to_device(st, 8)
    status = status_word()
    sc = torch.from_numpy(scores).to(DEV)
    stride = st.pos_map.shape[2]
    idx = torch.full((2, 2, stride), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros((2, 2), dtype=torch.int32, device=DEV)
    refs_d = i32(refs)
    se.se_topk_select(dc, sc, idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT, k=k, prune_range=(lo, hi),
                      block_refs=refs_d, status=status)
    got = lists_from(idx, cnt)
    for b in range(2):
        for g in range(2):
            assert got[b][g].tolist() == kept[b][g].tolist()
    se.se_topk_select(dc, sc, idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT, k=k, prune_range=(lo, hi),
                      block_refs=refs_d, emit_dropped=True, status=status)
    got = lists_from(idx, cnt)
    for b in range(2):
        for g in range(2):
            assert got[b][g].tolist() == dropped[b][g].tolist()
    se.se_compact_evict(dc, idx, cnt, mode=se.SE_COMPACT_EVICT_SLOTS, status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), oracle.evict_slots(st, dropped))


def test_topk_range_pruning_inside_a_window_exact():
    # items are the last 600 slots (scores indexed from the window's first slot): busy pages are looked up
    # relative to the window's first page
    banner("range pruning inside a window")
    inp = snap_inputs(B=2, N=5000, seed=15)
    st = inp["cache"]
    rs = np.random.default_rng(16)
    refs = (rs.random(st.num_blocks) < 0.3).astype(np.int32)
    W_ = 600
    scores = (rs.random((2, 2, W_)) * 20).round().astype(np.float32)
    lo, hi, k = 4500, 4950, 90
    want = oracle.topk_largest(scores, st, k, window=W_, prune_range=(lo, hi), block_refs=refs)
    dc = to_device(st, 8)
    status = status_word()
    idx = torch.full((2, 2, W_), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros((2, 2), dtype=torch.int32, device=DEV)
    se.se_topk_select(dc, torch.from_numpy(scores).to(DEV), idx, cnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT,
                      k=k, window=W_, prune_range=(lo, hi), block_refs=i32(refs), status=status)
    assert se.se_status_read(status) == 0
    got = lists_from(idx, cnt)
    for b in range(2):
        for g in range(2):
            assert got[b][g].tolist() == want[b][g].tolist()


def test_slot_eviction_reports_bad_entries_and_capacity():
    banner("slot eviction errors")
    inp = snap_inputs(B=1, N=300)
    st = punch_holes(inp["cache"], 0.01, 2)  # fills part of the slot stacks
    dc = to_device(st, 8)
    status = status_word()
    idx, cnt = W.pack_lists([[np.array([7, 5, 9], np.int32), np.array([2], np.int32)]], 4)  # out of order
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_EVICT_SLOTS, status=status)
    assert se.se_status_read(status) & se.SE_DEV_INDEX
    free = [s for s in range(300) if st.pos_map[0, 0, s] >= 0 and s not in (7, 9)][:20]
    idx, cnt = W.pack_lists([[np.array(free, np.int32), np.array([], np.int32)]], 20)
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_EVICT_SLOTS, status=status)
    assert se.se_status_read(status) & se.SE_DEV_CAPACITY
    d = dc.to_numpy()
    cap = st.slot_stack.shape[2]
    assert d["slot_top"][0, 0] == cap  # filled to capacity, nothing beyond
    assert (d["pos_map"][0, 0, :300] < 0).sum() == cap and d["ctx_len"][0, 0] == 300 - cap


# ------------------------------------------------------------------ accumulating window scores --------------------
@pytest.mark.parametrize("dtype,d,wq,N", [("bf16", 128, 64, 1300), ("bf16", 128, 128, 900), ("f32", 64, 32, 700)])
def test_window_score_accumulates_into_existing_scores(dtype, d, wq, N):
    # wq = 128 at group size 4: 512 query rows, so rows are split over workgroups and summed by the reduction
    banner(f"accumulating window scores {dtype} wq={wq} N={N}")
    inp = snap_inputs(d=d, dtype=dtype, N=N, wq=wq, protect=8, keep=16)
    st = punch_holes(inp["cache"], 0.01, 3)
    ora = oracle.window_score_causal(st, inp["q_win"], inp["q_pos"], inp["scale"])
    dc = to_device(st, 8)
    S = st.pos_map.shape[2]
    init = np.random.default_rng(7).random((2, 2, S)).astype(np.float32)
    scores = torch.from_numpy(init.copy()).to(DEV)
    status = status_word()
    se.se_window_score(dc, storage_tensor(inp["q_win"], dtype), i32(inp["q_pos"]), scores, scale=inp["scale"],
                       mode=se.SE_SCORE_CAUSAL, n_query=wq, accumulate=True, status=status)
    assert se.se_status_read(status) == 0
    got = scores.cpu().numpy().astype(np.float64) - init
    mass = np.full((2, 2), 4.0 * wq)
    for b in range(2):
        tol = 1e-3 * np.abs(ora[b, :, :N]) + 1e-6 * mass[b][:, None] + 2e-7  # + the fp32 add to init < 1
        assert np.all(np.abs(got[b, :, :N] - ora[b, :, :N]) <= tol)
    np.testing.assert_array_equal(scores.cpu().numpy()[:, :, N:], init[:, :, N:])  # past n_slots: untouched


# ------------------------------------------------------------------ chunk append ----------------------------------
@pytest.mark.parametrize("N,T,dtype,d", [(47, 512, "bf16", 128), (64, 37, "bf16", 128), (100, 1, "bf16", 128),
                                         (30, 70, "f32", 64)])
def test_chunk_append_bit_exact(N, T, dtype, d):
    banner(f"chunk append N={N} T={T} {dtype}")
    cfg = W.H2O("t", B=3, hq=8, hkv=2, d=d, N=N, budget=N + T, recent=4, steps=T, zipf=1.1, dtype=dtype)
    inp = W.gen_h2o(cfg, seed=8, threads=2)
    st = punch_holes(inp["cache"], 0.02, 4)  # freed slots stay on the stacks: a chunk goes to the high-water mark
    kc = np.ascontiguousarray(inp["k_new"].transpose(1, 2, 0, 3))
    vc = np.ascontiguousarray(inp["v_new"].transpose(1, 2, 0, 3))
    pos0 = np.full((3,), N, np.int32)
    ref = oracle.cache_append_chunk(st, kc, vc, pos0)
    dc = to_device(st, 8)
    status = status_word()
    se.se_cache_append_chunk(dc, storage_tensor(kc, dtype), storage_tensor(vc, dtype), i32(pos0), status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref)


def test_chunk_append_is_all_or_nothing():
    banner("chunk append capacity")
    cfg = W.H2O("t", B=2, hq=8, hkv=2, d=128, N=40, budget=100, recent=4, steps=60, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=9, threads=2)
    st = inp["cache"]
    st.free_top[0] = 1  # each sequence needs more than one new block
    before = st.copy()
    kc = np.ascontiguousarray(inp["k_new"].transpose(1, 2, 0, 3))
    dc = to_device(st, 8)
    status = status_word()
    se.se_cache_append_chunk(dc, storage_tensor(kc, "bf16"), storage_tensor(kc, "bf16"),
                             i32(np.full((2,), 40, np.int32)), status=status)
    assert se.se_status_read(status) & se.SE_DEV_CAPACITY
    compare_cache(dc.to_numpy(), before)


def test_chunk_append_after_compaction_with_unequal_heads():
    # after a whole-cache gather the heads of a sequence hold different slot counts: the chunk's blocks follow the
    # longest head, the shorter heads' new slots fall in allocated blocks
    banner("chunk append after compaction, unequal heads")
    cfg = W.H2O("t", B=2, hq=8, hkv=2, d=128, N=300, budget=600, recent=4, steps=100, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=10, threads=2)
    st = inp["cache"]
    counts = np.array([[40, 290], [150, 7]], np.int32)
    keep = W.gen_keep_sets(3, st.n_slots, counts, pattern="random")
    ref = oracle.compact_gather(st, keep)
    dc = to_device(st, 8)
    idx, cnt = W.pack_lists(keep, 300)
    status = status_word()
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, status=status)
    kc = np.ascontiguousarray(inp["k_new"].transpose(1, 2, 0, 3))
    vc = np.ascontiguousarray(inp["v_new"].transpose(1, 2, 0, 3))
    pos0 = np.full((2,), 300, np.int32)
    ref = oracle.cache_append_chunk(ref, kc, vc, pos0)
    se.se_cache_append_chunk(dc, storage_tensor(kc, "bf16"), storage_tensor(vc, "bf16"), i32(pos0), status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref)
