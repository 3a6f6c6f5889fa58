"""The C-ABI library loads and exports every entry point include/se.h declares; host-side validation answers
without touching a device (no compute calls here)."""
import ctypes as C
import os
import re

import pytest

from sparse_decode_attention_se_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "se.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(se_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_symbols()
    assert len(names) >= 14
    for name in names:
        assert hasattr(lib, name), name
    # the binding declares the same set
    assert set(names) == set(_lib.EXPORTS)


def test_python_binding_names_match_c():
    import sparse_decode_attention_se_amd as se

    for name in ("se_window_score", "se_topk_select", "se_token2chunk", "se_compact_evict", "se_cache_append",
                 "se_page_bounds", "se_sparse_decode_attn", "se_status_read", "se_version"):
        assert callable(getattr(se, name))


def test_host_validation_without_device():
    lib = _lib.load()
    assert lib.se_version().decode().startswith("libse")
    assert lib.se_error_string(_lib.SE_ERR_NULL)
    assert lib.se_error_string(_lib.SE_DEV_INDEX).startswith(b"device")
    # null descriptor / params: rejected before any HIP call
    assert lib.se_window_score(None, None, None, None, None, None, None, 0, None) == _lib.SE_ERR_NULL
    assert lib.se_sparse_decode_attn(None, None, None, None, None, None, None, None, 0, None) == _lib.SE_ERR_NULL
    c = _lib.se_cache_t()
    c.k_pool = c.v_pool = c.block_table = c.pos_map = c.ctx_len = c.n_slots = 16  # fake non-null, never touched
    c.B, c.n_kv, c.n_q, c.d, c.page, c.num_blocks, c.max_blocks, c.dtype = 1, 2, 3, 128, 16, 4, 4, 1
    p = _lib.se_decode_params_t(0.1, 0, 0, 0, 0)
    # n_q not a multiple of n_kv
    assert lib.se_sparse_decode_attn(C.byref(c), 16, None, None, C.byref(p), 16, None, None, 0, None) == \
        _lib.SE_ERR_SHAPE
    c.n_q = 8
    c.d = 96  # unsupported head dim
    assert lib.se_sparse_decode_attn(C.byref(c), 16, None, None, C.byref(p), 16, None, None, 0, None) == \
        _lib.SE_ERR_DTYPE
    c.d = 128
    # workspace missing
    assert lib.se_sparse_decode_attn(C.byref(c), 16, None, None, C.byref(p), 16, None, None, 0, None) == \
        _lib.SE_ERR_WORKSPACE
    tp = _lib.se_topk_params_t(0, 0, -1, 0, 0, 0, 0, 0, 64, 64)
    assert lib.se_topk_select(C.byref(c), 16, C.byref(tp), 16, 16, None, None, 0, None) == _lib.SE_ERR_PARAM
    wp = _lib.se_window_params_t(0.1, 1, 512, 512, 600, 512)  # protect > window
    assert lib.se_window_score(C.byref(c), 16, None, C.byref(wp), 16, None, None, 0, None) == _lib.SE_ERR_PARAM
    cp = _lib.se_compact_params_t(7, 0, 8)  # unknown mode
    c.free_blocks = c.free_top = 16
    assert lib.se_compact_evict(C.byref(c), 16, 16, C.byref(cp), None, None, 0, None) == _lib.SE_ERR_PARAM
    cp = _lib.se_compact_params_t(0, 0, 8)  # GATHER needs its small workspace
    assert lib.se_compact_evict(C.byref(c), 16, 16, C.byref(cp), None, None, 0, None) == _lib.SE_ERR_WORKSPACE
    # H2O's fused step: needs the cumulative scores and a slot stack, and non-negative budget and recent
    hp = _lib.se_h2o_params_t(0.1, 8, 4)
    assert lib.se_h2o_decode_evict(C.byref(c), 16, C.byref(hp), 16, 16, 16, None, None, 0, None) == _lib.SE_ERR_NULL
    c.cum_score = c.slot_stack = c.slot_top = 16
    c.slot_cap = 4
    assert lib.se_h2o_decode_evict(C.byref(c), 16, C.byref(hp), 16, None, 16, None, None, 0, None) == _lib.SE_ERR_NULL
    hp = _lib.se_h2o_params_t(0.1, -1, 4)
    assert lib.se_h2o_decode_evict(C.byref(c), 16, C.byref(hp), 16, 16, 16, None, None, 0, None) == _lib.SE_ERR_PARAM
    # 64 slots per unit fit one workgroup's LDS: the fused path needs no workspace
    hp = _lib.se_h2o_params_t(0.1, 8, 4)
    assert lib.se_h2o_decode_evict_workspace_size(C.byref(c), C.byref(hp)) == 0


def test_workspace_sizes_are_host_only():
    lib = _lib.load()
    c = _lib.se_cache_t()
    c.k_pool = c.v_pool = c.block_table = c.pos_map = c.ctx_len = c.n_slots = 16
    c.B, c.n_kv, c.n_q, c.d, c.page, c.num_blocks, c.max_blocks, c.dtype = 8, 8, 32, 128, 16, 16384, 2048, 1
    p = _lib.se_decode_params_t(0.1, 0, 0, 2048, 0)  # split-K partials
    assert lib.se_sparse_decode_attn_workspace_size(C.byref(c), C.byref(p), 0) > 0
    p = _lib.se_decode_params_t(0.1, 0, 0, 2048, 1)  # accumulating, logits fit in LDS: no workspace
    assert lib.se_sparse_decode_attn_workspace_size(C.byref(c), C.byref(p), 0) == 0
    p = _lib.se_decode_params_t(0.1, 0, 0, 0, 1)  # accumulating over 32768 slots: partials and logits
    assert lib.se_sparse_decode_attn_workspace_size(C.byref(c), C.byref(p), 0) > 8 * 8 * 32768 * 4 * 4
    wp = _lib.se_window_params_t(0.1, 0, 64, 0, 0, 32768)
    assert lib.se_window_score_workspace_size(C.byref(c), C.byref(wp)) > 0
    cp = _lib.se_compact_params_t(0, 0, 2048)
    assert lib.se_compact_evict_workspace_size(C.byref(c), C.byref(cp)) >= (2 * 8 + 1) * 4
    cp = _lib.se_compact_params_t(1, 0, 1)
    assert lib.se_compact_evict_workspace_size(C.byref(c), C.byref(cp)) == 0


def test_compression_loop_schedule_and_sequence_views_on_host():
    # host logic only: the workflow's schedule against the oracle's, and a sequence view's tensors are the rows
    # of the whole cache's (no copy), with the pool and free stack shared
    import workloads as W
    from oracle import pipelines as P
    import sparse_decode_attention_se_amd as se
    from sparse_decode_attention_se_amd import workflows as WF

    cfg = W.scaled(W.C2, B=12, hq=4, hkv=2, d=16, N=200, window=32, protect=4, period=8, dtype="f32", page=4)
    inp = W.gen_kara(cfg, seed=1, threads=1)
    dc = se.DeviceCache.from_arrays(cfg.hq, cfg.dtype, "cpu", **{f: getattr(inp["cache"], f)
                                                                 for f in se.DeviceCache.FIELDS
                                                                 if getattr(inp["cache"], f) is not None})
    for policy in ("periodic", "threshold"):
        loop = WF.CompressionLoop(dc, policy=policy, period=cfg.period, window=cfg.window, protect=cfg.protect,
                                  n_cand=cfg.n_cand, budget=cfg.budget, max_gap=cfg.max_gap, scale=inp["scale"])
        for t in range(3 * cfg.period):
            assert loop.due(t) == P.runs_of(P.policy_due(policy, t, cfg.B, cfg.period))
    with pytest.raises(ValueError):
        WF.CompressionLoop(dc, policy="sometimes", period=8, window=32, protect=4, n_cand=5, budget=6, max_gap=2,
                           scale=1.0)
    v = dc.seq_view(3, 7)
    for f in se.DeviceCache.FIELDS:
        x, y = getattr(dc, f), getattr(v, f)
        if x is None:
            assert y is None
        elif f in se.DeviceCache.SHARED:
            assert y is x
        else:
            assert y.shape[0] == 4 and y.data_ptr() == x[3].data_ptr() and y.is_contiguous()
    c = v.desc()
    assert c.B == 4 and c.block_table == dc.block_table[3].data_ptr() and c.k_pool == dc.k_pool.data_ptr()
    for bad in ((0, 0), (-1, 2), (5, 13)):
        with pytest.raises(ValueError):
            dc.seq_view(*bad)


def test_binding_rejects_bad_operands_before_the_library():
    # the kernels index operands by the cache's sizes: a short, mistyped or strided tensor is refused on the host
    import torch

    import sparse_decode_attention_se_amd as se
    import workloads as W

    cfg = W.scaled(W.C2, B=3, hq=4, hkv=2, d=16, N=64, window=32, protect=4, period=4, dtype="f32", page=4)
    inp = W.gen_kara(cfg, seed=1, threads=1)
    dc = se.DeviceCache.from_arrays(cfg.hq, cfg.dtype, "cpu", **{f: getattr(inp["cache"], f)
                                                                 for f in se.DeviceCache.FIELDS
                                                                 if getattr(inp["cache"], f) is not None})
    k = torch.zeros((3, 2, 16), dtype=torch.float32)
    pos = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="k_new holds"):
        se.se_cache_append(dc, k[:2], k, pos)
    with pytest.raises(TypeError, match="dtype"):
        se.se_cache_append(dc, k, k, pos.long())
    with pytest.raises(ValueError, match="contiguous"):
        se.se_cache_append(dc, k.transpose(0, 1), k, pos)
    with pytest.raises(ValueError, match="required"):
        se.se_cache_append(dc, k, None, pos)
    q = torch.zeros((3, 4, 16), dtype=torch.float32)
    with pytest.raises(ValueError, match="out holds"):
        se.se_sparse_decode_attn(dc, q, torch.zeros((3, 4, 8)), scale=0.25)
    scores = torch.zeros((3, 2, 28), dtype=torch.float32)
    with pytest.raises(ValueError, match="q_win holds"):
        se.se_window_score(dc, torch.zeros((3, 4, 31, 16)), None, scores, scale=0.25, mode=se.SE_SCORE_BIDIR,
                           n_query=32, window=32, protect=4)
    with pytest.raises(ValueError, match="count holds"):
        se.se_topk_select(dc, scores, torch.zeros((3, 2, 28), dtype=torch.int32), torch.zeros((3, 1), dtype=torch.int32),
                          mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT, k=4, window=32, protect=4)
