"""The allocation-free decode entry point (se_sparse_decode_attn_noalloc) against se_sparse_decode_attn.

Both run the same kernels; the first keeps its scratch in the library's static per-GPU array instead of a caller
workspace, so their outputs must agree bit for bit: on two calls in a row, the second with a smaller input, on a
page selection with accumulated scores (the logits path of the scratch), and on an accumulating call that needs no
scratch at all. A call whose scratch would exceed the array is refused on the host, before anything is launched.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import sparse_decode_attention_se_amd as se
import workloads as W
from gpu_util import DEV, i32, status_word, storage_tensor, to_device

pytestmark = pytest.mark.gpu


def banner(name):
    print(f"\n[case] {name}", flush=True)


def pages_of(n_slots, top, seed):
    """A seeded ascending page selection of `top` pages per unit (first and last page included)."""
    rs = np.random.default_rng(seed)
    B, G = n_slots.shape
    n_pages = -(-n_slots // 16)
    sel = np.zeros((B, G, top), np.int32)
    cnt = np.zeros((B, G), np.int32)
    for b in range(B):
        for g in range(G):
            p = n_pages[b, g]
            mid = rs.choice(np.arange(1, p - 1), size=top - 2, replace=False)
            row = np.sort(np.concatenate([[0, p - 1], mid])).astype(np.int32)
            sel[b, g, :row.size] = row
            cnt[b, g] = row.size
    return sel, cnt


def both(dc, q, scale, **kw):
    """(output of the workspace entry point, output of the allocation-free one) on the same inputs."""
    B, Hq, d = q.shape
    want = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    got = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    status = status_word()
    se.se_sparse_decode_attn(dc, q, want, scale=scale, status=status, **kw)
    se.se_sparse_decode_attn_noalloc(dc, q, got, scale=scale, status=status, **kw)
    assert se.se_status_read(status) == 0
    return want, got


def test_noalloc_decode_matches_the_workspace_entry_point_on_two_calls_in_a_row():
    banner("no-alloc decode: 8 x 16000 all slots, then 2 x 3000 over 40 pages")
    cfg = W.SnapKV("noalloc-a", B=8, hq=32, hkv=8, d=128, N=16000, wq=1, protect=0, keep=0, dtype="bf16")
    inp = W.gen_snapkv(cfg, seed=31, threads=8)
    dc = to_device(inp["cache"], cfg.hq)
    q = storage_tensor(inp["q_dec"], "bf16")
    p = se._lib.se_decode_params_t(inp["scale"], 0, 0, 0, 0)
    need = se._lib.load().se_sparse_decode_attn_workspace_size(C.byref(dc.desc()), C.byref(p), 0)
    assert 0 < need <= se.SE_NOALLOC_SCRATCH_BYTES  # this call uses the scratch array
    want, got = both(dc, q, inp["scale"])
    assert torch.equal(want, got)
    del dc
    cfg = W.SnapKV("noalloc-b", B=2, hq=32, hkv=8, d=128, N=3000, wq=1, protect=0, keep=0, dtype="bf16")
    inp = W.gen_snapkv(cfg, seed=32, threads=4)
    dc = to_device(inp["cache"], cfg.hq)
    sel, cnt = pages_of(inp["cache"].n_slots, 40, 33)
    want, got = both(dc, storage_tensor(inp["q_dec"], "bf16"), inp["scale"], sel_pages=i32(sel), sel_count=i32(cnt))
    assert torch.equal(want, got)


def test_noalloc_accumulating_decode_matches_with_and_without_scratch():
    banner("no-alloc decode with cumulative scores: page selection (logits in scratch), all slots (none)")
    cfg = W.H2O("noalloc-h2o", B=4, hq=32, hkv=8, d=128, N=2000, budget=2000, recent=16, steps=1, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=34, threads=4)
    st = inp["cache"]
    st.cum_score[:] = np.random.default_rng(35).random(st.cum_score.shape).astype(np.float32)
    q = storage_tensor(inp["q_steps"][0], "bf16")
    sel, cnt = pages_of(st.n_slots, 30, 36)
    for kw in (dict(sel_pages=i32(sel), sel_count=i32(cnt)), {}):
        a, b = to_device(st, cfg.hq), to_device(st, cfg.hq)
        want = torch.empty((cfg.B, cfg.hq, cfg.d), dtype=torch.float32, device=DEV)
        got = torch.empty_like(want)
        status = status_word()
        se.se_sparse_decode_attn(a, q, want, scale=inp["scale"], accumulate=True, status=status, **kw)
        se.se_sparse_decode_attn_noalloc(b, q, got, scale=inp["scale"], accumulate=True, status=status, **kw)
        assert se.se_status_read(status) == 0
        assert torch.equal(want, got)
        assert torch.equal(a.cum_score, b.cum_score)


def test_noalloc_refuses_a_call_beyond_its_scratch_before_launching():
    banner("no-alloc decode: 128 x 8 units over 32768-slot views need more than the scratch array")
    B, G, mb = 128, 8, 2048
    dc = se.DeviceCache(
        32, k_pool=torch.zeros((4, G, 16, 128), dtype=torch.bfloat16, device=DEV),
        v_pool=torch.zeros((4, G, 16, 128), dtype=torch.bfloat16, device=DEV),
        block_table=torch.full((B, mb), -1, dtype=torch.int32, device=DEV),
        pos_map=torch.full((B, G, mb * 16), -1, dtype=torch.int32, device=DEV),
        ctx_len=torch.zeros((B, G), dtype=torch.int32, device=DEV),
        n_slots=torch.zeros((B, G), dtype=torch.int32, device=DEV),
        free_blocks=torch.arange(4, dtype=torch.int32, device=DEV), free_top=i32([4]),
        slot_stack=torch.zeros((B, G, 1), dtype=torch.int32, device=DEV),
        slot_top=torch.zeros((B, G), dtype=torch.int32, device=DEV))
    p = se._lib.se_decode_params_t(0.1, 0, 0, 0, 0)
    assert se._lib.load().se_sparse_decode_attn_workspace_size(C.byref(dc.desc()), C.byref(p), 0) > \
        se.SE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, 32, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, 32, 128), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(se.SEError) as e:
        se.se_sparse_decode_attn_noalloc(dc, q, out, scale=0.1)
    assert e.value.code == se.SE_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing ran
