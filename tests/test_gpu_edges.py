"""Degenerate inputs through every call: a sequence emptied by compaction (an empty view), then given one token, and
a bidirectional window longer than a sequence's cache. Oracle parity at the stages' bars (lists, maps and caches
bit-exact; scores 1e-3 relative; decode outputs 2e-3 absolute), error bits where the calls define them, and no
writes outside the entries a call defines."""
import numpy as np
import pytest
import torch

import oracle
import sparse_decode_attention_se_amd as se
import workloads as W
from gpu_util import DEV, assert_scores_close, compare_cache, i32, lists_from, status_word, storage_tensor, to_device

pytestmark = pytest.mark.gpu
SENTINEL = 7.0


def banner(name):
    print(f"\n[case] {name}", flush=True)


def test_emptied_sequence_through_every_call():
    banner("a sequence emptied by compaction: decode, causal scores, top-K, append, bidirectional window, "
           "Token2Chunk")
    cfg = W.SnapKV("t", B=3, hq=8, hkv=2, d=128, N=300, wq=16, protect=8, keep=40, dtype="bf16", spike_frac=0.04)
    inp = W.gen_snapkv(cfg, seed=21, threads=3)
    st = inp["cache"]
    r = cfg.hq // cfg.hkv

    # compaction: sequence 1 keeps nothing (both heads), the others keep ragged sets, one of them everything
    counts = np.array([[37, 120], [0, 0], [300, 50]], np.int32)
    keep = W.gen_keep_sets(22, st.n_slots, counts)
    ref = oracle.compact_gather(st, keep)
    assert (ref.n_slots[1] == 0).all() and (ref.ctx_len[1] == 0).all()
    dc = to_device(st, cfg.hq)
    status = status_word()
    idx, cnt = W.pack_lists(keep, 300)
    se.se_compact_evict(dc, i32(idx), i32(cnt), mode=se.SE_COMPACT_GATHER, status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref)

    # decode over every slot: the empty view gives 0
    out = torch.full((3, cfg.hq, 128), SENTINEL, dtype=torch.float32, device=DEV)
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], status=status)
    assert se.se_status_read(status) == 0
    o_ref, _ = oracle.decode_attn(ref, inp["q_dec"], inp["scale"])
    got = out.cpu().numpy()
    assert np.all(got[1] == 0.0)
    np.testing.assert_allclose(got, o_ref, atol=2e-3, rtol=0)

    # causal window scores: slots below n_slots only, nothing written past them (the empty unit: nothing at all)
    S = ref.pos_map.shape[2]
    scores = torch.full((3, 2, S), SENTINEL, dtype=torch.float32, device=DEV)
    se.se_window_score(dc, storage_tensor(inp["q_win"], "bf16"), i32(inp["q_pos"]), scores, scale=inp["scale"],
                       mode=se.SE_SCORE_CAUSAL, n_query=cfg.wq, status=status)
    assert se.se_status_read(status) == 0
    s_ref = oracle.window_score_causal(ref, inp["q_win"], inp["q_pos"], inp["scale"])
    got = scores.cpu().numpy()
    for b in range(3):
        for g in range(2):
            n = int(ref.n_slots[b, g])
            assert_scores_close(got[b, g, :n][None], s_ref[b, g, :n][None], mass=np.array([r * cfg.wq], np.float64))
            assert np.all(got[b, g, n:] == SENTINEL), (b, g)

    # top-K over the scores of the compacted cache: the empty unit returns nothing
    s32 = s_ref.astype(np.float32)
    t_ref = oracle.topk_largest(s32, ref, 10, protect=4)
    tidx = torch.full((3, 2, 64), -7, dtype=torch.int32, device=DEV)
    tcnt = torch.full((3, 2), -7, dtype=torch.int32, device=DEV)
    se.se_topk_select(dc, torch.from_numpy(s32).to(DEV), tidx, tcnt, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT,
                      k=10, protect=4, status=status)
    assert se.se_status_read(status) == 0
    t_got = lists_from(tidx, tcnt)
    assert (tcnt.cpu().numpy()[1] == 0).all()
    for b in range(3):
        for g in range(2):
            assert t_got[b][g].tolist() == t_ref[b][g].tolist(), (b, g)

    # one appended token per sequence: the emptied one takes slot 0 (in a block from the free stack)
    rs = np.random.default_rng(23)
    k_new = W.to_storage(rs.standard_normal((3, 2, 128)), "bf16")
    v_new = W.to_storage(rs.standard_normal((3, 2, 128)), "bf16")
    pos = np.full((3,), 300, np.int32)
    ref2, _ = oracle.cache_append(ref, k_new, v_new, pos)
    se.se_cache_append(dc, storage_tensor(k_new, "bf16"), storage_tensor(v_new, "bf16"), i32(pos), status=status)
    assert se.se_status_read(status) == 0
    compare_cache(dc.to_numpy(), ref2)
    assert (ref2.n_slots[1] == 1).all()
    se.se_sparse_decode_attn(dc, storage_tensor(inp["q_dec"], "bf16"), out, scale=inp["scale"], status=status)
    assert se.se_status_read(status) == 0
    o_ref2, _ = oracle.decode_attn(ref2, inp["q_dec"], inp["scale"])
    np.testing.assert_allclose(out.cpu().numpy(), o_ref2, atol=2e-3, rtol=0)

    # a bidirectional window of 32 slots (8 protected): sequence 1 holds one slot, an index error that leaves its
    # scores unwritten; the other sequences are scored as the oracle scores them alone
    window, protect = 32, 8
    R = window - protect
    qw = W.to_storage(rs.standard_normal((3, cfg.hq, window, 128)), "bf16")
    bscores = torch.full((3, 2, R), SENTINEL, dtype=torch.float32, device=DEV)
    bstatus = status_word()
    se.se_window_score(dc, storage_tensor(qw, "bf16"), None, bscores, scale=inp["scale"], mode=se.SE_SCORE_BIDIR,
                       n_query=window, window=window, protect=protect, status=bstatus)
    assert se.se_status_read(bstatus) == se.SE_DEV_INDEX
    got = bscores.cpu().numpy()
    assert np.all(got[1] == SENTINEL)
    with pytest.raises(ValueError):
        oracle.window_score_bidir(ref2, qw, inp["scale"], window, protect)
    for b in (0, 2):
        sub = oracle.sequence_range(ref2, b, b + 1)
        b_ref = oracle.window_score_bidir(sub, qw[b:b + 1], inp["scale"], window, protect)
        assert_scores_close(got[b:b + 1], b_ref, mass=np.full((1, 2), r * window, np.float64))

    # Token2Chunk of an empty candidate list (sequence 0, head 0) is empty; the other lists as the oracle fills them
    b_scores = np.zeros((3, 2, R), np.float32)
    b_scores[[0, 2]] = got[[0, 2]]
    cand = [[np.zeros(0, np.int32), np.array([int(ref2.n_slots[0, 1]) - window + j for j in (1, 4, 9)], np.int32)],
            [np.zeros(0, np.int32), np.zeros(0, np.int32)],
            [np.array([int(ref2.n_slots[2, 0]) - window + j for j in (0, 2, 3, 12)], np.int32),
             np.array([int(ref2.n_slots[2, 1]) - window + j for j in (5, 6)], np.int32)]]
    sub02 = [oracle.sequence_range(ref2, b, b + 1) for b in (0, 2)]
    want = {b: oracle.token2chunk([cand[b]], b_scores[b:b + 1], sub02[i], max_gap=8, budget=10, window=window,
                                  protect=protect)[0] for i, b in enumerate((0, 2))}
    cidx, ccnt = W.pack_lists(cand, 8)
    kout = torch.full((3, 2, 40), -7, dtype=torch.int32, device=DEV)
    kcnt = torch.full((3, 2), -7, dtype=torch.int32, device=DEV)
    tstatus = status_word()
    se.se_token2chunk(dc, i32(cidx), i32(ccnt), torch.from_numpy(b_scores).to(DEV), kout, kcnt, max_gap=8,
                      budget=10, window=window, protect=protect, status=tstatus)
    # sequence 1's window is longer than its cache: an index error and no list; the others are filled
    assert se.se_status_read(tstatus) == se.SE_DEV_INDEX
    k_got = lists_from(kout, kcnt)
    assert (kcnt.cpu().numpy()[1] == 0).all()
    assert k_got[0][0].tolist() == []
    for b in (0, 2):
        for g in range(2):
            assert k_got[b][g].tolist() == want[b][g].tolist(), (b, g)
