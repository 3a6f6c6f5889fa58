"""H2O's fused decode step (se_h2o_decode_evict: accumulating decode, bottom-1 and slot eviction in one call)
against the same step made as three calls (se_sparse_decode_attn, se_topk_select, se_compact_evict): outputs,
evicted slots and every cache field bit for bit after every step, on the single-workgroup path (the choice made
inside the decode's workgroup) and on a view too long for it (the three calls made in turn), with exactly tied
cumulative scores broken by position, and with budgets that evict and that do not."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import i32, status_word, storage_tensor, to_device
from sparse_decode_attention_se_amd import workflows as WF

import sparse_decode_attention_se_amd as se

pytestmark = pytest.mark.gpu


def banner(name):
    print(f"\n[case] {name}", flush=True)


def _tied(inp, b, g, slots):
    """Give slots of (b, g) one key (slot slots[0]'s) and one cumulative score, so their scores stay exactly tied."""
    st = inp["cache"]
    page = st.page

    def at(s):
        return st.block_table[b, s // page], g, s % page

    k0 = st.k_pool[at(slots[0])].copy()
    for s in slots:
        st.k_pool[at(s)] = k0
        st.cum_score[b, g, s] = 0.0


@pytest.mark.parametrize("N,budget,recent,steps", [(300, 250, 16, 24), (300, 1000, 16, 6), (10100, 10000, 64, 4)])
def test_h2o_fused_step_equals_three_calls(N, budget, recent, steps):
    banner(f"H2O fused step against three calls: N={N} budget={budget} recent={recent} steps={steps}")
    cfg = W.H2O("t", B=3, hq=8, hkv=2, d=128, N=N, budget=budget, recent=recent, steps=steps, zipf=1.1)
    inp = W.gen_h2o(cfg, seed=31, threads=3)
    rs = np.random.default_rng(32)
    st = inp["cache"]
    # scores of whole eighths from 1/8 up; the tied slots start at 0 below all of them, so the first evictions
    # choose among exact ties (by the higher position)
    st.cum_score[:, :, :N] = ((1 + rs.integers(0, 40, size=(3, 2, N))) / 8.0).astype(np.float32)
    _tied(inp, 0, 0, list(range(40, 48)))
    _tied(inp, 2, 1, [5, 77, 150, 151])
    dev = [to_device(st, cfg.hq), to_device(st, cfg.hq)]
    status = [status_word(), status_word()]
    steps_ = [WF.H2OStep(dev[i], scale=inp["scale"], budget=budget, recent=recent, status=status[i],
                         fused=(i == 0)) for i in range(2)]
    for s in range(steps):
        pos = i32(np.full((3,), N + s, np.int32))
        outs = []
        for i in range(2):
            o = steps_[i].run(storage_tensor(inp["k_new"][s], "bf16"), storage_tensor(inp["v_new"][s], "bf16"), pos,
                              storage_tensor(inp["q_steps"][s], "bf16"))
            outs.append(o.clone())
        assert torch.equal(outs[0], outs[1]), s
        assert torch.equal(steps_[0].evict_count, steps_[1].evict_count), s
        cnt = steps_[0].evict_count.cpu().numpy()
        e0, e1 = steps_[0].evict[:, :, 0].cpu().numpy(), steps_[1].evict[:, :, 0].cpu().numpy()
        np.testing.assert_array_equal(np.where(cnt > 0, e0, -1), np.where(cnt > 0, e1, -1))
        if budget < N:
            assert (cnt == 1).all(), s
        else:
            assert (cnt == 0).all(), s
        a, b = dev[0].to_numpy(), dev[1].to_numpy()
        for f in a:
            np.testing.assert_array_equal(a[f], b[f], err_msg=f"{f} after step {s}")
    for i in range(2):
        assert se.se_status_read(status[i]) == 0
