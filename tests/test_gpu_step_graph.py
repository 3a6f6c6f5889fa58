"""The benchmark times each step of a restored workload as one captured HIP graph. These tests check that a replay
does exactly what the host-launched step does."""
import os
import sys

import pytest
import torch

import sparse_decode_attention_se_amd as se
import workloads as W
from gpu_util import DEV, status_word
from sparse_decode_attention_se_amd import workflows as WF

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def _snapshot(wl):
    return {k: v.clone() for k, v in wl.outputs.items()}


def _assert_equal(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs from the host-launched step"


@pytest.mark.parametrize("which", ["c1", "c2"])
def test_a_captured_step_replays_like_the_host_launched_step(which):
    """Small instances of the SnapKV event (scores, top-K, whole-cache gather, decode) and of Kara's event and decode
    step (scores, candidates, Token2Chunk, trailing gather, append, decode). Three replays of the captured step,
    each on the restored cache, with a host-launched step and synchronisations between them, give bit for bit the
    host-launched step's cache (every field), scores, lists and decode output."""
    print(f"\n[case] step graph {which}", flush=True)
    cfg = {"c1": W.scaled(W.C1, B=2, N=4096),
           "c2": W.scaled(W.C2, B=8, N=2048, period=1, events=1)}[which]
    status = status_word()
    wl = bench.SETUPS[which](se, WF, W, DEV, status, 1, cfg=cfg)
    wl.restore()
    for _, fn in wl.step(0):
        fn()
    torch.cuda.synchronize()
    assert se.se_status_read(status) == 0
    eager = _snapshot(wl)
    graph = bench.capture_step(wl, 0)
    for r in range(3):
        wl.restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert se.se_status_read(status) == 0
        _assert_equal(eager, _snapshot(wl), f"replay {r}")
        wl.restore()
        for _, fn in wl.step(0):
            fn()
        torch.cuda.synchronize()
        _assert_equal(eager, _snapshot(wl), f"host-launched step after replay {r}")
