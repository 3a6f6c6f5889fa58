"""Host-side parts of the benchmark (no device): the one-GPU contract and the profile summaries it reads."""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_a_device_error_stops_the_benchmark():
    # every call reports index and capacity errors into one status word; a nonzero word after the warm-up or the
    # timed steps must end the run instead of printing figures for work that was skipped
    import bench

    class FakeSe:
        SE_DEV_INDEX = 1

        def __init__(self, code):
            self.code = code

        def se_status_read(self, status):
            return self.code

    bench.require_clean_status(FakeSe(0), None, "the timed steps")
    with pytest.raises(SystemExit, match="index or capacity"):
        bench.require_clean_status(FakeSe(1), None, "the timed steps")


def _setup_calls(tree):
    """(function name, call node) for every call made inside bench.py's workload drivers."""
    for fn in tree.body:
        if isinstance(fn, ast.FunctionDef) and (fn.name.startswith("setup_") or fn.name == "run_policy_loop"):
            for node in ast.walk(fn):
                if isinstance(node, ast.Call):
                    yield fn.name, node


def test_every_call_and_driver_in_the_benchmark_takes_the_status_word():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    seen = 0
    for fname, call in _setup_calls(tree):
        f = call.func
        name = f.attr if isinstance(f, ast.Attribute) else getattr(f, "id", "")
        base = getattr(f.value, "id", "") if isinstance(f, ast.Attribute) else ""
        entry = base == "se" and name.startswith("se_") and name != "se_status_read"
        driver = base == "WF"
        if entry or driver:
            seen += 1
            kws = {k.arg for k in call.keywords}
            # the policy loop's drivers get it through **kw, which holds status
            assert "status" in kws or any(k.arg is None for k in call.keywords), (fname, name)
    assert seen > 20


def test_the_default_workload_is_the_largest():
    import bench
    import workloads as W

    ap_default = [ln for ln in open(os.path.join(ROOT, "bench.py")) if '"--workload", default=' in ln]
    assert len(ap_default) == 1 and 'default="c2"' in ap_default[0]
    sizes = {c.name: c.B * c.N * c.hkv for c in (W.C1, W.C2, W.C3, W.C4)}
    assert max(sizes, key=sizes.get) == W.C2.name
    assert bench.SETUPS["c2"] is bench.setup_c2


def test_every_workload_has_a_traffic_summary_for_its_dominant_call():
    # the benchmark reads each workload's HBM traffic from its committed counter summary (and reports it only while
    # the kernel sources match the digest recorded there)
    import workloads as W

    dominant = {"c1_snapkv_llama8b": "se_window_score", "c2_kara_qwen3_4b": "se_sparse_decode_attn",
                "c3_quest_128k": "se_sparse_decode_attn", "c4_h2o": "se_h2o_decode_evict",
                "c5_quest_128k_append": "se_sparse_decode_attn", "c6_prune_llama8b": "se_window_score",
                "c7_h2o_prefill_llama8b": "se_window_score", "c8_kvllm_policy_qwen3_4b": "se_sparse_decode_attn"}
    assert set(dominant) == {c.name for c in W.FULL.values()} - {W.C0.name}
    for workload, call in dominant.items():
        path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
        lines = [ln.split() for ln in open(path) if ln.startswith(f"traffic {call} ")]
        assert len(lines) == 1, workload
        kv = dict(x.split("=", 1) for x in lines[0][2:])
        # bytes, read and written are each rounded from the scaled counters
        assert abs(int(kv["bytes"]) - int(kv["read"]) - int(kv["written"])) <= 2 and int(kv["bytes"]) > 0
        assert len(kv["sources"]) == 16


def test_oracle_samples_draw_the_workload_sequences_they_name():
    # a CPU-baseline worker on sequences [first, first + n) generates exactly those sequences of the larger batch
    import numpy as np

    import workloads as W

    for gen, cfg in ((W.gen_quest, W.scaled(W.C3, N=1024, top_pages=8)),
                     (W.gen_h2o, W.scaled(W.C4, N=256, budget=256, recent=32, steps=3))):
        whole = gen(W.scaled(cfg, B=3), seed=0, threads=1)
        part = gen(W.scaled(cfg, B=1), seed=0, threads=1, first=2)
        for key in ("q_dec", "q_steps", "k_new", "v_new"):
            if key in whole:
                axis = 1 if key in ("q_steps", "k_new", "v_new") else 0
                assert np.array_equal(np.take(whole[key], [2], axis=axis), part[key]), key
        for pool in ("k_pool", "v_pool"):
            # the sequence's mapped blocks, through its block-table row in each cache
            ta, tb = whole["cache"].block_table[2], part["cache"].block_table[0]
            assert np.array_equal(ta >= 0, tb >= 0) and (ta >= 0).sum() > 0
            a = getattr(whole["cache"], pool)[ta[ta >= 0]]
            b = getattr(part["cache"], pool)[tb[tb >= 0]]
            assert np.array_equal(a, b), pool
