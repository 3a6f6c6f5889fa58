"""Host-side parts of the benchmark (no device): the one-GPU contract and the profile summaries it reads."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_too_many_pristine_copies_are_refused():
    r = run_bench("--steps", "60", "--warmup", "10")
    assert r.returncode == 2 and "<= 64" in r.stderr


def test_every_workload_has_a_traffic_summary_for_its_dominant_call():
    # the benchmark reads each workload's HBM traffic from its committed counter summary (and reports it only while
    # the kernel sources match the digest recorded there)
    import workloads as W

    dominant = {"c1_snapkv_llama8b": "se_window_score", "c2_kara_qwen3_4b": "se_sparse_decode_attn",
                "c3_quest_128k": "se_sparse_decode_attn", "c4_h2o": "se_sparse_decode_attn",
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
