"""Benchmark of the sparse-KV hot path on one MI355X. Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c1|...|c8] [--no-cpu-baseline]

A step is one pass of the workload's hot path over its batch, with every input resident in HBM before timing:

  c2 (default, the headline: the largest workload) Kara periodic compression on 128 Qwen3-4B-shaped sequences x
     16384 tokens (32 q / 8 KV heads, d 128, bf16, page 16; an 8.6 GB cache): bidirectional scores of the trailing
     512-token window, top-20% candidates, Token2Chunk, trailing-block compaction, then one decode step (append +
     attention over the whole cache).
  c1 SnapKV-style prefill-end eviction on 8 Llama-3.1-8B-shaped sequences x 32768 tokens: causal window scores of
     the last 64 queries, top-1984 + 64 protected keys per KV head, in-place compaction with block freeing, one
     decode step over the retained KV.
  c3 Quest decode on 2 sequences x 131072 tokens: page bounds against the query, top-256 pages + first/last,
     decode attention over the 258 selected pages (page metadata built once, outside the step).
  c4 H2O continuous eviction on 64 sequences at the 8192-token budget: append, decode with cumulative scores,
     bottom-1 eviction outside the 256 most recent positions. The workload's 1024 steps run as one captured HIP
     graph, replayed on a restored cache; the line's step time is the replay's per decode step, and the per-call
     figures come from eager steps timed with events.
  c5 c3's Quest decode with its cache maintenance: append the decode token, refresh the metadata of its page,
     then page bounds, page choice and decode.
  c6 range-restricted pruning on c1's cache: window scores, the best 20% of positions [1024, 31744) among idle
     blocks (5% of blocks busy), the rest of the range freed, one decode step over the pruned cache.
  c7 H2O's chunked-prefill eviction on 8 x 8192 prompt tokens: per chunk of 512, the chunk's causal scores added
     to the cumulative scores, bottom-K down to the 2048 budget, slots freed (one step = the whole prefill).
  c8 compression policy loop on c2's batch: 128 decode steps (append + attention over the whole batch), with
     Kara's event on the sequences each policy names: KvLLM's periodic policy (all 128 sequences after step 128)
     against a threshold trigger (each sequence when its staggered uncompressed tail reaches 128 tokens, one
     event per step). A step is one decode step; the line reports decode tokens/s under the periodic policy and
     both policies' compression share. --steps and --warmup do not apply (one period, after an untimed pass).

Every workload but c4 changes its cache or would leave its working set in the 256 MB last-level cache between
steps, so before each of its steps the cache is copied back from one pristine clone and 1 GiB is read to flush
the last-level cache (leaving clean lines), outside the timed region; each step's wall time is taken between two device
synchronisations. c4's eager steps run back to back on one evolving cache. Per-call times come from HIP events on the
stream the calls are launched on. Every call reports index and capacity errors into one status word, checked
after the warm-up and after the timed steps. For c1 to c4 the oracle is timed on the host first, on all cores
(one worker process per core) and on one core.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# workloads whose step the oracle is timed on (the CPU baseline), and how many of H2O's steps its sample cycles over
ORACLE_WORKLOADS = ("c1", "c2", "c3", "c4")
ORACLE_H2O_STEPS = 64


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev_bf16(x, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)


def device_cache(se, cfg, c, dev):
    return se.DeviceCache.from_arrays(cfg.hq, cfg.dtype, dev, **{f: getattr(c, f) for f in se.DeviceCache.FIELDS
                                                                  if getattr(c, f, None) is not None})


# kernels each call launches (for matching profiler rows to calls) and the sources they are built from
CALL_KERNELS = {
    "se_window_score": ["window_stream", "window_bidir", "colsum_reduce", "stats_valu", "colsum_valu"],
    "se_topk_select": ["topk_kernel"],
    "se_token2chunk": ["t2c_kernel"],
    "se_compact_evict": ["gather_move", "gather_small", "gather_extents", "gather_push", "evict_slots_kernel"],
    "se_cache_append": ["append_plan", "append_copy"],
    "se_cache_append_chunk": ["chunk_plan", "chunk_write"],
    "se_page_bounds": ["pages_score", "pages_build"],
    "se_page_bounds_refresh": ["pages_refresh"],
    "se_h2o_decode_evict": ["h2o_decode_unit"],
    "se_sparse_decode_attn": ["decode_partial", "decode_merge", "decode_cum", "decode_unit"],
}
CALL_SOURCES = {
    "se_window_score": "score.hip", "se_topk_select": "topk.hip", "se_token2chunk": "t2c.hip",
    "se_compact_evict": "compact.hip", "se_cache_append": "compact.hip", "se_cache_append_chunk": "compact.hip", "se_page_bounds": "pages.hip",
    "se_page_bounds_refresh": "pages.hip",
    "se_sparse_decode_attn": "decode.hip", "se_h2o_decode_evict": "decode.hip",
}
CSRC = os.path.join(ROOT, "sparse_decode_attention_se_amd", "csrc")


def source_digest(call):
    """Digest of a call's kernel sources with comments and blank space removed, so that only code changes count."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in (CALL_SOURCES[call], "common.hpp"):
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def call_of(kernel_name):
    for call, ks in CALL_KERNELS.items():
        if any(k in kernel_name for k in ks):
            return call
    return None


def measured_traffic(workload, call):
    """HBM bytes per call from the committed counter summary of this workload, or None when that summary is
    missing or the call's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and f[0] == "traffic" and f[1] == call:
            kv = dict(x.split("=", 1) for x in f[2:] if "=" in x)
            if kv.get("sources") != source_digest(call):
                return None
            return int(float(kv["bytes"]))
    return None


def read_csv(path):
    import csv

    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def summarize_profile(directories, calls_per_run, copy_bytes, fetch_factor, write_factor):
    """Text summary of rocprofv3 CSV output directories: per-kernel duration statistics (kernel trace), per-kernel
    counter averages and per-call counter sums (counter collection). With both FETCH_SIZE and WRITE_SIZE present,
    prints one ``traffic`` line per call: HBM bytes per call, each counter divided by the factor a plain copy of
    known size reads for it, tagged with a digest of the call's sources. Kernels dispatched fewer times than
    there were calls (set-up work outside the step) are left out of the per-call sums."""
    import glob

    out = []
    per_call = {}
    for directory in directories:
        for path in sorted(glob.glob(os.path.join(directory, "**", "*_kernel_stats.csv"), recursive=True)):
            out.append(f"kernel statistics ({os.path.basename(path)}):")
            out.append(f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10}  kernel")
            for r in read_csv(path):
                out.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                           f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}  {r['Name'][:110]}")
        for path in sorted(glob.glob(os.path.join(directory, "**", "*_counter_collection.csv"), recursive=True)):
            per_kernel = {}
            for r in read_csv(path):
                pk = per_kernel.setdefault((r["Kernel_Name"], r["Counter_Name"]), [0.0, 0])
                pk[0] += float(r["Counter_Value"])
                pk[1] += 1
            out.append(f"counters ({os.path.basename(path)}), per dispatch:")
            for (name, ctr), (tot, n) in sorted(per_kernel.items()):
                c = call_of(name) or ("copy" if copy_bytes and "neg_kernel" in name else None)
                if c is None:
                    continue
                out.append(f"  {ctr:12s} {tot / n:14.1f} KiB avg over {n:3d} dispatches  {name[:100]}")
                if c == "copy":
                    out.append(f"calibration {ctr} factor={tot * 1024 / (n * copy_bytes):.4f} "
                               f"(counter bytes / bytes each copy launch reads or writes)")
                elif n >= calls_per_run:
                    per_call[(c, ctr)] = per_call.get((c, ctr), 0.0) + tot / calls_per_run
    for (c, ctr), kib in sorted(per_call.items()):
        out.append(f"per-call {c} {ctr}_KiB={kib:.1f}")
    for c in sorted({c for c, _ in per_call}):
        if (c, "FETCH_SIZE") in per_call and (c, "WRITE_SIZE") in per_call:
            fetch = per_call[(c, "FETCH_SIZE")] * 1024 / fetch_factor
            write = per_call[(c, "WRITE_SIZE")] * 1024 / write_factor
            out.append(f"traffic {c} bytes={fetch + write:.0f} read={fetch:.0f} written={write:.0f} "
                       f"sources={source_digest(c)}")
    return "\n".join(out)


def calibrate_copy(mib, reps):
    """A plain streaming copy of known size (torch's elementwise negation: reads and writes mib MiB per launch), for
    counter calibration."""
    import torch

    n = mib * 2**20 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": reps}), flush=True)


def copy_ceiling(reps):
    """What a plain streaming kernel reaches at the byte counts of the smaller calls: torch's elementwise negation
    moving 2 x S bytes (S read, S written) per launch, timed with events over reps back-to-back launches."""
    import torch

    for mib in (8, 16, 32, 64, 128, 256, 1024):
        n = mib * 2**20 // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.neg(x, out=y)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        moved = 2 * n * 4
        print(json.dumps({"copy_mib": mib, "bytes_moved": moved, "us": round(us, 2),
                          "gb_s": round(moved / us / 1e3, 1), "frac_of_8tb": round(moved / us / 8e6, 3)}), flush=True)
        del x, y


# ---------------------------------------------------------------------------------------------------------------
# workloads: each builds a Workload on the device
# ---------------------------------------------------------------------------------------------------------------


class Workload:
    """A benchmark workload on the device.

    step(i) -> [(entry point, fn)]: the calls of step i, in order. restore: None for a workload whose steps run
    back to back on one evolving cache (H2O); otherwise a function that puts the cache back into its pristine state
    before a step (a device copy from one pristine clone), outside the timed region. tokens: KV tokens per step (the
    metric's unit); alg: algorithmic bytes (and flops for scoring) per call of each entry point."""

    def __init__(self, cfg, tokens, alg, step, restore=None, outputs=None):
        self.cfg, self.tokens, self.alg, self.step, self.restore = cfg, tokens, alg, step, restore
        self.outputs = outputs or {}  # named device tensors a step writes besides the cache (for tests)


def per_call_marks(wl, args, prepare, calls, first):
    """[(start, end) event per call] for each of args.steps steps (numbered from `first`; restored first when the
    workload restores) queued behind a device spin."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(1 << 22)
    e1.record()
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 22) / max(e0.elapsed_time(e1), 1e-3)
    spin_ms = 4.0
    marks = []
    i = tried = 0  # a retried step of an evolving cache takes the next step's inputs (its own were consumed)
    while i < args.steps:
        prepare()
        torch.cuda.synchronize()
        torch.cuda._sleep(int(spin_ms * cycles_per_ms))
        m = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
        step = first + (i if wl.restore else tried)
        tried += 1
        for (name, fn), (a, b) in zip(wl.step(step), m):
            a.record()
            fn()
            b.record()
        late = m[0][0].query()  # the device reached the first call before the host had queued the step
        torch.cuda.synchronize()
        if late and spin_ms < 1000:
            spin_ms *= 2
            continue
        marks.append(m)
        i += 1
    return marks


def capture_step(wl, i):
    """The calls of step ``i`` captured as one HIP graph on a side stream (run once eagerly there first, as capture
    requires), on the restored cache; the caller restores it again before each replay."""
    import torch

    wl.restore()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, fn in wl.step(i):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    wl.restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn in wl.step(i):
            fn()
    torch.cuda.synchronize()
    return g


def cache_tensors(se, c):
    """Every field of a device cache, by name."""
    return {f"cache.{f}": getattr(c, f) for f in se.DeviceCache.FIELDS if getattr(c, f) is not None}


def restorer(se, work):
    """A pristine clone of the cache and a function that copies it back into ``work`` (every field)."""
    pristine = work.clone()

    def restore():
        for f in se.DeviceCache.FIELDS:
            x = getattr(work, f)
            if x is not None:
                x.copy_(getattr(pristine, f))

    return restore


def setup_c1(se, WF, W, dev, status, steps, cfg=None):
    import torch

    cfg = cfg or W.C1
    inp = W.gen_snapkv(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    q_win, q_dec = to_dev_bf16(inp["q_win"], dev), to_dev_bf16(inp["q_dec"], dev)
    q_pos = torch.from_numpy(inp["q_pos"]).to(dev)
    e = WF.SnapKVEvent(c, wq=cfg.wq, protect=cfg.protect, keep=cfg.keep, scale=inp["scale"], status=status)
    calls = [("se_window_score", lambda: e.score(q_win, q_pos)), ("se_topk_select", e.select),
             ("se_compact_evict", e.compact), ("se_sparse_decode_attn", lambda: e.decode(q_dec))]
    B, G, N, r, row = cfg.B, cfg.hkv, cfg.N, cfg.hq // cfg.hkv, cfg.d * 2
    keep = cfg.keep + cfg.protect
    alg = {
        "se_window_score": {"bytes": B * G * N * row + B * cfg.hq * cfg.wq * row + B * G * N * 4,
                            "flops": 2.0 * B * G * r * cfg.wq * N * cfg.d},
        "se_topk_select": {"bytes": B * G * N * 4 * 2 + B * G * keep * 4},
        "se_compact_evict": {"bytes": 2 * (B * G * keep * row * 2) + 2 * B * G * keep * 4},
        "se_sparse_decode_attn": {"bytes": B * G * keep * row * 2 + B * cfg.hq * cfg.d * (2 + 4)},
    }
    return Workload(cfg, B * N, alg, lambda i: calls, restorer(se, c),
                    outputs=dict(cache_tensors(se, c), scores=e.scores, idx=e.idx, count=e.count, out=e.out))


def setup_c2(se, WF, W, dev, status, steps, cfg=None):
    """Kara's event on the whole batch (bidirectional window scores, top-K candidates, Token2Chunk, trailing-window
    compaction), then one decode step (append, attention over every resident slot)."""
    import torch

    cfg = cfg or W.scaled(W.C2, period=1, events=1)
    inp = W.gen_kara(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    # the fresh cache's trailing window holds positions N - window .. N - 1, the first queries the workload keeps
    assert inp["q_first_pos"] == cfg.N - cfg.window
    q_win = to_dev_bf16(np.ascontiguousarray(inp["q_all"][:, :, :cfg.window]), dev)
    k_new, v_new = to_dev_bf16(inp["k_new"][0], dev), to_dev_bf16(inp["v_new"][0], dev)
    q = to_dev_bf16(np.ascontiguousarray(inp["q_all"][:, :, cfg.N - inp["q_first_pos"]]), dev)
    pos = torch.full((cfg.B,), cfg.N, dtype=torch.int32, device=dev)
    del inp
    ev = WF.KaraEvent(c, window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                      max_gap=cfg.max_gap, scale=1.0 / np.sqrt(cfg.d), status=status)
    dec = WF.DecodeStep(c, scale=ev.scale, status=status)
    calls = [
        ("se_window_score", lambda: se.se_window_score(
            c, q_win, None, ev.scores, scale=ev.scale, mode=se.SE_SCORE_BIDIR, n_query=cfg.window,
            window=cfg.window, protect=cfg.protect, status=status)),
        ("se_topk_select", lambda: se.se_topk_select(
            c, ev.scores, ev.cand, ev.cand_count, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_SLOT,
            k=cfg.n_cand, window=cfg.window, protect=cfg.protect, status=status)),
        ("se_token2chunk", lambda: se.se_token2chunk(
            c, ev.cand, ev.cand_count, ev.scores, ev.keep, ev.keep_count, max_gap=cfg.max_gap,
            budget=cfg.budget, window=cfg.window, protect=cfg.protect, status=status)),
        ("se_compact_evict", lambda: se.se_compact_evict(
            c, ev.keep, ev.keep_count, mode=se.SE_COMPACT_GATHER, window=cfg.window, status=status)),
        ("se_cache_append", lambda: se.se_cache_append(c, k_new, v_new, pos, status=status)),
        ("se_sparse_decode_attn", lambda: se.se_sparse_decode_attn(c, q, dec.out, scale=dec.scale,
                                                                   status=status)),
    ]
    B, G, N, r, row, W_ = cfg.B, cfg.hkv, cfg.N, cfg.hq // cfg.hkv, cfg.d * 2, cfg.window
    R = W_ - cfg.protect
    kept = cfg.budget + cfg.protect  # upper bound of the retained window
    after = N - W_ + kept + 1
    alg = {
        "se_window_score": {"bytes": B * G * R * row + B * cfg.hq * W_ * row + B * G * R * 4,
                            "flops": 2.0 * B * G * r * W_ * R * cfg.d},
        "se_topk_select": {"bytes": B * G * (R * 4 + W_ * 4)},
        "se_token2chunk": {"bytes": B * G * (R * 4 + 2 * kept * 4)},
        "se_compact_evict": {"bytes": 2 * B * G * kept * (2 * row + 4)},
        "se_cache_append": {"bytes": 2 * B * G * row * 2},
        "se_sparse_decode_attn": {"bytes": B * G * after * (2 * row + 4) + B * cfg.hq * cfg.d * (2 + 4)},
    }
    return Workload(cfg, B * W_, alg, lambda i: calls, restorer(se, c),
                    outputs=dict(cache_tensors(se, c), scores=ev.scores, cand=ev.cand, keep=ev.keep,
                                 keep_count=ev.keep_count, out=dec.out))


def setup_c3(se, WF, W, dev, status, steps):
    cfg = W.C3
    inp = W.gen_quest(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    q = to_dev_bf16(inp["q_dec"], dev)
    qs = WF.QuestStep(c, top_pages=cfg.top_pages, scale=inp["scale"], status=status)
    qs.build()  # page metadata: built once for the cache, outside the step
    calls = [
        ("se_page_bounds", lambda: se.se_page_bounds(c, se.SE_PAGES_SCORE, q, qs.page_scores, status=status)),
        ("se_topk_select", lambda: se.se_topk_select(
            c, qs.page_scores, qs.pages, qs.count, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_PAGE,
            k=cfg.top_pages, forced_ends=1, status=status)),
        ("se_sparse_decode_attn", lambda: se.se_sparse_decode_attn(
            c, q, qs.out, scale=qs.scale, sel_pages=qs.pages, sel_count=qs.count, status=status)),
    ]
    B, G, N, row = cfg.B, cfg.hkv, cfg.N, cfg.d * 2
    P_ = N // cfg.page
    sel = cfg.top_pages + 2
    alg = {
        "se_page_bounds": {"bytes": B * G * P_ * 2 * row + B * G * P_ * 4 + B * cfg.hq * row},
        "se_topk_select": {"bytes": B * G * P_ * 4 + B * G * sel * 4},
        "se_sparse_decode_attn": {"bytes": B * G * sel * cfg.page * (2 * row + 4) + B * cfg.hq * cfg.d * (2 + 4)},
    }
    return Workload(cfg, B * N, alg, lambda i: calls, restorer(se, c))


def setup_c5(se, WF, W, dev, status, steps):
    """C3's Quest decode step with its cache maintenance: append the decode token, refresh the metadata of the page
    it wrote, then page scores, page choice and decode."""
    import torch

    cfg = W.C5
    inp = W.gen_quest(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    q = to_dev_bf16(inp["q_dec"], dev)
    k_new, v_new = to_dev_bf16(inp["k_new"][0], dev), to_dev_bf16(inp["v_new"][0], dev)
    pos = torch.full((cfg.B,), cfg.N, dtype=torch.int32, device=dev)
    qs = WF.QuestStep(c, top_pages=cfg.top_pages, scale=inp["scale"], status=status)
    qs.build()
    calls = [
        ("se_cache_append", lambda: se.se_cache_append(c, k_new, v_new, pos, status=status)),
        ("se_page_bounds_refresh", qs.refresh_last_page),
        ("se_page_bounds", lambda: se.se_page_bounds(c, se.SE_PAGES_SCORE, q, qs.page_scores, status=status)),
        ("se_topk_select", lambda: se.se_topk_select(
            c, qs.page_scores, qs.pages, qs.count, mode=se.SE_TOPK_LARGEST, unit=se.SE_UNIT_PAGE,
            k=cfg.top_pages, forced_ends=1, status=status)),
        ("se_sparse_decode_attn", lambda: se.se_sparse_decode_attn(
            c, q, qs.out, scale=qs.scale, sel_pages=qs.pages, sel_count=qs.count, status=status)),
    ]
    B, G, N, row = cfg.B, cfg.hkv, cfg.N + 1, cfg.d * 2
    P_ = -(-N // cfg.page)
    sel = cfg.top_pages + 2
    alg = {
        "se_cache_append": {"bytes": B * G * 2 * row * 2 + B * G * 4 * 4},
        "se_page_bounds_refresh": {"bytes": B * G * (cfg.page * row + 2 * row)},
        "se_page_bounds": {"bytes": B * G * P_ * 2 * row + B * G * P_ * 4 + B * cfg.hq * row},
        "se_topk_select": {"bytes": B * G * P_ * 4 + B * G * sel * 4},
        "se_sparse_decode_attn": {"bytes": B * G * sel * cfg.page * (2 * row + 4) + B * cfg.hq * cfg.d * (2 + 4)},
    }
    return Workload(cfg, B * N, alg, lambda i: calls, restorer(se, c))


def setup_c6(se, WF, W, dev, status, steps):
    """Range-restricted pruning on the Llama-8B cache: window scores, the range's best slots among idle blocks (the
    dropped list), slot eviction, then a decode step over the pruned cache."""
    import torch

    cfg = W.C6
    inp = W.gen_prune(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    q_win, q_dec = to_dev_bf16(inp["q_win"], dev), to_dev_bf16(inp["q_dec"], dev)
    q_pos = torch.from_numpy(inp["q_pos"]).to(dev)
    refs = torch.from_numpy(inp["block_refs"]).to(dev)
    out = torch.empty((cfg.B, cfg.hq, cfg.d), dtype=torch.float32, device=dev)
    p = WF.PruneRange(c, wq=cfg.wq, scale=inp["scale"], status=status)
    calls = [("se_window_score", lambda: p.score(q_win, q_pos)),
             ("se_topk_select", lambda: p.select(cfg.range_lo, cfg.range_hi, cfg.keep, refs)),
             ("se_compact_evict", p.evict),
             ("se_sparse_decode_attn", lambda: se.se_sparse_decode_attn(c, q_dec, out, scale=inp["scale"],
                                                                        status=status))]
    B, G, N, r, row, page = cfg.B, cfg.hkv, cfg.N, cfg.hq // cfg.hkv, cfg.d * 2, cfg.page
    # slots each unit frees: the idle slots of the range beyond the kept ones (every slot starts resident)
    c0 = inp["cache"]
    slots = np.arange(cfg.range_lo, cfg.range_hi)
    dropped = sum(max(int((inp["block_refs"][c0.block_table[b, slots // page]] == 0).sum()) - cfg.keep, 0)
                  for b in range(B)) * G
    alg = {
        "se_window_score": {"bytes": B * G * N * row + B * cfg.hq * cfg.wq * row + B * G * N * 4,
                            "flops": 2.0 * B * G * r * cfg.wq * N * cfg.d},
        "se_topk_select": {"bytes": B * G * N * 4 * 2 + 2 * B * (N // page) * 4 + dropped * 4},
        "se_compact_evict": {"bytes": dropped * 4 * 3},
        "se_sparse_decode_attn": {"bytes": (B * G * N - dropped) * row * 2 + B * G * N * 4 + B * cfg.hq * cfg.d * 6},
    }
    return Workload(cfg, B * N, alg, lambda i: calls, restorer(se, c))


def setup_c7(se, WF, W, dev, status, steps):
    """H2O's chunked-prefill eviction on 8 x 8192 prompt tokens: per chunk of 512, the chunk appended, its causal
    window scores added to the cumulative scores, the recent 256 plus the best 1792 others kept (the 2048 budget)
    and the cache compacted in place. One step is the whole prefill (16 chunks)."""
    import torch

    cfg = W.C7
    inp = W.gen_h2o_prefill(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    n_chunks = cfg.N // cfg.chunk
    sl = [slice(k * cfg.chunk, (k + 1) * cfg.chunk) for k in range(n_chunks)]
    q_ch = [to_dev_bf16(np.ascontiguousarray(inp["q_all"][:, :, x]), dev) for x in sl]
    k_ch = [to_dev_bf16(np.ascontiguousarray(inp["k_all"][:, :, x]), dev) for x in sl]
    v_ch = [to_dev_bf16(np.ascontiguousarray(inp["v_all"][:, :, x]), dev) for x in sl]
    q_pos = [torch.arange(x.start, x.stop, dtype=torch.int32, device=dev).repeat(cfg.B, 1) for x in sl]
    pos0 = [torch.full((cfg.B,), x.start, dtype=torch.int32, device=dev) for x in sl]
    pf = WF.H2OPrefillChunk(c, chunk=cfg.chunk, budget=cfg.budget, recent=cfg.recent, scale=inp["scale"],
                            status=status)
    calls = []
    for k in range(n_chunks):
        if k > 0:
            calls.append(("se_cache_append_chunk", lambda k=k: pf.append(k_ch[k], v_ch[k], pos0[k])))
        calls += [("se_window_score", lambda k=k: pf.score(q_ch[k], q_pos[k])),
                  ("se_topk_select", pf.select), ("se_compact_evict", pf.compact)]
    B, G, r, row, d = cfg.B, cfg.hkv, cfg.hq // cfg.hkv, cfg.d * 2, cfg.d
    # per chunk k: the keys its queries see (the budget's survivors, then the chunk; the cache is dense), and the
    # rows compaction keeps
    keys = [min(k * cfg.chunk, cfg.budget) + cfg.chunk for k in range(n_chunks)]
    kept = [min(kk, cfg.budget) for kk in keys]
    alg = {
        "se_cache_append_chunk": {"bytes": (n_chunks - 1) * B * G * cfg.chunk * (2 * row * 2 + 4)},
        "se_window_score": {"bytes": sum(B * G * (kk * row + kk * 8) + B * cfg.hq * cfg.chunk * row for kk in keys),
                            "flops": sum(2.0 * B * G * r * cfg.chunk * kk * d for kk in keys)},
        "se_topk_select": {"bytes": sum(B * G * (kk * 8 + kp * 4) for kk, kp in zip(keys, kept))},
        "se_compact_evict": {"bytes": sum(B * G * kp * (2 * row * 2 + 8) for kp in kept)},
    }
    return Workload(cfg, B * cfg.N, alg, lambda i: calls, restorer(se, c))


def setup_c4(se, WF, W, dev, status, steps):
    """H2O's decode loop: each step appends its token, attends with cumulative scores, evicts the lowest score
    outside the recent positions. The workload's 1024 steps run as one captured HIP graph (`graph`, replayed on a
    restored cache); the per-call figures come from steps run eagerly with events on a copy."""
    import torch

    cfg = W.C4
    inp = W.gen_h2o(cfg, seed=0, threads=16)
    c = device_cache(se, cfg, inp["cache"], dev)
    k_new = [to_dev_bf16(inp["k_new"][s], dev) for s in range(cfg.steps)]
    v_new = [to_dev_bf16(inp["v_new"][s], dev) for s in range(cfg.steps)]
    q = [to_dev_bf16(inp["q_steps"][s], dev) for s in range(cfg.steps)]
    pos = [torch.full((cfg.B,), cfg.N + s, dtype=torch.int32, device=dev) for s in range(cfg.steps)]
    del inp
    restore = restorer(se, c)
    h2o = WF.H2OStep(c, scale=1.0 / np.sqrt(cfg.d), budget=cfg.budget, recent=cfg.recent, status=status)

    def step(s):
        s = s % cfg.steps
        return [
            ("se_cache_append", lambda: se.se_cache_append(c, k_new[s], v_new[s], pos[s], status=status)),
            ("se_h2o_decode_evict", lambda: se.se_h2o_decode_evict(c, q[s], h2o.out, h2o.evict, h2o.evict_count,
                                                                   scale=h2o.scale, budget=cfg.budget,
                                                                   recent=cfg.recent, status=status)),
        ]

    B, G, row = cfg.B, cfg.hkv, cfg.d * 2
    n = cfg.budget + 1
    alg = {
        "se_cache_append": {"bytes": 2 * B * G * row * 2},
        # K and V rows, positions, cumulative scores read and written; queries and outputs; the eviction's writes
        "se_h2o_decode_evict": {"bytes": B * G * n * (2 * row + 4 + 8) + B * cfg.hq * cfg.d * (2 + 4) + B * G * 28},
    }
    wl = Workload(cfg, B * n, alg, step)

    def capture():
        return WF.H2OGraph(c, k_new, v_new, pos, q, scale=h2o.scale, budget=cfg.budget, recent=cfg.recent,
                           status=status)

    wl.graph, wl.graph_restore = capture, restore
    return wl


SETUPS = {"c1": setup_c1, "c2": setup_c2, "c3": setup_c3, "c4": setup_c4, "c5": setup_c5, "c6": setup_c6,
          "c7": setup_c7}


def run_policy_loop(se, WF, W, dev, status):
    """c8: one period of decode steps under each compression policy. Returns the JSON line."""
    import torch

    cfg = W.C8
    t0 = time.time()
    inp = W.gen_kara(cfg, seed=0, threads=16)
    base = device_cache(se, cfg, inp["cache"], dev)
    S, B, G, row = cfg.steps, cfg.B, cfg.hkv, cfg.d * 2
    q0 = inp["q_first_pos"]
    k_new = [to_dev_bf16(inp["k_new"][t], dev) for t in range(S)]
    v_new = [to_dev_bf16(inp["v_new"][t], dev) for t in range(S)]
    q_dec = [to_dev_bf16(np.ascontiguousarray(inp["q_all"][:, :, cfg.N + t - q0]), dev) for t in range(S)]
    pos = [torch.full((B,), cfg.N + t, dtype=torch.int32, device=dev) for t in range(S)]
    # each event's window queries are those of its sequences' `window` most recent tokens: a slice of the stored
    # queries, staged per scheduled run before timing (the schedules do not depend on the data)
    q_run = {}
    kw = dict(period=cfg.period, window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
              max_gap=cfg.max_gap, scale=inp["scale"], status=status)
    for policy in WF.CompressionLoop.POLICIES:
        probe = WF.CompressionLoop(base, policy=policy, **kw)
        for t in range(S):
            s = cfg.N + t + 1 - cfg.window - q0
            for b0, b1 in probe.due(t):
                if (b0, b1, t) not in q_run:
                    q_run[(b0, b1, t)] = to_dev_bf16(
                        np.ascontiguousarray(inp["q_all"][b0:b1, :, s:s + cfg.window]), dev)

    def window_queries(b0, b1, t):
        return q_run[(b0, b1, t)]

    del inp
    torch.cuda.synchronize()
    log(f"{cfg.name}: inputs ready in {time.time() - t0:.1f} s, {torch.cuda.memory_allocated() / 2**30:.1f} GiB "
        f"resident")

    results = {}
    for policy in WF.CompressionLoop.POLICIES:
        # untimed pass: warms up and records each step's view size (the kernels are deterministic, so the timed
        # pass on a fresh copy sees the same sizes)
        loop = WF.CompressionLoop(base.clone(), policy=policy, **kw)
        view_rows = []
        for t in range(S):
            loop.decode(k_new[t], v_new[t], pos[t], q_dec[t])
            view_rows.append(int(loop.cache.n_slots.sum()))
            for b0, b1 in loop.due(t):
                loop.compress(b0, b1, window_queries(b0, b1, t))
        require_clean_status(se, status, f"the untimed {policy} pass")
        del loop
        loop = WF.CompressionLoop(base.clone(), policy=policy, **kw)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(S)]
        prev = se.set_operand_checks(False)  # the untimed pass checked operands of the same shapes
        compress_steps = []
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for t in range(S):
            e = ev[t]
            se.se_cache_append(loop.cache, k_new[t], v_new[t], pos[t], status=status)
            e[0].record()
            se.se_sparse_decode_attn(loop.cache, q_dec[t], loop.out, scale=loop.scale, status=status)
            e[1].record()
            runs = loop.due(t)
            if runs:
                compress_steps.append(t)
                for b0, b1 in runs:
                    loop.compress(b0, b1, window_queries(b0, b1, t))
                e[2].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        se.set_operand_checks(prev)
        require_clean_status(se, status, f"the timed {policy} pass")
        dec_ms = [ev[t][0].elapsed_time(ev[t][1]) for t in range(S)]
        comp_ms = sum(ev[t][1].elapsed_time(ev[t][2]) for t in compress_steps)
        n_events = sum(len(loop.due(t)) for t in range(S))
        dec_bytes = float(np.mean(view_rows)) * (2 * row + 4) + B * cfg.hq * cfg.d * (2 + 4)
        results[policy] = {
            "ms_per_step": round(elapsed * 1e3 / S, 4),
            "tokens_per_s": round(B * S / elapsed, 1),
            "events": n_events,
            "decode_ms": round(float(np.mean(dec_ms)), 4),
            "decode_gb_s": round(dec_bytes / (float(np.mean(dec_ms)) * 1e-3) / 1e9, 1),
            "compress_ms_total": round(comp_ms, 3),
            "compress_share": round(comp_ms / (elapsed * 1e3), 4),
        }
        log(f"{policy}: {results[policy]}")
        del loop
        torch.cuda.empty_cache()

    per = results["periodic"]
    a = per["decode_gb_s"]
    return {
        "metric": "decode tokens/s",
        "value": per["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": S,
        "ms_per_step": per["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "seq_len": cfg.N, "q_heads": cfg.hq, "kv_heads": cfg.hkv,
                   "head_dim": cfg.d, "page": cfg.page, "window": cfg.window, "period": cfg.period,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(a / HBM_PEAK_GBS, 4), "kernel": "se_sparse_decode_attn",
                     "launches": CALL_KERNELS["se_sparse_decode_attn"],
                     "traffic": measured_traffic(cfg.name, "se_sparse_decode_attn")},
        "policies": results,
        "threshold_vs_periodic": round(results["threshold"]["tokens_per_s"] / per["tokens_per_s"], 4),
    }


# ---------------------------------------------------------------------------------------------------------------
# the oracle on the host cores (a baseline, not the target)
# ---------------------------------------------------------------------------------------------------------------


def _oracle_sample(workload, first, n_seq):
    """Inputs of sequences [first, first + n_seq) of a workload and a function running its step on the oracle once
    (returns the KV tokens of the metric that step covers)."""
    import oracle.pipelines as P
    import workloads as W

    if workload == "c1":
        cfg = W.scaled(W.C1, B=n_seq)
        inp = W.gen_snapkv(cfg, seed=0, threads=1, first=first)
        return lambda: (P.snapkv_event(inp), n_seq * cfg.N)[1]
    if workload == "c2":
        cfg = W.scaled(W.C2, B=n_seq, period=1, events=1)
        inp = W.gen_kara(cfg, seed=0, threads=1, first=first)

        def run():
            ev = P.kara_event(inp, inp["cache"])
            P.kara_decode_step(inp, ev["cache"], 0)
            return n_seq * cfg.window

        return run
    if workload == "c3":
        cfg = W.scaled(W.C3, B=n_seq)
        inp = W.gen_quest(cfg, seed=0, threads=1, first=first)
        return lambda: (P.quest_step(inp), n_seq * cfg.N)[1]
    if workload == "c4":
        # the workload's own inputs (1024 steps drawn); the sample cycles over its first ORACLE_H2O_STEPS steps,
        # starting again from the initial cache after the last of them
        cfg = W.scaled(W.C4, B=n_seq)
        inp = W.gen_h2o(cfg, seed=0, threads=1, first=first)
        state = {"cache": inp["cache"].copy(), "t": 0}

        def run():
            if state["t"] == ORACLE_H2O_STEPS:
                state["cache"], state["t"] = inp["cache"].copy(), 0
            state["cache"], _ = P.h2o_step(inp, state["cache"], state["t"])
            state["t"] += 1
            return n_seq * (cfg.budget + 1)

        return run
    raise ValueError(workload)


def _oracle_worker(workload, first, n_seq, min_seconds, barrier, results):
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):  # one core per worker: numpy's BLAS would otherwise start a pool of its own
        run = _oracle_sample(workload, first, n_seq)
        if barrier is not None:
            barrier.wait()
        tokens, reps = 0, 0
        t0 = time.perf_counter()
        while True:
            tokens += run()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                results.put((tokens, reps, dt))
                return


def _run_workers(ctx, workload, n, n_seq, min_seconds):
    """n forked worker processes, worker w on sequences [w n_seq, (w + 1) n_seq), timed from a common start."""
    barrier = ctx.Barrier(n) if n > 1 else None
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(workload, w * n_seq, n_seq, min_seconds, barrier, results))
             for w in range(n)]
    for p in procs:
        p.start()
    out = [results.get() for _ in procs]
    for p in procs:
        p.join()
        if p.exitcode != 0:
            raise RuntimeError(f"oracle worker exited with {p.exitcode}")
    return out


def host_cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return n


def cpu_baseline(workload, n_seq, min_seconds, max_workers=16):
    """The oracle as it stands, timed on the host: once with one worker process per core (up to ``max_workers``,
    each on its own ``n_seq`` sequences of the workload, started together), once on a single core. Each worker runs
    the workload's step on its sample until ``min_seconds`` have passed. Runs before the GPU is touched (the
    workers are forked)."""
    import multiprocessing as mp

    ctx = mp.get_context("fork")
    avail = host_cores()
    n = max(1, min(max_workers, avail))
    res = _run_workers(ctx, workload, n, n_seq, min_seconds)
    wall = max(r[2] for r in res)
    tokens = sum(r[0] for r in res)
    one = _run_workers(ctx, workload, 1, n_seq, min_seconds)[0]
    what = {"c1": "the whole event (window scores, top-K, compaction, decode)",
            "c2": "the whole step (Kara's event: window scores, top-K, Token2Chunk, compaction; then append and "
                  "decode)",
            "c3": "the whole step (page metadata build, page scores, top pages, decode over them)",
            "c4": f"decode steps (append, decode with cumulative scores, bottom-1, eviction) cycling over the first "
                  f"{ORACLE_H2O_STEPS} of the workload's 1024"}[workload]
    return {
        "value": round(tokens / wall, 1), "unit": "KV tokens/s", "cores": n, "kind": "oracle",
        "sample": f"{n} worker processes (one per core of {avail} available, BLAS limited to one thread each), "
                  f"worker w on sequences [{n_seq}w, {n_seq}w + {n_seq}) of the same workload, {what}, repeated "
                  f"for at least {min_seconds:g} s: {sum(r[1] for r in res)} steps of {n_seq} sequences in "
                  f"{wall:.1f} s",
        "single_core": {"value": round(one[0] / one[2], 1), "unit": "KV tokens/s", "cores": 1,
                        "sample": f"sequences [0, {n_seq}), {one[1]} steps in {one[2]:.1f} s"},
    }


def require_clean_status(se, status, when):
    """Stop the benchmark if any call flagged a device-side error (index or capacity): the figures would be for
    work that was skipped."""
    code = se.se_status_read(status)
    if code != 0:
        raise SystemExit(f"device status {code:#x} after {when}: a call reported an index or capacity error")


def flush_llc(buf):
    """Read 1 GiB so that nothing a step reads is left in the 256 MB last-level cache. A read leaves clean lines
    behind: a write would leave 256 MB of dirty lines whose write-back the step's first large kernel would pay."""
    buf.amax()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2", choices=sorted(SETUPS) + ["c8"])
    ap.add_argument("--cpu-seqs", type=int, help="sequences per oracle worker in the CPU baseline (default: 1 for "
                    "c3's 128K-token sequences, else 2)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="host-launched steps only: no captured HIP graph and no separate per-call pass (for profiler "
                         "runs that count calls per step)")
    ap.add_argument("--calibrate-copy", type=int, metavar="MIB", help="run only a plain copy of MIB MiB, --steps times")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time plain copies of 8 MiB to 1 GiB (--steps launches each) and exit")
    ap.add_argument("--summarize-profile", metavar="DIR", nargs="+",
                    help="print a summary of rocprofv3 CSV output directories")
    ap.add_argument("--fetch-factor", type=float, default=1.0, help="FETCH_SIZE bytes per byte a plain copy reads")
    ap.add_argument("--write-factor", type=float, default=1.0, help="WRITE_SIZE bytes per byte a plain copy writes")
    ap.add_argument("--calls-per-run", type=int, default=1, help="calls of each entry point in the profiled run")
    ap.add_argument("--copy-bytes", type=int, default=0, help="bytes per launch of the calibration copy")
    args = ap.parse_args()
    if args.summarize_profile:
        print(summarize_profile(args.summarize_profile, args.calls_per_run, args.copy_bytes, args.fetch_factor,
                                args.write_factor))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every step works within one (sequence, KV head) and shards across GPUs "
              "by sequence or KV head with no exchange, so one GPU's throughput is the figure", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    # the host baseline first: its workers are forked, which must happen before anything touches the GPU
    cpu = None
    if args.workload in ORACLE_WORKLOADS and not args.no_cpu_baseline:
        log(f"timing the oracle on the host ({host_cores()} cores available)")
        n_seq = args.cpu_seqs or (1 if args.workload == "c3" else 2)
        cpu = cpu_baseline(args.workload, n_seq, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.0f} tokens/s on {cpu['cores']} cores, {cpu['single_core']['value']:.0f} on one")

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, args.steps)
        return
    if args.copy_ceiling:
        copy_ceiling(args.steps)
        return

    import torch

    import sparse_decode_attention_se_amd as se
    import workloads as W
    from sparse_decode_attention_se_amd import workflows as WF

    dev = "cuda:0"
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    if args.workload == "c8":
        print(json.dumps(run_policy_loop(se, WF, W, dev, status)), flush=True)
        return
    t0 = time.time()
    wl = SETUPS[args.workload](se, WF, W, dev, status, args.warmup + args.steps)
    cfg, alg = wl.cfg, wl.alg
    flush = torch.zeros(2**28, dtype=torch.float32, device=dev) if wl.restore else None
    torch.cuda.synchronize()
    log(f"{cfg.name}: inputs ready in {time.time() - t0:.1f} s, {torch.cuda.memory_allocated() / 2**30:.1f} GiB "
        f"resident")
    calls = [name for name, _ in wl.step(0)]

    def prepare():
        # outside the timed region: the pristine cache back, then the last-level cache flushed
        if wl.restore:
            wl.restore()
            flush_llc(flush)

    for i in range(args.warmup):
        prepare()
        for _, fn in wl.step(i):
            fn()
    torch.cuda.synchronize()
    require_clean_status(se, status, "the warm-up steps")
    # the warm-up steps ran with the binding's operand checks; the timed steps pass the same tensors
    se.set_operand_checks(False)
    marks = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
             for _ in range(args.steps)]
    elapsed = 0.0
    if wl.restore:
        # each step on a restored cache with a cold last-level cache; the wall time of each step is taken between
        # two device synchronisations, and the steps' times are summed
        for i in range(args.steps):
            prepare()
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for (name, fn), (e0, e1) in zip(wl.step(args.warmup + i), marks[i]):
                e0.record()
                fn()
                e1.record()
            torch.cuda.synchronize()
            elapsed += time.perf_counter() - t_start
    else:
        # the steps back to back on one evolving cache
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            for (name, fn), (e0, e1) in zip(wl.step(args.warmup + i), marks[i]):
                e0.record()
                fn()
                e1.record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    if not args.eager:
        # Per-call times: K more steps (the restored steps again, or the evolving cache's next steps), each behind
        # a device spin long enough that the host has queued the whole step before the first call starts, so that
        # the events around each call see only device time (with small calls the device would otherwise wait for
        # the host between them). A spin that ended before the host had queued the step is doubled and the step
        # run again.
        marks = per_call_marks(wl, args, prepare, calls,
                               args.warmup if wl.restore else args.warmup + args.steps)
    se.set_operand_checks(True)
    require_clean_status(se, status, "the timed steps")
    # per entry point: its time per step (summed over its calls when a step makes several, as C7's chunks do)
    per_call_ms = {}
    for j, n in enumerate(calls):
        per_call_ms[n] = per_call_ms.get(n, 0.0) + float(np.mean([m[j][0].elapsed_time(m[j][1]) for m in marks]))
    log("per call ms: " + ", ".join(f"{k} {v:.4f}" for k, v in per_call_ms.items()))
    ms_per_step = elapsed * 1e3 / args.steps

    def roof(name, bound=None):
        t = per_call_ms[name] * 1e-3
        if (bound or ("mfma" if "flops" in alg[name] else "hbm")) == "mfma":
            a = alg[name]["flops"] / t / 1e12
            return {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
        a = alg[name]["bytes"] / t / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}

    dominant = max(per_call_ms, key=per_call_ms.get)
    roofline = roof(dominant)
    roofline["kernel"] = dominant
    roofline["launches"] = CALL_KERNELS[dominant]
    roofline["traffic"] = measured_traffic(cfg.name, dominant)
    breakdown = {}
    for n in calls:
        breakdown[n] = dict(ms=round(per_call_ms[n], 4), **{k: v for k, v in roof(n, "hbm").items() if k != "bound"})
        if "flops" in alg[n]:
            breakdown[n]["mfma_tflops"] = roof(n, "mfma")["achieved"]
            breakdown[n]["mfma_frac"] = roof(n, "mfma")["frac"]
    result = {
        "metric": "KV tokens scored+compacted/s",
        "value": round(wl.tokens / (ms_per_step * 1e-3), 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "seq_len": cfg.N, "q_heads": cfg.hq, "kv_heads": cfg.hkv,
                   "head_dim": cfg.d, "page": cfg.page, "parallelism": "single GPU",
                   "timing": "each step on a restored cache after a last-level-cache flush" if wl.restore
                   else "steps back to back on one cache"},
        "roofline": roofline,
        "calls": breakdown,
    }
    if wl.restore and getattr(wl, "graph", None) is None and not args.eager:
        # One step captured as a HIP graph (a serving loop launches it that way) and replayed, each time on the
        # restored cache after a last-level-cache flush, between two device synchronisations: the line's step time
        # is the mean replay. The per-call times and the roofline above come from the eager steps.
        step_graph = capture_step(wl, args.warmup + args.steps)
        # untimed warm-up replays: a graph's first launch can carry one-off set-up work
        for i in range(max(1, args.warmup)):
            prepare()
            step_graph.replay()
        torch.cuda.synchronize()
        replays = []
        for i in range(args.steps):
            prepare()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            step_graph.replay()
            torch.cuda.synchronize()
            replays.append(time.perf_counter() - t0)
        replay_s = sum(replays)
        require_clean_status(se, status, "the graph replays")
        ms_per_step = replay_s * 1e3 / args.steps
        result["value"] = round(wl.tokens / (ms_per_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_per_step, 4)
        result["config"]["timing"] = ("each step as one captured HIP graph, replayed on a restored cache after a "
                                      f"last-level-cache flush; host-launched steps took {elapsed * 1e3 / args.steps:.4f}"
                                      " ms; per-call times from those")
        log(f"step graph: {ms_per_step:.4f} ms per replay (min {min(replays) * 1e3:.4f}, max {max(replays) * 1e3:.4f}), "
            f"host-launched {elapsed * 1e3 / args.steps:.4f} ms")
    if getattr(wl, "graph", None) is not None and not args.eager:
        # the workload's whole loop as one captured graph, replayed on the restored cache after a flush: the line's
        # step time is the replay's per decode step
        flush = torch.zeros(2**28, dtype=torch.float32, device=dev)
        wl.graph_restore()
        torch.cuda.synchronize()
        graph = wl.graph()
        replay_ms = []
        for i in range(2):  # the first replay is untimed
            wl.graph_restore()
            flush_llc(flush)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            graph.replay()
            torch.cuda.synchronize()
            replay_ms.append((time.perf_counter() - t0) * 1e3)
        require_clean_status(se, status, "the graph replays")
        n_graph = graph.steps
        ms_per_step = replay_ms[-1] / n_graph
        result["value"] = round(wl.tokens / (ms_per_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_per_step, 4)
        result["steps"], result["warmup"] = n_graph, n_graph
        result["config"]["timing"] = (f"the workload's {n_graph} decode steps as one captured HIP graph, replayed on a "
                                      f"restored cache after a last-level-cache flush ({replay_ms[-1]:.1f} ms; an "
                                      f"untimed replay first); per-call times from {args.steps} eager steps")
        log(f"graph of {n_graph} steps: replays {', '.join(f'{x:.1f}' for x in replay_ms)} ms")
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
