"""The five workloads run end to end on the oracle (test infrastructure only).

Each driver calls the oracle steps in the order the method takes them:

* SnapKV one-shot eviction (SparseEngine page, "How it works": selection and eviction after the last prompt
  chunk): causal window scores -> top-K + protected tail -> whole-cache compaction -> one decode step over the
  retained KV (no append: the decode query attends over the cache as it stands).
* Kara periodic compression (KARA page, "Method" parts 1-3): at an event, bidirectional window scores -> top-K
  candidates -> Token2Chunk -> trailing-window compaction; between events, decode steps that append their token
  first and then attend.
* Quest (SparseEngine page, "How it works": ``build_decode_selection``): page metadata -> page bounds -> top
  pages plus the first and last -> decode over the selected pages.
* H2O (SparseEngine page, "What it is"): per step append -> decode with cumulative-score accumulation ->
  when over budget, evict the lowest score outside the recent positions.
* The compression policy loop (KARA page, "Method" part 3, and "Problem" point 1): decode steps over the whole
  batch; after a step, Kara's event on the sequences the policy names (KvLLM's periodic schedule, or the
  threshold trigger it replaces), one event per run of consecutive sequences.
"""
import numpy as np

from .cache_ops import (cache_append, cache_append_chunk, compact_gather, evict_slots, put_sequence_range,
                        sequence_range)
from .decode import decode_attn
from .pages import page_bounds_build, page_bounds_score
from .score import window_score_bidir, window_score_causal
from .select import token2chunk, topk_largest, topk_smallest


def snapkv_event(inp):
    cfg, cache = inp["cfg"], inp["cache"]
    scores = window_score_causal(cache, inp["q_win"], inp["q_pos"], inp["scale"])
    keep = topk_largest(scores, cache, cfg.keep, protect=cfg.protect)
    compacted = compact_gather(cache, keep)
    out, _ = decode_attn(compacted, inp["q_dec"], inp["scale"])
    return dict(scores=scores, keep=keep, cache=compacted, out=out)


def kara_window_queries(inp, cache):
    """The queries of each window slot's token, [B][hq][window][d], looked up by position (harness plumbing:
    the workload keeps the query of every token since the first window)."""
    cfg = inp["cfg"]
    B, hq = cfg.B, cfg.hq
    r = hq // cfg.hkv
    q = np.zeros((B, hq, cfg.window, cfg.d), inp["q_all"].dtype)
    for b in range(B):
        for g in range(cfg.hkv):
            n = int(cache.n_slots[b, g])
            pos = cache.pos_map[b, g, n - cfg.window:n] - inp["q_first_pos"]
            if np.any(pos < 0):
                raise ValueError("window holds a token without a stored query")
            q[b, g * r:(g + 1) * r] = inp["q_all"][b, g * r:(g + 1) * r][:, pos]
    return q


def kara_event(inp, cache, keep=None):
    """Kara's event on the whole batch. ``keep`` (per (b, g)) replaces the Token2Chunk result when given: an
    equally valid choice made elsewhere where near-tied scores allow several (teacher forcing)."""
    cfg = inp["cfg"]
    q_win = kara_window_queries(inp, cache)
    scores = window_score_bidir(cache, q_win, inp["scale"], cfg.window, cfg.protect)
    cand = topk_largest(scores, cache, cfg.n_cand, window=cfg.window, protect=cfg.protect)
    scores32 = scores.astype(np.float32)
    chosen = token2chunk(cand, scores32, cache, max_gap=cfg.max_gap, budget=cfg.budget, window=cfg.window,
                         protect=cfg.protect)
    compacted = compact_gather(cache, chosen if keep is None else keep, window=cfg.window)
    keep = chosen
    return dict(q_win=q_win, scores=scores, cand=cand, keep=keep, cache=compacted)


def kara_decode_step(inp, cache, step: int):
    cfg = inp["cfg"]
    pos = np.full((cfg.B,), cfg.N + step, np.int32)
    cache, _ = cache_append(cache, inp["k_new"][step], inp["v_new"][step], pos)
    q = np.ascontiguousarray(inp["q_all"][:, :, cfg.N + step - inp["q_first_pos"]])
    out, _ = decode_attn(cache, q, inp["scale"])
    return cache, out


def quest_step(inp, cache=None):
    cfg = inp["cfg"]
    cache = inp["cache"] if cache is None else cache
    meta = page_bounds_build(cache)
    with_meta = cache.copy()
    with_meta.page_meta = meta
    pscores = page_bounds_score(with_meta, meta, inp["q_dec"])
    pages = topk_largest(pscores, with_meta, cfg.top_pages, unit="page", forced_ends=True)
    out, _ = decode_attn(with_meta, inp["q_dec"], inp["scale"], pages=pages)
    return dict(meta=meta, page_scores=pscores, pages=pages, out=out, cache=with_meta)


def h2o_step(inp, cache, step: int, evict=None):
    """One H2O decode step: append, attend with cumulative scores, evict the lowest score outside the recent
    positions. ``evict`` (per (b, g)) replaces the oracle's choice when given: an equally valid choice made
    elsewhere where near-tied cumulative scores allow several (teacher forcing); the returned ``evict`` is
    always the oracle's own."""
    cfg = inp["cfg"]
    pos = np.full((cfg.B,), cfg.N + step, np.int32)
    cache, slots = cache_append(cache, inp["k_new"][step], inp["v_new"][step], pos)
    out, cum = decode_attn(cache, inp["q_steps"][step], inp["scale"], accumulate=True)
    cache.cum_score = cum
    chosen = topk_smallest(cum, cache, 1, budget=cfg.budget, recent=cfg.recent)
    cache = evict_slots(cache, chosen if evict is None else evict)
    evict = chosen
    return cache, dict(out=out, evict=evict, slots=slots, cum=cum)


def h2o_prefill_chunk(inp, cache, c: int, keep=None):
    """Chunk c of H2O's chunked prefill (SparseEngine page, "What it is": H2O keeps cumulative attention scores and
    evicts physically; "How it works": eviction at the prefill hook). The chunk's keys and values are appended
    (the first chunk is already in the cache); the chunk's queries add their causal weights to the cumulative
    scores (float32 storage); then, while the context exceeds the budget, the lowest scores outside the most recent
    positions are evicted. The cache stays dense (compacted after every chunk), so its last ``recent`` slots are
    the most recent positions and H2O's choice is: keep those, plus the best ``budget - recent`` of the rest.
    ``keep`` replaces that choice when given (teacher forcing, as in ``h2o_step``)."""
    cfg = inp["cfg"]
    lo, hi = c * cfg.chunk, (c + 1) * cfg.chunk
    if c > 0:
        cache = cache_append_chunk(cache, inp["k_all"][:, :, lo:hi], inp["v_all"][:, :, lo:hi],
                                   np.full((cfg.B,), lo, np.int32))
    else:
        cache = cache.copy()
    q_pos = np.broadcast_to(np.arange(lo, hi, dtype=np.int32), (cfg.B, cfg.chunk))
    s = window_score_causal(cache, inp["q_all"][:, :, lo:hi], q_pos, inp["scale"])
    cache.cum_score = (cache.cum_score.astype(np.float64) + s).astype(np.float32)
    chosen = topk_largest(cache.cum_score, cache, cfg.budget - cfg.recent, protect=cfg.recent)
    cum = cache.cum_score.copy()
    cache = compact_gather(cache, chosen if keep is None else keep)
    keep = chosen
    return cache, dict(scores=s, keep=keep, cum=cum)


def kara_event_range(cache, q_win, b0: int, b1: int, *, scale, window, protect, n_cand, budget, max_gap,
                     keep=None):
    """Kara's compression event on the sequences [b0, b1) alone; every other sequence is left as it is (KARA
    page, "Method" part 3: the trailing blocks of selected sequences are compressed). q_win [b1-b0][hq][window][d]
    are the window's queries. ``keep`` (per sequence of the range, per KV head) replaces the Token2Chunk result
    when given: an equally valid choice made elsewhere where near-tied scores allow several."""
    sub = sequence_range(cache, b0, b1)
    scores = window_score_bidir(sub, q_win, scale, window, protect)
    cand = topk_largest(scores, sub, n_cand, window=window, protect=protect)
    chosen = token2chunk(cand, scores.astype(np.float32), sub, max_gap=max_gap, budget=budget, window=window,
                         protect=protect)
    sub = compact_gather(sub, chosen if keep is None else keep, window=window)
    return dict(scores=scores, cand=cand, keep=chosen, cache=put_sequence_range(cache, sub, b0))


def policy_due(policy: str, t: int, B: int, period: int):
    """Sequences compressed after decode step t (0-based).

    periodic (KvLLM, KARA page "Method" part 3): every sequence, after every ``period``-th step.
    threshold (KARA page, "Problem" point 1): sequence b joins with (b * period) // B tokens already in its
    uncompressed tail and is compressed when the tail reaches ``period`` tokens; the staggered tails make a few
    sequences reach the threshold at almost every step.
    """
    if policy == "periodic":
        return list(range(B)) if (t + 1) % period == 0 else []
    if policy == "threshold":
        return [b for b in range(B) if (t + 1 + (b * period) // B) % period == 0]
    raise ValueError(policy)


def runs_of(seqs):
    """Maximal runs [b0, b1) of consecutive sequence ids, ascending."""
    out = []
    for b in sorted(seqs):
        if out and out[-1][1] == b:
            out[-1][1] = b + 1
        else:
            out.append([b, b + 1])
    return [tuple(r) for r in out]


def kara_recent_window_queries(inp, b0: int, b1: int, t: int):
    """Queries of the ``window`` most recent tokens of sequences [b0, b1) once decode step t has appended its
    token (positions N + t + 1 - window .. N + t; t = -1 before the first step), [b1-b0][hq][window][d] (harness
    plumbing: a slice of the stored queries)."""
    cfg = inp["cfg"]
    s = cfg.N + t + 1 - cfg.window - inp["q_first_pos"]
    if s < 0:
        raise ValueError("window reaches before the first stored query")
    return np.ascontiguousarray(inp["q_all"][b0:b1, :, s:s + cfg.window])


def kara_policy_loop(inp, cache, policy: str, steps: int):
    """``steps`` decode steps of the whole batch (append, then attend); after each, Kara's event on every run of
    consecutive sequences the policy names, scored with the queries of each sequence's most recent tokens.
    Returns the final cache, the decode outputs per step and the events as (step, b0, b1)."""
    cfg = inp["cfg"]
    outs, events = [], []
    for t in range(steps):
        cache, o = kara_decode_step(inp, cache, t)
        outs.append(o)
        for b0, b1 in runs_of(policy_due(policy, t, cfg.B, cfg.period)):
            ev = kara_event_range(cache, kara_recent_window_queries(inp, b0, b1, t), b0, b1, scale=inp["scale"],
                                  window=cfg.window, protect=cfg.protect, n_cand=cfg.n_cand, budget=cfg.budget,
                                  max_gap=cfg.max_gap)
            cache = ev["cache"]
            events.append((t, b0, b1))
    return cache, outs, events
