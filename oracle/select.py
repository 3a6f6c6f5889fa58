"""Retention choices: top-K candidates, H2O bottom eviction, Token2Chunk span filling (test infrastructure only).

* Top-K (KARA page, "Method" part 1 "Selection": the K most important discrete KV pairs of the window become
  retention candidates; SnapKV keeps the top keys per KV head after its observation window; Quest keeps the top
  pages). Order: score descending, ties to the lower position (lower page id for pages). Protected trailing
  slots and forced pages are always kept and are not candidates.
* Bottom eviction (H2O, SparseEngine page "What it is": continuous attention scores during generation and
  physical eviction): among resident slots outside the most recent positions, the lowest cumulative score is
  evicted when the context exceeds the budget. Ties go to the higher position (the mirror image of the
  lower-position tie-break of retention).
* Token2Chunk (KARA page, "Method" part 2): consecutive candidates in index order are the endpoints of possible
  chunks; a chunk is rated by its endpoints' importance and its length and the best ones are filled in.
  Concrete rule (the Kara workload): a gap of g = b - a - 1 slots between consecutive candidates a < b
  qualifies when 1 <= g <= max_gap; its priority is the float32 quotient (s_a + s_b) / (b - a); gaps are taken
  in priority order (ties to the lower a), a gap is filled whole when it still fits in the budget and skipped
  otherwise, until the candidate count reaches the budget.
"""
import numpy as np


def _items(cache, b, g, unit, page):
    """(item count, order key per item, resident mask) of (b, g) for slot or page units."""
    n = int(cache.n_slots[b, g])
    if unit == "slot":
        pos = cache.pos_map[b, g, :n].astype(np.int64)
        return n, pos, pos >= 0
    n_pages = -(-n // page)
    return n_pages, np.arange(n_pages, dtype=np.int64), np.ones(n_pages, bool)


def topk_largest(scores, cache, k: int, *, window: int = 0, protect: int = 0, unit: str = "slot",
                 forced_ends: bool = False, prune_range=None, block_refs=None, emit: str = "kept"):
    """Per (b, g): the k best candidates plus the always-kept items, as an ascending item list.

    Range-restricted pruning (SparseEngine page, "How it differs", sparse prefix-cache pruning: the application
    names a position range [L, R), a scoring policy keeps part of it, the mask applies to idle blocks only, and
    the resident set becomes R' = (R minus T) plus I). With ``prune_range = (L, R)`` (slot unit) a slot is a
    candidate only if its position lies in [L, R) and, when ``block_refs`` (per physical block, > 0 = busy) is
    given, its block is idle; every other resident slot is always kept. ``emit = "dropped"`` returns the
    candidates that were not chosen (the slots to free) instead of the kept list.

    scores: [B][n_kv][S] (float32 or float64). Slot unit: items are slots ``[0, n_slots)``; with ``window`` > 0
    the candidate region starts at ``base = n_slots - window`` and scores are indexed by ``slot - base``,
    otherwise base is 0 and scores are indexed by slot. The last ``protect`` slots are kept and are not
    candidates; only resident slots count. Page unit: items are pages ``[0, ceil(n_slots / page))``, scores are
    indexed by page; with ``forced_ends`` the first and last page are kept and are not candidates. If fewer than
    k candidates exist all are kept.
    """
    B, n_kv = cache.n_slots.shape
    out = []
    for b in range(B):
        row = []
        for g in range(n_kv):
            n, key, resident = _items(cache, b, g, unit, cache.page)
            if unit == "slot":
                base = n - window if window > 0 else 0
                if base < 0:
                    raise ValueError("window longer than the cache")
                cand = [i for i in range(base, n - protect) if resident[i]]
                kept = [i for i in range(max(n - protect, 0), n) if resident[i]]
                if prune_range is not None:
                    lo, hi = prune_range

                    def prunable(i):
                        if not lo <= key[i] < hi:
                            return False
                        return block_refs is None or block_refs[cache.block_table[b, i // cache.page]] == 0

                    kept = sorted(kept + [i for i in cand if not prunable(i)])
                    cand = [i for i in cand if prunable(i)]
            else:
                base = 0
                if forced_ends and n >= 2:
                    cand, kept = list(range(1, n - 1)), [0, n - 1]
                elif forced_ends:
                    cand, kept = [], list(range(n))
                else:
                    cand, kept = list(range(n)), []
            ranked = sorted(cand, key=lambda i: (-scores[b, g, i - base], key[i]))
            chosen = ranked[:min(k, len(ranked))]
            if emit == "dropped":
                row.append(np.array(sorted(ranked[len(chosen):]), np.int32))
            else:
                row.append(np.array(sorted(chosen + kept), np.int32))
        out.append(row)
    return out


def topk_smallest(scores, cache, k: int, *, budget: int, recent: int):
    """Per (b, g): slots to evict, ascending.

    Evicts ``min(k, ctx_len - budget)`` (none when within budget) of the eligible slots with the lowest score,
    ties to the higher position. Eligible: resident and ``pos <= max resident pos - recent`` (outside the most
    recent ``recent`` positions). scores: [B][n_kv][max_slots] indexed by slot.
    """
    B, n_kv = cache.n_slots.shape
    out = []
    for b in range(B):
        row = []
        for g in range(n_kv):
            n = int(cache.n_slots[b, g])
            over = int(cache.ctx_len[b, g]) - budget
            pos = cache.pos_map[b, g, :n].astype(np.int64)
            if over <= 0 or not np.any(pos >= 0):
                row.append(np.zeros(0, np.int32))
                continue
            limit = pos.max() - recent
            eligible = [s for s in range(n) if pos[s] >= 0 and pos[s] <= limit]
            ranked = sorted(eligible, key=lambda s: (scores[b, g, s], -pos[s]))
            row.append(np.array(sorted(ranked[:min(k, over)]), np.int32))
        out.append(row)
    return out


def token2chunk(lists, scores, cache, *, max_gap: int, budget: int, window: int, protect: int):
    """Fill whole gaps between consecutive candidates (see the module docstring) and return ascending lists.

    lists: per (b, g) ascending slots as returned by ``topk_largest`` for a window; entries at or beyond
    ``n_slots - protect`` are the protected tail and pass through unchanged (they are not chunk endpoints).
    scores: [B][n_kv][window - protect] float32-representable window scores indexed by ``slot - (n_slots -
    window)``. ``budget`` counts candidates plus filled slots.
    """
    out = []
    for b, row in enumerate(lists):
        new_row = []
        for g, sel in enumerate(row):
            n = int(cache.n_slots[b, g])
            base = n - window
            cand = [int(s) for s in sel if s < n - protect]
            tail = [int(s) for s in sel if s >= n - protect]
            s32 = [np.float32(scores[b, g, s - base]) for s in cand]
            gaps = []
            for i in range(len(cand) - 1):
                a, c = cand[i], cand[i + 1]
                gap = c - a - 1
                if 1 <= gap <= max_gap:
                    prio = np.float32(s32[i] + s32[i + 1]) / np.float32(c - a)
                    gaps.append((np.float32(prio), a, c))
            gaps.sort(key=lambda x: (-float(x[0]), x[1]))
            count = len(cand)
            fill = []
            for _, a, c in gaps:
                if count >= budget:
                    break
                gap = c - a - 1
                if count + gap <= budget:
                    fill.extend(range(a + 1, c))
                    count += gap
            new_row.append(np.array(sorted(cand + fill) + tail, np.int32))
        out.append(new_row)
    return out
