"""Decode attention over the view of the cache (test infrastructure only).

SparseEngine page, "How it works": for selection-based methods the CacheManager builds a view from the
persistent cache state C and the selected token or page ids I, ``View = BuildView(C, I)``, and attention runs
on it, ``o = Attention(q, View)``; logical selection only changes which resident entries attention reads.
Here the view of (b, g) is every resident slot (no selection) or the resident slots of the selected pages, and
attention is grouped-query softmax attention of each query head of the group over that view.

H2O (SparseEngine page, "What it is": continuous attention scores during generation; the H2O workload: the
softmax probabilities of each decode step are added to per-token cumulative scores kept in float32): when the
cache carries ``cum_score`` and ``accumulate`` is set, ``cum[b,g,s] += sum_{h in G(g)} p_h(s)`` with the sum
formed in float64 and the stored value rounded to float32.
"""
import numpy as np

from ._values import group, slot_rows, widen


def view_slots(cache, b: int, g: int, pages=None) -> np.ndarray:
    """Resident slots of (b, g), restricted to the listed logical pages when ``pages`` is given."""
    n = int(cache.n_slots[b, g])
    if pages is None:
        slots = np.arange(n)
    else:
        slots = np.concatenate([np.arange(p * cache.page, (p + 1) * cache.page) for p in pages] or
                               [np.zeros(0, np.int64)])
        slots = slots[slots < n]
    return slots[cache.pos_map[b, g, slots] >= 0]


def decode_attn(cache, q: np.ndarray, scale: float, pages=None, accumulate: bool = False):
    """o[b, h] = sum_{s in View(b,g)} softmax_s(scale * q[b,h] . k_s) v_s for h in G(g).

    q: [B][hq][d] stored values; pages: None or per (b, g) a list of logical page ids. Returns (o float64
    [B][hq][d], new cum_score or None). An empty view gives o = 0.
    """
    B, hq, d = q.shape
    n_kv = cache.n_kv
    r = hq // n_kv
    out = np.zeros((B, hq, d))
    cum = None
    if accumulate:
        if cache.cum_score is None:
            raise ValueError("cache has no cumulative scores")
        cum = cache.cum_score.copy()
    for b in range(B):
        for g in range(n_kv):
            slots = view_slots(cache, b, g, None if pages is None else pages[b][g])
            if slots.size == 0:
                continue
            k = slot_rows(cache, cache.k_pool, b, g, slots)
            v = slot_rows(cache, cache.v_pool, b, g, slots)
            mass = np.zeros(slots.size)
            for h in group(g, r):
                z = scale * (k @ widen(q[b, h], cache.dtype))
                e = np.exp(z - z.max())
                p = e / e.sum()
                out[b, h] = p @ v
                mass += p
            if cum is not None:
                cum[b, g, slots] = (cum[b, g, slots].astype(np.float64) + mass).astype(np.float32)
    return out, cum
