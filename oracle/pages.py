"""Quest page metadata and page upper bounds (test infrastructure only).

SparseEngine page, "What it is" and "How it works": Quest selects pages depending on the query, at the decode
hook ``build_decode_selection``, and method metadata is kept beside the KV. The Quest workload fixes the
formulas: the metadata of a page is the elementwise minimum and maximum of its keys, and the page score is
``sum_d max(q_d * min_d, q_d * max_d)`` maximised over the query heads of the GQA group. Because each term is
at least ``q_d * k_d`` for every key of the page, the score bounds every ``q . k`` in the page from above.
"""
import numpy as np

from ._values import group, widen


def page_bounds_build(cache):
    """meta [B][n_kv][max_blocks][2][d] in storage dtype: [.., 0, :] = min, [.., 1, :] = max over the resident
    keys of each page. Pages with no resident key hold min = +inf, max = -inf (exact in both dtypes)."""
    B, n_kv = cache.n_slots.shape
    page, d = cache.page, cache.d
    f = np.float32
    meta = np.zeros((B, n_kv, cache.max_blocks, 2, d), np.float64)
    meta[:, :, :, 0, :] = np.inf
    meta[:, :, :, 1, :] = -np.inf
    for b in range(B):
        for g in range(n_kv):
            n = int(cache.n_slots[b, g])
            n_pages = -(-n // page)
            slots = np.arange(n_pages * page)
            inside = slots < n
            resident = np.zeros(slots.size, bool)
            resident[inside] = cache.pos_map[b, g, slots[inside]] >= 0
            blocks = cache.block_table[b, slots // page]
            k = widen(cache.k_pool[blocks, g, slots % page], cache.dtype).reshape(n_pages, page, d)
            keep = resident.reshape(n_pages, page, 1)
            meta[b, g, :n_pages, 0] = np.where(keep, k, np.inf).min(axis=1)
            meta[b, g, :n_pages, 1] = np.where(keep, k, -np.inf).max(axis=1)
    if cache.dtype == "f32":
        return meta.astype(f)
    # min/max of bf16 values are bf16 values: narrow exactly back to bit patterns
    return (meta.astype(f).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def page_bounds_score(cache, meta, q: np.ndarray):
    """U[b, g, p] = max over h in G(g) of sum_d max(q[b,h,d] * min[p,d], q[b,h,d] * max[p,d]).

    q: [B][hq][d] stored values. Pages past ``ceil(n_slots / page)`` and pages without resident keys score
    -inf. Returns float64 [B][n_kv][max_blocks].
    """
    B, hq, d = q.shape
    n_kv = cache.n_kv
    r = hq // n_kv
    out = np.full((B, n_kv, cache.max_blocks), -np.inf)
    for b in range(B):
        for g in range(n_kv):
            n_pages = -(-int(cache.n_slots[b, g]) // cache.page)
            lo = widen(meta[b, g, :n_pages, 0], cache.dtype)
            hi = widen(meta[b, g, :n_pages, 1], cache.dtype)
            empty = np.any(lo > hi, axis=1)
            lo = np.where(np.isfinite(lo), lo, 0.0)
            hi = np.where(np.isfinite(hi), hi, 0.0)
            best = np.full(n_pages, -np.inf)
            for h in group(g, r):
                qh = widen(q[b, h], cache.dtype)
                u = np.maximum(qh[None, :] * lo, qh[None, :] * hi).sum(axis=1)
                best = np.maximum(best, u)
            best[empty] = -np.inf
            out[b, g, :n_pages] = best
    return out
