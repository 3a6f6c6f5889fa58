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


def page_bounds_refresh(cache, meta, mode: str, page_lo=None, max_pages=None):
    """Quest metadata maintenance (SparseEngine page, "How it works": method metadata is kept beside the KV and
    follows the cache manager's writes and evictions): the metadata of the chosen pages becomes what
    ``page_bounds_build`` gives for the cache as it is now; every other page keeps its value from ``meta``.

    mode "last": page ceil(n_slots / page) - 1 of each (b, g), the page a high-water append writes (none when
    n_slots = 0). mode "from": pages [page_lo[b][g], ceil(n_slots / page)) (page_lo None = 0), at most
    ``max_pages`` of them.
    """
    full = page_bounds_build(cache)
    out = meta.copy()
    B, n_kv = cache.n_slots.shape
    for b in range(B):
        for g in range(n_kv):
            n_pages = -(-int(cache.n_slots[b, g]) // cache.page)
            if mode == "last":
                lo, hi = n_pages - 1, n_pages
            elif mode == "from":
                lo, hi = (0 if page_lo is None else int(page_lo[b][g])), n_pages
                if max_pages is not None:
                    hi = min(hi, lo + max_pages)
            else:
                raise ValueError(mode)
            lo = max(lo, 0)
            if lo < hi:
                out[b, g, lo:hi] = full[b, g, lo:hi]
    return out
