"""Observation-window attention scores (test infrastructure only).

* Causal window scoring (SnapKV at the prefill ``finish_step`` hook, SparseEngine page "How it works"; the
  formula is the one the tiny and Llama-8B workloads fix): each of the last Wq queries attends causally over
  the keys, and the softmax weights are summed per key and over the GQA group.
* Bidirectional window scoring (KARA page, "Method", part 1): every query of the window scores the keys of the
  compressible region (the window minus its protected tail) with no causal mask, and the weights are summed.
  Reading: the softmax of each query row runs over the region keys only.
"""
import numpy as np

from ._values import group, slot_rows, widen


def _softmax_rows(z: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row-wise softmax of z over the entries where mask is true; rows with no true entry are all zero."""
    z = np.where(mask, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(z - m), 0.0)
    s = e.sum(axis=1, keepdims=True)
    return np.divide(e, s, out=np.zeros_like(e), where=s > 0)


def window_score_causal(cache, q_win: np.ndarray, q_pos: np.ndarray, scale: float) -> np.ndarray:
    """scores[b, g, s] = sum over h in G(g), t in window of softmax_j(scale * q[b,h,t] . k_j)[s].

    q_win: [B][hq][Wq][d] stored values; q_pos: [B][Wq] position of each window query. Key slot s of (b, g) is
    visible to query t when it is resident (pos_map >= 0) and pos_map[s] <= q_pos[b, t]. Scores of slots that
    no query sees are zero. Returns float64 [B][n_kv][max_slots].
    """
    B, hq, Wq, d = q_win.shape
    n_kv = cache.n_kv
    r = hq // n_kv
    out = np.zeros(cache.pos_map.shape, np.float64)
    for b in range(B):
        for g in range(n_kv):
            n = int(cache.n_slots[b, g])
            if n == 0:
                continue
            slots = np.arange(n)
            pos = cache.pos_map[b, g, :n]
            resident = pos >= 0
            k = np.zeros((n, d))
            k[resident] = slot_rows(cache, cache.k_pool, b, g, slots[resident])
            visible = resident[None, :] & (pos[None, :] <= q_pos[b][:, None])
            for h in group(g, r):
                q = widen(q_win[b, h], cache.dtype)
                p = _softmax_rows(scale * (q @ k.T), visible)
                out[b, g, :n] += p.sum(axis=0)
    return out


def window_score_bidir(cache, q_win: np.ndarray, scale: float, window: int, protect: int) -> np.ndarray:
    """Bidirectional scores of the compressible region of each (b, g)'s trailing window.

    The window is the last ``window`` slots ``[w0, n)`` with ``w0 = n_slots - window``; the region is
    ``[w0, w0 + window - protect)``. q_win: [B][hq][window][d], the queries of the window's tokens in slot
    order. Every query row is a softmax over the resident region keys; weights are summed over the window's
    queries and the GQA group. Returns float64 [B][n_kv][window - protect], indexed by slot - w0.
    """
    B, hq, W, d = q_win.shape
    if W != window:
        raise ValueError("q_win must hold one query per window slot")
    R = window - protect
    n_kv = cache.n_kv
    r = hq // n_kv
    out = np.zeros((B, n_kv, R), np.float64)
    for b in range(B):
        for g in range(n_kv):
            n = int(cache.n_slots[b, g])
            w0 = n - window
            if w0 < 0:
                raise ValueError("window longer than the cache")
            slots = np.arange(w0, w0 + R)
            resident = cache.pos_map[b, g, slots] >= 0
            k = np.zeros((R, d))
            k[resident] = slot_rows(cache, cache.k_pool, b, g, slots[resident])
            mask = np.broadcast_to(resident[None, :], (W, R))
            for h in group(g, r):
                q = widen(q_win[b, h], cache.dtype)
                out[b, g] += _softmax_rows(scale * (q @ k.T), mask).sum(axis=0)
    return out
