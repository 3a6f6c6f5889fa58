"""Python binding of libse (sparse KV selection, eviction and sparse decode attention on MI355X).

Every function here has the name of its C entry point in include/se.h and only marshals arguments: torch
tensors supply device memory and the current stream, and every step runs in the HIP kernels of libse.so.
Importing this package does not load the library; the first call does, and raises if it is not built.
"""
import ctypes as C

import numpy as np
import torch

from . import _lib
from ._lib import (SE_COMPACT_EVICT_SLOTS, SE_COMPACT_GATHER, SE_DEV_CAPACITY, SE_DEV_INDEX, SE_DTYPE_BF16,
                   SE_DTYPE_F32, SE_ERR_SCRATCH_LIMIT, SE_NOALLOC_SCRATCH_BYTES, SE_PAGES_BUILD, SE_PAGES_SCORE, SE_REFRESH_FROM_PAGE, SE_REFRESH_LAST_PAGE,
                   SE_SCORE_BIDIR, SE_SCORE_CAUSAL, SE_TOPK_LARGEST, SE_TOPK_SMALLEST, SE_UNIT_PAGE, SE_UNIT_SLOT)

__all__ = [
    "DeviceCache", "SEError", "se_window_score", "se_topk_select", "se_token2chunk", "se_compact_evict",
    "se_cache_append", "se_cache_append_chunk", "se_page_bounds", "se_page_bounds_refresh", "se_sparse_decode_attn",
    "se_sparse_decode_attn_noalloc", "se_h2o_decode_evict", "se_status_read",
    "se_version", "set_operand_checks", "SE_SCORE_CAUSAL", "SE_SCORE_BIDIR", "SE_TOPK_LARGEST", "SE_TOPK_SMALLEST", "SE_UNIT_SLOT",
    "SE_UNIT_PAGE", "SE_COMPACT_GATHER", "SE_COMPACT_EVICT_SLOTS", "SE_PAGES_BUILD", "SE_PAGES_SCORE",
    "SE_REFRESH_LAST_PAGE", "SE_REFRESH_FROM_PAGE", "SE_DEV_INDEX", "SE_DEV_CAPACITY",
]


class SEError(RuntimeError):
    def __init__(self, call, code):
        msg = _lib.load().se_error_string(code).decode()
        super().__init__(f"{call} failed with status {code}: {msg}")
        self.code = code


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


_CHECKS = [True]


def set_operand_checks(on):
    """Turn the binding's host-side operand checks on or off; returns the previous setting. They are on by
    default; a hot loop whose operands were checked once (same tensors, same shapes) may turn them off to save
    their Python cost per call."""
    prev = _CHECKS[0]
    _CHECKS[0] = bool(on)
    return prev


def _need(call, name, t, n, dtype, device, optional=False):
    """Host-side check of an operand before its pointer crosses the C ABI: a contiguous tensor of `dtype` on the
    cache's device holding at least `n` elements (the kernels index it that far)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{call}: {name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{call}: {name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{call}: {name} has dtype {t.dtype}, needs {dtype}")
    if t.device != device:
        raise ValueError(f"{call}: {name} is on {t.device}, the cache on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{call}: {name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{call}: {name} holds {t.numel()} elements, needs at least {n}")


def _dims(cache):
    """(B, n_kv, n_q, d, page, max_blocks, num_blocks, pool dtype, device)."""
    num_blocks, n_kv, page, d = cache.k_pool.shape
    B, max_blocks = cache.block_table.shape
    return B, n_kv, cache.n_q, d, page, max_blocks, num_blocks, cache.k_pool.dtype, cache.k_pool.device


I32, F32 = torch.int32, torch.float32


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s, C.c_void_p(s.cuda_stream)


def _check(call, rc):
    if rc != 0:
        raise SEError(call, rc)


def _workspace(nbytes, device, stream):
    if nbytes == 0:
        return None
    ws = torch.empty(int(nbytes), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


class DeviceCache:
    """The persistent cache state C (se_cache_t) as device tensors.

    Fields mirror se_cache_t: k_pool, v_pool [num_blocks][n_kv][page][d] (torch.bfloat16 or float32),
    block_table [B][max_blocks], pos_map [B][n_kv][max_blocks*page], ctx_len, n_slots [B][n_kv],
    free_blocks [num_blocks], free_top [1], slot_stack [B][n_kv][slot_cap], slot_top [B][n_kv] (int32),
    optional page_meta [B][n_kv][max_blocks][2][d] (pool dtype) and cum_score [B][n_kv][max_blocks*page] (float32).
    """

    FIELDS = ("k_pool", "v_pool", "block_table", "pos_map", "ctx_len", "n_slots", "free_blocks", "free_top",
              "slot_stack", "slot_top", "page_meta", "cum_score")

    def __init__(self, n_q, **tensors):
        for f in self.FIELDS:
            setattr(self, f, tensors.get(f))
        self.n_q = int(n_q)
        self._desc = None

    @classmethod
    def from_arrays(cls, n_q, dtype, device="cuda", **arrays):
        """Copy host numpy arrays (bf16 pools as uint16 bit patterns) to the device."""
        t = {}
        for f in cls.FIELDS:
            x = arrays.get(f)
            if x is None:
                continue
            x = np.ascontiguousarray(x)
            if f in ("k_pool", "v_pool", "page_meta") and dtype == "bf16":
                t[f] = torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
            else:
                t[f] = torch.from_numpy(x).to(device)
        return cls(n_q, **t)

    def to_numpy(self):
        out = {}
        for f in self.FIELDS:
            x = getattr(self, f)
            if x is None:
                continue
            if x.dtype == torch.bfloat16:
                out[f] = x.view(torch.int16).cpu().numpy().view(np.uint16)
            else:
                out[f] = x.cpu().numpy()
        return out

    def clone(self):
        return DeviceCache(self.n_q, **{f: (None if getattr(self, f) is None else getattr(self, f).clone())
                                        for f in self.FIELDS})

    SHARED = ("k_pool", "v_pool", "free_blocks", "free_top")

    def seq_view(self, b0, b1):
        """Sequences [b0, b1) as a cache of their own, without copying: the per-sequence tensors are views of
        those rows and the block pool and free-block stack are this cache's (blocks are shared by every
        sequence). A call on the view reads and changes those sequences alone, plus the shared pool and stack."""
        B = self.block_table.shape[0]
        if not 0 <= b0 < b1 <= B:
            raise ValueError(f"sequence range [{b0}, {b1}) outside [0, {B})")
        return DeviceCache(self.n_q, **{f: (getattr(self, f) if f in self.SHARED or getattr(self, f) is None
                                            else getattr(self, f)[b0:b1]) for f in self.FIELDS})

    @property
    def device(self):
        return self.k_pool.device

    def desc(self):
        """A fresh se_cache_t pointing at the current tensors."""
        kp = self.k_pool
        num_blocks, n_kv, page, d = kp.shape
        B, max_blocks = self.block_table.shape
        c = _lib.se_cache_t()
        for f in self.FIELDS:
            setattr(c, f, None if getattr(self, f) is None else getattr(self, f).data_ptr())
        c.B, c.n_kv, c.n_q, c.d, c.page = B, n_kv, self.n_q, d, page
        c.num_blocks, c.max_blocks = num_blocks, max_blocks
        c.slot_cap = 0 if self.slot_stack is None else self.slot_stack.shape[2]
        c.dtype = SE_DTYPE_BF16 if kp.dtype == torch.bfloat16 else SE_DTYPE_F32
        return c


# ---------------------------------------------------------------------------------------------------------------
def se_window_score(cache, q_win, q_pos, scores, *, scale, mode, n_query, window=0, protect=0, score_stride=None,
                    accumulate=False, status=None, stream=None):
    stride = score_stride if score_stride is not None else scores.shape[-1]
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_window_score"
        _need(call, "q_win", q_win, B * Hq * n_query * d, pdt, dev)
        _need(call, "q_pos", q_pos, B * n_query, I32, dev, optional=mode != SE_SCORE_CAUSAL)
        _need(call, "scores", scores, B * G * stride, F32, dev)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    p = _lib.se_window_params_t(scale, mode, n_query, window, protect, stride, int(accumulate))
    nb = lib.se_window_score_workspace_size(C.byref(c), C.byref(p))
    ws = _workspace(nb, cache.device, stream)
    _check("se_window_score", lib.se_window_score(C.byref(c), _ptr(q_win), _ptr(q_pos), C.byref(p), _ptr(scores),
                                                  _ptr(status), _ptr(ws), nb, sp))


def se_topk_select(cache, scores, idx, count, *, mode, unit, k, window=0, protect=0, forced_ends=0, budget=0,
                   recent=0, score_stride=None, out_stride=None, prune_range=None, block_refs=None,
                   emit_dropped=False, status=None, stream=None):
    sstride = score_stride if score_stride is not None else scores.shape[-1]
    ostride = out_stride if out_stride is not None else idx.shape[-1]
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_topk_select"
        _need(call, "scores", scores, B * G * sstride, F32, dev)
        _need(call, "idx", idx, B * G * ostride, I32, dev)
        _need(call, "count", count, B * G, I32, dev)
        _need(call, "block_refs", block_refs, nblk, I32, dev, optional=True)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    lo, hi = prune_range if prune_range is not None else (0, 0)
    p = _lib.se_topk_params_t(mode, unit, k, window, protect, forced_ends, budget, recent, sstride, ostride, int(lo),
                              int(hi), int(emit_dropped), _ptr(block_refs))
    nb = lib.se_topk_select_workspace_size(C.byref(c), C.byref(p))
    ws = _workspace(nb, cache.device, stream)
    _check("se_topk_select", lib.se_topk_select(C.byref(c), _ptr(scores), C.byref(p), _ptr(idx), _ptr(count),
                                                _ptr(status), _ptr(ws), nb, sp))


def se_token2chunk(cache, idx, count, scores, idx_out, count_out, *, max_gap, budget, window, protect,
                   status=None, stream=None):
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_token2chunk"
        _need(call, "idx", idx, B * G * idx.shape[-1], I32, dev)
        _need(call, "count", count, B * G, I32, dev)
        _need(call, "scores", scores, B * G * scores.shape[-1], F32, dev)
        _need(call, "idx_out", idx_out, B * G * idx_out.shape[-1], I32, dev)
        _need(call, "count_out", count_out, B * G, I32, dev)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    p = _lib.se_t2c_params_t(max_gap, budget, window, protect, scores.shape[-1], idx.shape[-1], idx_out.shape[-1])
    _check("se_token2chunk", lib.se_token2chunk(C.byref(c), _ptr(idx), _ptr(count), _ptr(scores), C.byref(p),
                                                _ptr(idx_out), _ptr(count_out), _ptr(status), None, 0, sp))


def se_compact_evict(cache, idx, count, *, mode, window=0, status=None, stream=None):
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_compact_evict"
        _need(call, "idx", idx, B * G * idx.shape[-1], I32, dev)
        _need(call, "count", count, B * G, I32, dev)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    p = _lib.se_compact_params_t(mode, window, idx.shape[-1])
    nb = lib.se_compact_evict_workspace_size(C.byref(c), C.byref(p))
    ws = _workspace(nb, cache.device, stream)
    _check("se_compact_evict", lib.se_compact_evict(C.byref(c), _ptr(idx), _ptr(count), C.byref(p), _ptr(status),
                                                    _ptr(ws), nb, sp))


def se_cache_append(cache, k_new, v_new, pos, *, status=None, stream=None):
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_cache_append"
        _need(call, "k_new", k_new, B * G * d, pdt, dev)
        _need(call, "v_new", v_new, B * G * d, pdt, dev)
        _need(call, "pos", pos, B, I32, dev)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    nb = lib.se_cache_append_workspace_size(C.byref(c))
    ws = _workspace(nb, cache.device, stream)
    _check("se_cache_append", lib.se_cache_append(C.byref(c), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(status),
                                                  _ptr(ws), nb, sp))


def se_cache_append_chunk(cache, k_new, v_new, pos0, *, counts=None, status=None, stream=None):
    """Append T tokens per (sequence, KV head) at the high-water slots (counts[b] <= T for sequence b when given);
    k_new, v_new [B][n_kv][T][d], pos0 [B]."""
    T = int(k_new.shape[2])
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_cache_append_chunk"
        _need(call, "k_new", k_new, B * G * T * d, pdt, dev)
        _need(call, "v_new", v_new, B * G * T * d, pdt, dev)
        _need(call, "pos0", pos0, B, I32, dev)
        _need(call, "counts", counts, B, I32, dev, optional=True)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    nb = lib.se_cache_append_chunk_workspace_size(C.byref(c), T)
    ws = _workspace(nb, cache.device, stream)
    _check("se_cache_append_chunk", lib.se_cache_append_chunk(C.byref(c), _ptr(k_new), _ptr(v_new), _ptr(pos0), T,
                                                              _ptr(counts), _ptr(status), _ptr(ws), nb, sp))


def se_page_bounds(cache, op, q=None, page_scores=None, *, status=None, stream=None):
    stride = 0 if page_scores is None else page_scores.shape[-1]
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_page_bounds"
        _need(call, "q", q, B * Hq * d, pdt, dev, optional=op != SE_PAGES_SCORE)
        _need(call, "page_scores", page_scores, B * G * stride, F32, dev, optional=op != SE_PAGES_SCORE)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    _check("se_page_bounds", lib.se_page_bounds(C.byref(c), op, _ptr(q), _ptr(page_scores), stride, _ptr(status),
                                                None, 0, sp))


def se_page_bounds_refresh(cache, mode, page_lo=None, max_pages=0, *, status=None, stream=None):
    """Quest metadata maintenance: BUILD's values for the last page of each unit (SE_REFRESH_LAST_PAGE) or for
    pages [page_lo[u], ceil(n_slots/page)), at most max_pages per unit (SE_REFRESH_FROM_PAGE; page_lo None =
    page 0; max_pages 0 = the block table's width)."""
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        _need("se_page_bounds_refresh", "page_lo", page_lo, B * G, I32, dev, optional=True)
        _need("se_page_bounds_refresh", "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    mp = int(max_pages) if max_pages else int(cache.block_table.shape[1])
    _check("se_page_bounds_refresh", lib.se_page_bounds_refresh(C.byref(c), int(mode), _ptr(page_lo), mp,
                                                                _ptr(status), None, 0, sp))


def se_sparse_decode_attn(cache, q, out, *, scale, sel_pages=None, sel_count=None, max_sel=0, max_slots=0,
                          accumulate=False, status=None, stream=None, ws=None):
    has_sel = sel_pages is not None
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_sparse_decode_attn"
        _need(call, "q", q, B * Hq * d, pdt, dev)
        _need(call, "out", out, B * Hq * d, F32, dev)
        _need(call, "sel_pages", sel_pages, B * G * (sel_pages.shape[-1] if has_sel else 0), I32, dev,
              optional=True)
        _need(call, "sel_count", sel_count, B * G, I32, dev, optional=not has_sel)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    p = _lib.se_decode_params_t(scale, sel_pages.shape[-1] if has_sel else 0,
                                (max_sel or sel_pages.shape[-1]) if has_sel else 0, max_slots, int(accumulate))
    nb = lib.se_sparse_decode_attn_workspace_size(C.byref(c), C.byref(p), int(has_sel))
    if ws is None:
        ws = _workspace(nb, cache.device, stream)
    elif ws.numel() * ws.element_size() < nb:
        raise ValueError(f"se_sparse_decode_attn: workspace of {ws.numel() * ws.element_size()} bytes, needs {nb}")
    _check("se_sparse_decode_attn", lib.se_sparse_decode_attn(C.byref(c), _ptr(q), _ptr(sel_pages), _ptr(sel_count),
                                                              C.byref(p), _ptr(out), _ptr(status), _ptr(ws), nb,
                                                              sp))


def se_h2o_decode_evict(cache, q, out, evict_idx, evict_count, *, scale, budget, recent, status=None, stream=None):
    """H2O's decode step after the append: accumulating decode over every resident slot, then the lowest
    cumulative score outside the recent positions is evicted (evict_idx, evict_count: [B][n_kv] int32)."""
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_h2o_decode_evict"
        _need(call, "q", q, B * Hq * d, pdt, dev)
        _need(call, "out", out, B * Hq * d, F32, dev)
        _need(call, "evict_idx", evict_idx, B * G, I32, dev)
        _need(call, "evict_count", evict_count, B * G, I32, dev)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    p = _lib.se_h2o_params_t(scale, budget, recent)
    nb = lib.se_h2o_decode_evict_workspace_size(C.byref(c), C.byref(p))
    ws = _workspace(nb, cache.device, stream)
    _check("se_h2o_decode_evict", lib.se_h2o_decode_evict(C.byref(c), _ptr(q), C.byref(p), _ptr(out), _ptr(evict_idx),
                                                          _ptr(evict_count), _ptr(status), _ptr(ws), nb, sp))


def se_sparse_decode_attn_noalloc(cache, q, out, *, scale, sel_pages=None, sel_count=None, max_sel=0, max_slots=0,
                                  accumulate=False, status=None, stream=None):
    """se_sparse_decode_attn without a workspace: the library's static per-GPU scratch array serves instead, so
    nothing is allocated (the C entry point rejects calls needing more than SE_NOALLOC_SCRATCH_BYTES)."""
    has_sel = sel_pages is not None
    if _CHECKS[0]:
        B, G, Hq, d, page, mb, nblk, pdt, dev = _dims(cache)
        call = "se_sparse_decode_attn_noalloc"
        _need(call, "q", q, B * Hq * d, pdt, dev)
        _need(call, "out", out, B * Hq * d, F32, dev)
        _need(call, "sel_pages", sel_pages, B * G * (sel_pages.shape[-1] if has_sel else 0), I32, dev,
              optional=True)
        _need(call, "sel_count", sel_count, B * G, I32, dev, optional=not has_sel)
        _need(call, "status", status, 1, I32, dev, optional=True)
    lib = _lib.load()
    st, sp = _stream(stream)
    c = cache.desc()
    p = _lib.se_decode_params_t(scale, sel_pages.shape[-1] if has_sel else 0,
                                (max_sel or sel_pages.shape[-1]) if has_sel else 0, max_slots, int(accumulate))
    _check("se_sparse_decode_attn_noalloc", lib.se_sparse_decode_attn_noalloc(
        C.byref(c), _ptr(q), _ptr(sel_pages), _ptr(sel_count), C.byref(p), _ptr(out), _ptr(status), sp))


def se_status_read(status, reset=True, stream=None):
    lib = _lib.load()
    st, sp = _stream(stream)
    v = C.c_int32(0)
    _check("se_status_read", lib.se_status_read(_ptr(status), C.byref(v), int(reset), sp))
    return v.value


def se_version():
    return _lib.load().se_version().decode()
