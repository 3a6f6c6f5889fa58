"""CacheManager state changes: physical compaction, slot eviction and append (test infrastructure only).

SparseEngine page, "How it works": physical eviction updates the retained slot mapping and the context length,
then returns the discarded slots to the allocator; the CacheManager owns allocate / write / update / free.
KARA page, "Method" part 3: KvLLM compresses the trailing blocks of a sequence periodically.

Readings fixed here:
* Compaction is in place and keeps a prefix: the j-th retained slot of (b, g) moves to slot ``w0 + j`` (w0 = 0
  for a whole-cache compaction, ``n_slots - window`` for a trailing-window one), keeping its K, V, position and
  per-slot metadata (the H2O cumulative score, when the cache has one); free slots inside the compacted range
  leave the slot stack (entries below w0 stay, in order). A sequence keeps logical blocks
  ``[0, ceil(max_g n_slots / page))`` with unchanged physical ids; the blocks past that, up to the old extent,
  go to the free stack in order of sequence then logical block, and their table entries become -1.
* Slot eviction marks the slot free (position -1, metadata score 0), pushes it on the (b, g) slot stack and
  decrements the context length. Append pops that stack first, else grows the high-water mark, and takes a
  block from the free stack (sequence order) when the slot falls in a logical block the sequence lacks.
"""
import numpy as np


class CapacityError(RuntimeError):
    pass


def _extent(cache, b):
    """Number of leading allocated logical blocks of sequence b."""
    row = cache.block_table[b]
    n = 0
    while n < row.size and row[n] >= 0:
        n += 1
    return n


def compact_gather(cache, keep, window: int = 0):
    """Return a new cache where each (b, g) holds exactly its retained slots, packed in order from w0.

    keep: per (b, g) ascending, distinct slots inside ``[w0, n_slots)``. Slots at or past the new high-water
    mark get position -1 (and metadata 0); their K/V bytes are unspecified.
    """
    src = cache
    out = cache.copy()
    B, n_kv = cache.n_slots.shape
    page = cache.page
    cum = src.cum_score
    out_cum = out.cum_score
    for b in range(B):
        for g in range(n_kv):
            n = int(src.n_slots[b, g])
            w0 = n - window if window > 0 else 0
            idx = np.asarray(keep[b][g], np.int64)
            if idx.size and (idx[0] < w0 or idx[-1] >= n or np.any(np.diff(idx) <= 0)):
                raise IndexError("retained slots must be ascending, distinct and inside the compacted range")
            if np.any(src.pos_map[b, g, idx] < 0):
                raise IndexError("retained slot is not resident")
            new_n = w0 + idx.size
            dst = np.arange(w0, new_n)
            # gather from the untouched source copy: the oracle has no in-place hazard
            sb = src.block_table[b, idx // page]
            db = src.block_table[b, dst // page]
            out.k_pool[db, g, dst % page] = src.k_pool[sb, g, idx % page]
            out.v_pool[db, g, dst % page] = src.v_pool[sb, g, idx % page]
            resident_in_range = int(np.count_nonzero(src.pos_map[b, g, w0:n] >= 0))
            out.pos_map[b, g, w0:new_n] = src.pos_map[b, g, idx]
            out.pos_map[b, g, new_n:] = -1
            if out_cum is not None:
                out_cum[b, g, w0:new_n] = cum[b, g, idx]
                out_cum[b, g, new_n:] = 0.0
            out.ctx_len[b, g] = src.ctx_len[b, g] - resident_in_range + idx.size
            out.n_slots[b, g] = new_n
            # free slots inside the compacted range no longer exist: drop them from the slot stack
            stack = [int(x) for x in src.slot_stack[b, g, :src.slot_top[b, g]] if x < w0]
            out.slot_stack[b, g, :] = -1
            out.slot_stack[b, g, :len(stack)] = stack
            out.slot_top[b, g] = len(stack)
    top = int(src.free_top[0])
    for b in range(B):
        old_ext = _extent(src, b)
        new_ext = -(-int(out.n_slots[b].max()) // page)
        for lb in range(new_ext, old_ext):
            out.free_blocks[top] = src.block_table[b, lb]
            top += 1
            out.block_table[b, lb] = -1
    out.free_top[0] = top
    return out


def evict_slots(cache, evict):
    """Free the listed slots of each (b, g) (ascending order of pushing onto the slot stack)."""
    out = cache.copy()
    cum = out.cum_score
    B, n_kv = cache.n_slots.shape
    cap = cache.slot_stack.shape[2]
    for b in range(B):
        for g in range(n_kv):
            for s in np.asarray(evict[b][g], np.int64):
                if s < 0 or s >= out.n_slots[b, g] or out.pos_map[b, g, s] < 0:
                    raise IndexError("evicted slot is not resident")
                if out.slot_top[b, g] >= cap:
                    raise CapacityError("slot stack full")
                out.pos_map[b, g, s] = -1
                if cum is not None:
                    cum[b, g, s] = 0.0
                out.slot_stack[b, g, out.slot_top[b, g]] = s
                out.slot_top[b, g] += 1
                out.ctx_len[b, g] -= 1
    return out


def cache_append(cache, k_new: np.ndarray, v_new: np.ndarray, pos: np.ndarray):
    """Write one token per (b, g): k_new, v_new [B][n_kv][d] stored values, pos [B] its position; its cumulative
    score (H2O, SparseEngine page "What it is") starts at 0.

    All or nothing: if the free stack cannot supply every block the call needs, nothing changes and
    CapacityError is raised.
    """
    out = cache.copy()
    B, n_kv = cache.n_slots.shape
    page = cache.page
    max_slots = cache.pos_map.shape[2]
    slots = np.zeros((B, n_kv), np.int64)
    need = []
    for b in range(B):
        for g in range(n_kv):
            if out.slot_top[b, g] > 0:
                out.slot_top[b, g] -= 1
                slots[b, g] = out.slot_stack[b, g, out.slot_top[b, g]]
            else:
                slots[b, g] = out.n_slots[b, g]
                out.n_slots[b, g] += 1
            if slots[b, g] >= max_slots:
                raise CapacityError("sequence is at its maximum number of slots")
        missing = sorted({int(s // page) for s in slots[b] if cache.block_table[b, s // page] < 0})
        need.append(missing)
    total = sum(len(m) for m in need)
    if total > int(cache.free_top[0]):
        raise CapacityError("free stack exhausted")
    top = int(cache.free_top[0])
    for b in range(B):
        for lb in need[b]:
            top -= 1
            out.block_table[b, lb] = cache.free_blocks[top]
    out.free_top[0] = top
    for b in range(B):
        for g in range(n_kv):
            s = slots[b, g]
            blk = out.block_table[b, s // page]
            out.k_pool[blk, g, s % page] = k_new[b, g]
            out.v_pool[blk, g, s % page] = v_new[b, g]
            out.pos_map[b, g, s] = pos[b]
            out.ctx_len[b, g] += 1
            if out.cum_score is not None:  # a token just written has received no attention yet
                out.cum_score[b, g, s] = 0.0
    return out, slots


def cache_append_chunk(cache, k_new: np.ndarray, v_new: np.ndarray, pos0: np.ndarray, counts=None):
    """Write T_b tokens per (b, g) at its high-water slots [n_slots, n_slots + T_b) (SparseEngine page, "How it
    works": the cache manager allocates and writes; a prefill chunk arrives as a block of tokens): k_new, v_new
    [B][n_kv][T][d] stored values (rows t < T_b), positions pos0[b] + t, with T_b = counts[b] (all T without
    counts). The slot stacks are left alone. The logical blocks the new slots need are taken from the free stack in
    order of sequence, then logical block.

    All or nothing: if a slot range or the free stack cannot take the whole call, nothing changes and
    CapacityError is raised.
    """
    out = cache.copy()
    B, n_kv = cache.n_slots.shape
    page = cache.page
    max_slots = cache.pos_map.shape[2]
    Tb = [int(k_new.shape[2]) if counts is None else int(counts[b]) for b in range(B)]
    need = []
    for b in range(B):
        blocks = set()
        T = Tb[b]
        for g in range(n_kv):
            n = int(cache.n_slots[b, g])
            if n + T > max_slots:
                raise CapacityError("sequence is at its maximum number of slots")
            blocks |= {s // page for s in range(n, n + T)}
        need.append(sorted(lb for lb in blocks if cache.block_table[b, lb] < 0))
    if sum(len(m) for m in need) > int(cache.free_top[0]):
        raise CapacityError("free stack exhausted")
    top = int(cache.free_top[0])
    for b in range(B):
        for lb in need[b]:
            top -= 1
            out.block_table[b, lb] = cache.free_blocks[top]
    out.free_top[0] = top
    for b in range(B):
        T = Tb[b]
        for g in range(n_kv):
            n = int(cache.n_slots[b, g])
            for t in range(T):
                s = n + t
                blk = out.block_table[b, s // page]
                out.k_pool[blk, g, s % page] = k_new[b, g, t]
                out.v_pool[blk, g, s % page] = v_new[b, g, t]
                out.pos_map[b, g, s] = pos0[b] + t
                if out.cum_score is not None:
                    out.cum_score[b, g, s] = 0.0
            out.n_slots[b, g] = n + T
            out.ctx_len[b, g] += T
    return out


_PER_SEQUENCE = ("block_table", "pos_map", "ctx_len", "n_slots", "slot_stack", "slot_top", "page_meta", "cum_score")


def sequence_range(cache, b0: int, b1: int):
    """The sequences [b0, b1) as a cache of their own (KARA page, "Method" part 3: KvLLM compresses selected
    sequences). Per-sequence arrays are those sequences' rows; the block pool and the free-block stack are the
    whole cache's, since blocks are shared by every sequence."""
    sub = cache.copy()
    for f in _PER_SEQUENCE:
        x = getattr(cache, f)
        if x is not None:
            setattr(sub, f, x[b0:b1].copy())
    return sub


def put_sequence_range(cache, sub, b0: int):
    """A copy of ``cache`` with the sequences [b0, b0 + sub.B) and the shared block pool and free-block stack
    taken from ``sub`` (a cache made by sequence_range and changed since)."""
    out = cache.copy()
    b1 = b0 + sub.B
    for f in _PER_SEQUENCE:
        x = getattr(out, f)
        if x is not None:
            x[b0:b1] = getattr(sub, f)
    for f in ("k_pool", "v_pool", "free_blocks", "free_top"):
        getattr(out, f)[...] = getattr(sub, f)
    return out
