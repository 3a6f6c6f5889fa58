"""Oracle-side exact widening of stored values and slot addressing (test infrastructure only).

A slot s of (sequence b, KV head g) lives in physical block ``block_table[b, s // page]`` at row ``s % page``
of that block's tile for head g: the paged layout of the CacheManager (SparseEngine page, "How it works":
physical layout and position mapping are cache-manager state).
"""
import numpy as np


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly. bf16 is the upper half of a float32 bit pattern."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


def slot_rows(cache, pool: np.ndarray, b: int, g: int, slots: np.ndarray) -> np.ndarray:
    """float64 [len(slots)][d] rows of head g of sequence b at the given slots."""
    slots = np.asarray(slots, dtype=np.int64)
    blocks = cache.block_table[b, slots // cache.page]
    if np.any(blocks < 0):
        raise IndexError("slot in an unallocated block")
    return widen(pool[blocks, g, slots % cache.page], cache.dtype)


def group(g: int, r: int) -> range:
    """Query heads sharing KV head g (grouped-query attention, r query heads per KV head)."""
    return range(g * r, (g + 1) * r)
