"""Seeded synthetic workloads for the sparse-KV hot path.

This module is shared by the CPU oracle tests, the GPU parity tests and the benchmark. It holds none of the
method's arithmetic: it only draws seeded random tensors, rounds them to the storage dtype, and lays each
sequence's contiguous context out in a paged KV pool (the initial persistent cache state C of the SparseEngine
page, "How it works": CacheManager owns layout, position mapping and allocation).

Random streams: every tensor kind ``tag`` and sequence ``b`` gets its own PCG64 stream spawned from
``SeedSequence(seed, spawn_key=(tag, b))``, so a sequence can be generated alone and results do not depend on
how many threads generate them. Draws are float64; they are rounded to float32 and, for bf16 workloads, to
bf16 with round-to-nearest-even. bf16 tensors are carried as ``uint16`` bit patterns.

Initial cache state (the same for every workload):
  * sequence b owns physical blocks ``[b*nb, (b+1)*nb)`` with ``nb = ceil(N / page)``;
  * the remaining blocks are spare and sit on the free stack in descending id order, so the stack top is the
    lowest spare id;
  * ``pos_map[b, g, s] = s`` for ``s < N`` and ``-1`` beyond; ``ctx_len = n_slots = N``; slot stacks empty.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# ---------------------------------------------------------------------------------------------------------------
# dtype helpers (storage only)
# ---------------------------------------------------------------------------------------------------------------

DTYPE_F32 = 0
DTYPE_BF16 = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 draws -> storage representation (float32 array, or uint16 bf16 bits)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


# stream tags: one per tensor kind
TAG_QWIN, TAG_K, TAG_V, TAG_QDEC, TAG_SPIKE, TAG_SHIFT, TAG_ZIPF, TAG_KNEW, TAG_VNEW, TAG_SCORES, TAG_IDX = range(11)
TAG_BUSY = 11
TAG_QALL = 12


def rng_for(seed: int, tag: int, b: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag, b))))


def _pmap(fn, items, threads):
    if threads <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


# ---------------------------------------------------------------------------------------------------------------
# workload definitions
# ---------------------------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class SnapKV:
    """One-shot prefill-end eviction (the SnapKV hook after the last prompt chunk).

    The last ``wq`` queries score all causally visible keys; the last ``protect`` tokens are always kept and
    ``keep`` more are chosen from the rest; the cache is compacted in place and one decode step follows.
    """

    name: str
    B: int
    hq: int
    hkv: int
    d: int
    N: int
    wq: int
    protect: int
    keep: int
    dtype: str
    page: int = 16
    spike_frac: float = 0.0  # fraction of key positions per head given a spike
    spike_std: float = 3.0   # spike amplitude ~ N(0, spike_std^2) along a random unit direction


@dataclass(frozen=True)
class Kara:
    """Periodic sliding-window compression (KvLLM policy): every ``period`` decode steps the trailing ``window``
    slots are scored bidirectionally, candidates picked, spans filled by Token2Chunk and the trailing blocks
    compacted."""

    name: str
    B: int
    hq: int
    hkv: int
    d: int
    N: int
    window: int
    protect: int
    cand_frac: float
    budget_frac: float
    max_gap: int
    period: int
    events: int
    rho: float
    dtype: str = "bf16"
    page: int = 16

    @property
    def region(self) -> int:
        return self.window - self.protect

    @property
    def n_cand(self) -> int:
        return int(math.floor(self.cand_frac * self.region))

    @property
    def budget(self) -> int:
        return int(math.floor(self.budget_frac * self.window))

    @property
    def steps(self) -> int:
        return self.period * self.events


@dataclass(frozen=True)
class Prune:
    """Sparse prefix-cache pruning over an application's position range [range_lo, range_hi): the last ``wq``
    queries score every causally visible key (SnapKV-style policy), ``keep`` slots of the range are retained among
    the slots of idle blocks, the rest of the range's idle slots are freed. ``busy_frac`` of the physical blocks
    carry references (seeded) and are never pruned."""

    name: str
    B: int
    hq: int
    hkv: int
    d: int
    N: int
    wq: int
    range_lo: int
    range_hi: int
    keep: int
    busy_frac: float
    dtype: str = "bf16"
    page: int = 16
    spike_frac: float = 0.04
    spike_std: float = 3.0


@dataclass(frozen=True)
class H2OPrefill:
    """H2O eviction during chunked prefill: when a chunk of ``chunk`` prompt tokens has been written, the causal
    attention weights of the chunk's queries are added to the cumulative score of every key they see, and while
    the context exceeds ``budget`` the lowest-score tokens outside the most recent ``recent`` positions are
    evicted (the cache is compacted and the freed blocks returned)."""

    name: str
    B: int
    hq: int
    hkv: int
    d: int
    N: int
    chunk: int
    budget: int
    recent: int
    dtype: str = "bf16"
    page: int = 16
    spike_frac: float = 0.04
    spike_std: float = 3.0


@dataclass(frozen=True)
class Quest:
    """Query-dependent page selection decode: per-page key min/max bounds, top pages per KV head plus the first
    and last page, then decode attention over the selected pages."""

    name: str
    B: int
    hq: int
    hkv: int
    d: int
    N: int
    top_pages: int
    shift_frac: float
    shift: float
    dtype: str = "bf16"
    page: int = 16
    steps: int = 0  # decode tokens appended after the prompt (room for them in the cache, and their K/V)


@dataclass(frozen=True)
class H2O:
    """Continuous decode eviction: append, decode with cumulative score accumulation, and evict the lowest
    cumulative score outside the most recent ``recent`` positions whenever the context exceeds ``budget``."""

    name: str
    B: int
    hq: int
    hkv: int
    d: int
    N: int
    budget: int
    recent: int
    steps: int
    zipf: float
    dtype: str = "bf16"
    page: int = 16
    slot_cap: int = 16


# The five workloads at their full sizes.
C0 = SnapKV("c0_snapkv_tiny", B=1, hq=8, hkv=2, d=64, N=1024, wq=32, protect=8, keep=256, dtype="f32")
C1 = SnapKV("c1_snapkv_llama8b", B=8, hq=32, hkv=8, d=128, N=32768, wq=64, protect=64, keep=2048 - 64,
            dtype="bf16", spike_frac=0.04, spike_std=3.0)
C2 = Kara("c2_kara_qwen3_4b", B=128, hq=32, hkv=8, d=128, N=16384, window=512, protect=64, cand_frac=0.2,
          budget_frac=0.2, max_gap=8, period=128, events=1, rho=0.9)
C3 = Quest("c3_quest_128k", B=2, hq=32, hkv=8, d=128, N=131072, top_pages=256, shift_frac=0.01, shift=2.0)
C4 = H2O("c4_h2o", B=64, hq=32, hkv=8, d=128, N=8192, budget=8192, recent=256, steps=1024, zipf=1.1)
# Quest decode with its metadata kept current: C3's cache and query, each step first appending a decode token
C5 = Quest("c5_quest_128k_append", B=2, hq=32, hkv=8, d=128, N=131072, top_pages=256, shift_frac=0.01, shift=2.0,
           steps=16)
# Range-restricted pruning on C1's cache: 20% of the positions [1024, 31744) kept, 5% of the blocks busy
C6 = Prune("c6_prune_llama8b", B=8, hq=32, hkv=8, d=128, N=32768, wq=64, range_lo=1024, range_hi=31744, keep=6144,
           busy_frac=0.05)

# H2O's chunked-prefill eviction on the Llama-8B head shape: 8 x 8192 prompt tokens in chunks of 512, budget 2048
C7 = H2OPrefill("c7_h2o_prefill_llama8b", B=8, hq=32, hkv=8, d=128, N=8192, chunk=512, budget=2048, recent=256)

# KvLLM's periodic compression against a threshold trigger on C2's batch: one period of 128 decode steps, every
# sequence compressed once (all together, or each when its staggered tail reaches 128 tokens)
C8 = Kara("c8_kvllm_policy_qwen3_4b", B=128, hq=32, hkv=8, d=128, N=16384, window=512, protect=64, cand_frac=0.2,
          budget_frac=0.2, max_gap=8, period=128, events=1, rho=0.9)

FULL = {c.name: c for c in (C0, C1, C2, C3, C4, C5, C6, C7, C8)}


def scaled(cfg, **kw):
    """A smaller instance of a workload (same structure, other sizes)."""
    return replace(cfg, **kw)


# ---------------------------------------------------------------------------------------------------------------
# paged cache state
# ---------------------------------------------------------------------------------------------------------------


@dataclass
class CacheState:
    """Host copy of the persistent cache arrays (layouts match the C descriptor ``se_cache_t``)."""

    k_pool: np.ndarray      # [num_blocks][n_kv][page][d]  float32 or uint16 (bf16 bits)
    v_pool: np.ndarray      # same
    block_table: np.ndarray  # [B][max_blocks] int32, -1 = none
    pos_map: np.ndarray     # [B][n_kv][max_blocks*page] int32, -1 = free slot
    ctx_len: np.ndarray     # [B][n_kv] int32: resident tokens
    n_slots: np.ndarray     # [B][n_kv] int32: high-water slot count
    free_blocks: np.ndarray  # [num_blocks] int32 LIFO stack
    free_top: np.ndarray    # [1] int32
    slot_stack: np.ndarray  # [B][n_kv][slot_cap] int32 LIFO of reusable slots
    slot_top: np.ndarray    # [B][n_kv] int32
    page_meta: np.ndarray | None  # [B][n_kv][max_blocks][2][d] same dtype as the pools, or None
    dtype: str
    page: int
    cum_score: np.ndarray | None = None  # [B][n_kv][max_blocks*page] float32 per-slot H2O score, or None

    @property
    def B(self):
        return self.block_table.shape[0]

    @property
    def n_kv(self):
        return self.pos_map.shape[1]

    @property
    def d(self):
        return self.k_pool.shape[3]

    @property
    def max_blocks(self):
        return self.block_table.shape[1]

    @property
    def num_blocks(self):
        return self.k_pool.shape[0]

    def copy(self) -> "CacheState":
        return CacheState(**{k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in self.__dict__.items()})


def empty_cache(B, n_kv, d, page, max_blocks, num_blocks, dtype, slot_cap=16, with_meta=False,
                with_cum=False) -> CacheState:
    sd = storage_np_dtype(dtype)
    return CacheState(
        k_pool=np.zeros((num_blocks, n_kv, page, d), sd),
        v_pool=np.zeros((num_blocks, n_kv, page, d), sd),
        block_table=np.full((B, max_blocks), -1, np.int32),
        pos_map=np.full((B, n_kv, max_blocks * page), -1, np.int32),
        ctx_len=np.zeros((B, n_kv), np.int32),
        n_slots=np.zeros((B, n_kv), np.int32),
        free_blocks=np.zeros((num_blocks,), np.int32),
        free_top=np.zeros((1,), np.int32),
        slot_stack=np.full((B, n_kv, slot_cap), -1, np.int32),
        slot_top=np.zeros((B, n_kv), np.int32),
        page_meta=np.zeros((B, n_kv, max_blocks, 2, d), sd) if with_meta else None,
        dtype=dtype,
        page=page,
        cum_score=np.zeros((B, n_kv, max_blocks * page), np.float32) if with_cum else None,
    )


def layout_initial(cache: CacheState, N: int):
    """Assign blocks, positions and the free stack for a cache whose B sequences each hold N tokens."""
    page = cache.page
    nb = -(-N // page)
    B = cache.B
    if B * nb > cache.num_blocks or nb > cache.max_blocks:
        raise ValueError("pool too small for the initial context")
    for b in range(B):
        cache.block_table[b, :nb] = np.arange(b * nb, (b + 1) * nb, dtype=np.int32)
    cache.pos_map[:, :, :N] = np.arange(N, dtype=np.int32)
    cache.ctx_len[:] = N
    cache.n_slots[:] = N
    spare = np.arange(cache.num_blocks - 1, B * nb - 1, -1, dtype=np.int32)
    cache.free_blocks[: spare.size] = spare
    cache.free_top[0] = spare.size
    return nb


def write_sequence(pool: np.ndarray, nb: int, b: int, x: np.ndarray, page: int):
    """Place a contiguous [n_kv][N][d] tensor of sequence b into its initial blocks."""
    n_kv, N, d = x.shape
    pad = nb * page - N
    if pad:
        x = np.concatenate([x, np.zeros((n_kv, pad, d), x.dtype)], axis=1)
    pool[b * nb:(b + 1) * nb] = x.reshape(n_kv, nb, page, d).transpose(1, 0, 2, 3)


def gather_contiguous(cache: CacheState, which: str = "k") -> np.ndarray:
    """Read back [B][n_kv][max_slots][d] in slot order (diagnostic helper for tests; no arithmetic)."""
    pool = cache.k_pool if which == "k" else cache.v_pool
    B, n_kv, S = cache.pos_map.shape
    out = np.zeros((B, n_kv, S, cache.d), pool.dtype)
    for b in range(B):
        for lb in range(cache.max_blocks):
            pb = cache.block_table[b, lb]
            if pb >= 0:
                out[b, :, lb * cache.page:(lb + 1) * cache.page] = pool[pb]
    return out


# ---------------------------------------------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------------------------------------------


def _normal(seed, tag, b, shape):
    return rng_for(seed, tag, b).standard_normal(shape)


def gen_snapkv(cfg: SnapKV, seed: int = 0, threads: int = 8, num_blocks: int | None = None, first: int = 0) -> dict:
    """Inputs of a SnapKV-style one-shot eviction: the full cache, the window queries and one decode query. With
    ``first`` > 0 the B sequences are those numbered ``first .. first + B - 1`` of a larger batch."""
    B, hq, hkv, d, N, page = cfg.B, cfg.hq, cfg.hkv, cfg.d, cfg.N, cfg.page
    max_blocks = -(-N // page)
    num_blocks = num_blocks or B * max_blocks
    cache = empty_cache(B, hkv, d, page, max_blocks, num_blocks, cfg.dtype)
    nb = layout_initial(cache, N)
    q_win = np.stack(_pmap(lambda b: to_storage(_normal(seed, TAG_QWIN, first + b, (hq, cfg.wq, d)), cfg.dtype),
                           range(B), threads))

    def fill(b):
        k = _normal(seed, TAG_K, first + b, (hkv, N, d))
        if cfg.spike_frac > 0:
            rs = rng_for(seed, TAG_SPIKE, first + b)
            n_spike = int(round(cfg.spike_frac * N))
            for g in range(hkv):
                where = rs.choice(N, size=n_spike, replace=False)
                u = rs.standard_normal(d)
                u /= np.linalg.norm(u)
                amp = rs.normal(0.0, cfg.spike_std, size=n_spike)
                k[g, where, :] += amp[:, None] * u[None, :]
        write_sequence(cache.k_pool, nb, b, to_storage(k, cfg.dtype), page)
        v = _normal(seed, TAG_V, first + b, (hkv, N, d))
        write_sequence(cache.v_pool, nb, b, to_storage(v, cfg.dtype), page)

    _pmap(fill, range(B), threads)
    q_dec = np.stack([to_storage(_normal(seed, TAG_QDEC, first + b, (hq, d)), cfg.dtype) for b in range(B)])
    q_pos = np.broadcast_to(np.arange(N - cfg.wq, N, dtype=np.int32), (B, cfg.wq)).copy()
    return dict(cfg=cfg, cache=cache, q_win=q_win, q_pos=q_pos, q_dec=q_dec, scale=1.0 / math.sqrt(d))


def _ar1(rng: np.random.Generator, shape_lead, T, d, rho):
    """Stationary AR(1) along the token axis: x_0 ~ N(0,1), x_t = rho x_{t-1} + sqrt(1-rho^2) eps_t."""
    from scipy.signal import lfilter

    eps = rng.standard_normal(shape_lead + (T, d))
    c = math.sqrt(1.0 - rho * rho)
    eps[..., 0, :] /= c
    return lfilter([c], [1.0, -rho], eps, axis=-2)


def gen_kara(cfg: Kara, seed: int = 0, threads: int = 8, first: int = 0) -> dict:
    """Inputs of the periodic sliding-window compression workload.

    The cache starts with N tokens. ``q_all`` holds the queries of positions ``[N - window, N + steps)`` (the
    first event's window and every decode step); ``k_new``/``v_new`` hold the keys and values of the appended
    decode tokens (positions ``N .. N + steps - 1``). All are AR(1) along the token axis, per (head, dim).
    With ``first`` > 0 the B sequences are those numbered ``first .. first + B - 1`` of a larger batch (the same
    draws, since every sequence has streams of its own).
    """
    B, hq, hkv, d, N, page = cfg.B, cfg.hq, cfg.hkv, cfg.d, cfg.N, cfg.page
    T = N + cfg.steps
    max_blocks = -(-T // page)
    nb0 = -(-N // page)
    num_blocks = B * max_blocks
    cache = empty_cache(B, hkv, d, page, max_blocks, num_blocks, cfg.dtype)
    nb = layout_initial(cache, N)
    assert nb == nb0
    sd = storage_np_dtype(cfg.dtype)
    k_new = np.zeros((cfg.steps, B, hkv, d), sd)
    v_new = np.zeros((cfg.steps, B, hkv, d), sd)
    q0 = N - cfg.window
    q_all = np.zeros((B, hq, T - q0, d), sd)

    def fill(b):
        k = _ar1(rng_for(seed, TAG_K, first + b), (hkv,), T, d, cfg.rho)
        ks = to_storage(k, cfg.dtype)
        write_sequence(cache.k_pool, nb, b, np.ascontiguousarray(ks[:, :N]), page)
        k_new[:, b] = ks[:, N:].transpose(1, 0, 2)
        v = _ar1(rng_for(seed, TAG_V, first + b), (hkv,), T, d, cfg.rho)
        vs = to_storage(v, cfg.dtype)
        write_sequence(cache.v_pool, nb, b, np.ascontiguousarray(vs[:, :N]), page)
        v_new[:, b] = vs[:, N:].transpose(1, 0, 2)
        q = _ar1(rng_for(seed, TAG_QWIN, first + b), (hq,), T - q0, d, cfg.rho)
        q_all[b] = to_storage(q, cfg.dtype)

    _pmap(fill, range(B), threads)
    return dict(cfg=cfg, cache=cache, q_all=q_all, q_first_pos=q0, k_new=k_new, v_new=v_new,
                scale=1.0 / math.sqrt(d))


def gen_prune(cfg: Prune, seed: int = 0, threads: int = 8) -> dict:
    """Inputs of range-restricted pruning: the SnapKV-style cache and queries of the same shape (same draws), slot
    stacks with room for every slot, and per-block reference counts (1 on a seeded ``busy_frac`` of blocks)."""
    snap = SnapKV(cfg.name, B=cfg.B, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, N=cfg.N, wq=cfg.wq, protect=0, keep=0,
                  dtype=cfg.dtype, page=cfg.page, spike_frac=cfg.spike_frac, spike_std=cfg.spike_std)
    inp = gen_snapkv(snap, seed=seed, threads=threads)
    c = inp["cache"]
    stack = np.full((cfg.B, cfg.hkv, c.pos_map.shape[2]), -1, np.int32)
    stack[:, :, :c.slot_stack.shape[2]] = c.slot_stack
    c.slot_stack = stack
    refs = (rng_for(seed, TAG_BUSY, 0).random(c.num_blocks) < cfg.busy_frac).astype(np.int32)
    return dict(inp, cfg=cfg, block_refs=refs)


def gen_h2o_prefill(cfg: H2OPrefill, seed: int = 0, threads: int = 8) -> dict:
    """Inputs of H2O's chunked-prefill eviction: the keys and values of every prompt token ``k_all``, ``v_all``
    [B][n_kv][N][d] (the SnapKV-style draws of the same shape), the query of every prompt token ``q_all``
    [B][hq][N][d] (a stream of its own), and a cache holding the first chunk, with the other blocks on the free
    stack, cumulative scores at 0 and slot stacks with room for every slot. Later chunks are appended."""
    snap = SnapKV(cfg.name, B=cfg.B, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, N=cfg.N, wq=1, protect=0, keep=0,
                  dtype=cfg.dtype, page=cfg.page, spike_frac=cfg.spike_frac, spike_std=cfg.spike_std)
    inp = gen_snapkv(snap, seed=seed, threads=threads)
    full = inp["cache"]
    k_all = np.ascontiguousarray(gather_contiguous(full, "k")[:, :, :cfg.N])
    v_all = np.ascontiguousarray(gather_contiguous(full, "v")[:, :, :cfg.N])
    max_blocks = -(-cfg.N // cfg.page)
    S = max_blocks * cfg.page
    c = empty_cache(cfg.B, cfg.hkv, cfg.d, cfg.page, max_blocks, cfg.B * max_blocks, cfg.dtype, slot_cap=S,
                    with_cum=True)
    nb = layout_initial(c, cfg.chunk)
    for b in range(cfg.B):
        write_sequence(c.k_pool, nb, b, k_all[b, :, :cfg.chunk], cfg.page)
        write_sequence(c.v_pool, nb, b, v_all[b, :, :cfg.chunk], cfg.page)
    q_all = np.stack(_pmap(lambda b: to_storage(_normal(seed, TAG_QALL, b, (cfg.hq, cfg.N, cfg.d)), cfg.dtype),
                           range(cfg.B), threads))
    return dict(cfg=cfg, cache=c, k_all=k_all, v_all=v_all, q_all=q_all, q_dec=inp["q_dec"], scale=inp["scale"])


def gen_quest(cfg: Quest, seed: int = 0, threads: int = 8, first: int = 0) -> dict:
    """Inputs of the Quest-style workload: a full cache with a fraction of pages shifted along the group's query
    direction, page metadata storage, and one decode query per sequence. With ``cfg.steps`` > 0 the cache has
    room for that many appended tokens, whose keys and values (``k_new``, ``v_new`` [steps][B][n_kv][d], i.i.d.
    N(0,1)) are drawn from streams of their own, so the prompt's draws do not change. With ``first`` > 0 the B
    sequences are those numbered ``first .. first + B - 1`` of a larger batch."""
    B, hq, hkv, d, N, page = cfg.B, cfg.hq, cfg.hkv, cfg.d, cfg.N, cfg.page
    max_blocks = -(-(N + cfg.steps) // page)
    cache = empty_cache(B, hkv, d, page, max_blocks, B * max_blocks, cfg.dtype, with_meta=True)
    nb = layout_initial(cache, N)
    r = hq // hkv
    q64 = [_normal(seed, TAG_QDEC, first + b, (hq, d)) for b in range(B)]
    q_dec = np.stack([to_storage(q, cfg.dtype) for q in q64])
    n_shift = int(round(cfg.shift_frac * nb))

    def fill(b):
        k = _normal(seed, TAG_K, first + b, (hkv, N, d))
        rs = rng_for(seed, TAG_SHIFT, first + b)
        for g in range(hkv):
            pages = rs.choice(nb, size=n_shift, replace=False)
            direction = q64[b][g * r:(g + 1) * r].sum(axis=0)
            direction /= np.linalg.norm(direction)
            for p in pages:
                k[g, p * page:min((p + 1) * page, N), :] += cfg.shift * direction
        write_sequence(cache.k_pool, nb, b, to_storage(k, cfg.dtype), page)
        v = _normal(seed, TAG_V, first + b, (hkv, N, d))
        write_sequence(cache.v_pool, nb, b, to_storage(v, cfg.dtype), page)

    _pmap(fill, range(B), threads)
    out = dict(cfg=cfg, cache=cache, q_dec=q_dec, scale=1.0 / math.sqrt(d))
    if cfg.steps:
        out["k_new"] = np.stack([to_storage(_normal(seed, TAG_KNEW, first + b, (cfg.steps, hkv, d)), cfg.dtype)
                                 for b in range(B)], axis=1)
        out["v_new"] = np.stack([to_storage(_normal(seed, TAG_VNEW, first + b, (cfg.steps, hkv, d)), cfg.dtype)
                                 for b in range(B)], axis=1)
    return out


def gen_h2o(cfg: H2O, seed: int = 0, threads: int = 8, first: int = 0) -> dict:
    """Inputs of the H2O continuous-eviction workload.

    Keys of every token (initial context and the ``steps`` appended ones) carry a per-sequence Zipf key-norm
    scale: a seeded permutation gives token t the rank rho_t in 1..N+steps, the scale is rho_t^-zipf normalised
    to unit RMS over the sequence, shared by all heads. With ``first`` > 0 the B sequences are those numbered
    ``first .. first + B - 1`` of a larger batch.
    """
    B, hq, hkv, d, N, page = cfg.B, cfg.hq, cfg.hkv, cfg.d, cfg.N, cfg.page
    T = N + cfg.steps
    # at most max(N, budget) + 1 slots are ever used: evicted slots are reused by the next append
    max_blocks = -(-(max(N, cfg.budget) + 1) // page)
    num_blocks = B * max_blocks
    cache = empty_cache(B, hkv, d, page, max_blocks, num_blocks, cfg.dtype, slot_cap=cfg.slot_cap, with_cum=True)
    nb = layout_initial(cache, N)
    sd = storage_np_dtype(cfg.dtype)
    k_new = np.zeros((cfg.steps, B, hkv, d), sd)
    v_new = np.zeros((cfg.steps, B, hkv, d), sd)

    def fill(b):
        k = _normal(seed, TAG_K, first + b, (hkv, T, d))
        rank = rng_for(seed, TAG_ZIPF, first + b).permutation(T) + 1
        s = rank.astype(np.float64) ** (-cfg.zipf)
        s /= math.sqrt(float(np.mean(s * s)))
        k *= s[None, :, None]
        ks = to_storage(k, cfg.dtype)
        write_sequence(cache.k_pool, nb, b, np.ascontiguousarray(ks[:, :N]), page)
        k_new[:, b] = ks[:, N:].transpose(1, 0, 2)
        v = to_storage(_normal(seed, TAG_V, first + b, (hkv, T, d)), cfg.dtype)
        write_sequence(cache.v_pool, nb, b, np.ascontiguousarray(v[:, :N]), page)
        v_new[:, b] = v[:, N:].transpose(1, 0, 2)

    _pmap(fill, range(B), threads)
    q_steps = np.stack([np.stack([to_storage(x, cfg.dtype) for x in
                                  _normal(seed, TAG_QDEC, first + b, (cfg.steps, hq, d))]) for b in range(B)], axis=1)
    return dict(cfg=cfg, cache=cache, q_steps=q_steps, k_new=k_new, v_new=v_new, scale=1.0 / math.sqrt(d))


# ---------------------------------------------------------------------------------------------------------------
# stage-isolated inputs (for testing one call alone)
# ---------------------------------------------------------------------------------------------------------------


def gen_scores(seed: int, shape, tie_frac: float = 0.0, levels: int = 0) -> np.ndarray:
    """float32 scores, optionally quantised to ``levels`` distinct values (many exact ties) and/or with a fraction
    of entries copied from another entry (exact duplicates)."""
    rs = rng_for(seed, TAG_SCORES)
    x = rs.random(shape)
    if levels:
        x = np.floor(x * levels) / levels
    x = x.astype(np.float32)
    if tie_frac > 0:
        flat = x.reshape(-1, x.shape[-1])
        for row in flat:
            m = int(tie_frac * row.size)
            src = rs.integers(0, row.size, m)
            dst = rs.integers(0, row.size, m)
            row[dst] = row[src]
    return x


def gen_keep_sets(seed: int, n_slots: np.ndarray, count: np.ndarray, lo: np.ndarray | None = None,
                  pattern: str = "random") -> list:
    """Ascending slot lists to keep, one per (b, g): ``count[b,g]`` distinct slots from ``[lo, n_slots)``.

    Patterns: ``random``, ``prefix`` (lo, lo+1, ...), ``shift1`` (lo+1, lo+2, ...: every slot moves by one),
    ``tail`` (the last ``count`` slots)."""
    rs = rng_for(seed, TAG_IDX)
    B, G = n_slots.shape
    out = []
    for b in range(B):
        row = []
        for g in range(G):
            a = int(lo[b, g]) if lo is not None else 0
            n, c = int(n_slots[b, g]), int(count[b, g])
            if pattern == "random":
                sel = np.sort(rs.choice(np.arange(a, n), size=c, replace=False))
            elif pattern == "prefix":
                sel = np.arange(a, a + c)
            elif pattern == "shift1":
                sel = np.arange(a + 1, a + 1 + c)
            elif pattern == "tail":
                sel = np.arange(n - c, n)
            else:
                raise ValueError(pattern)
            row.append(sel.astype(np.int32))
        out.append(row)
    return out


def pack_lists(lists, stride: int):
    """[B][G] lists -> (idx [B][G][stride] int32 padded with -1, count [B][G] int32)."""
    B, G = len(lists), len(lists[0])
    idx = np.full((B, G, stride), -1, np.int32)
    cnt = np.zeros((B, G), np.int32)
    for b in range(B):
        for g in range(G):
            x = lists[b][g]
            idx[b, g, :len(x)] = x
            cnt[b, g] = len(x)
    return idx, cnt
