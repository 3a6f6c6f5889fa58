"""Host drivers that run the lifecycle steps of each method through libse, in the order the method takes them.

They stand where the SparseEngine page ("How it works") puts its SparseController hooks: SnapKV selection and
eviction after the last prompt chunk, Quest's build_decode_selection before decode attention, H2O's score
accumulation and eviction every decode step; and where the KARA page ("Method" part 3) puts KvLLM's periodic
compression of trailing blocks. Output buffers are allocated once per driver; every step is a libse call on
the current stream, and nothing here synchronises.
"""
from collections import OrderedDict

import torch

from . import (SE_COMPACT_EVICT_SLOTS, SE_COMPACT_GATHER, SE_PAGES_BUILD, SE_PAGES_SCORE, SE_REFRESH_FROM_PAGE,
               SE_REFRESH_LAST_PAGE, SE_SCORE_BIDIR, SE_SCORE_CAUSAL, SE_TOPK_LARGEST, SE_TOPK_SMALLEST, SE_UNIT_PAGE,
               SE_UNIT_SLOT, se_cache_append, se_cache_append_chunk, se_compact_evict, se_h2o_decode_evict, se_page_bounds,
               se_page_bounds_refresh, se_sparse_decode_attn, se_token2chunk, se_topk_select, se_window_score)


def _dims(cache):
    B, G, S = cache.pos_map.shape
    return B, G, S, cache.k_pool.shape[3]


class SnapKVEvent:
    """Causal window scores -> top-K + protected tail -> whole-cache compaction -> one decode step."""

    def __init__(self, cache, *, wq, protect, keep, scale, status=None):
        B, G, S, d = _dims(cache)
        dev = cache.device
        self.cache, self.wq, self.protect, self.keep, self.scale, self.status = cache, wq, protect, keep, scale, status
        self.scores = torch.zeros((B, G, S), dtype=torch.float32, device=dev)
        self.idx = torch.zeros((B, G, keep + protect), dtype=torch.int32, device=dev)
        self.count = torch.zeros((B, G), dtype=torch.int32, device=dev)
        self.out = torch.zeros((B, cache.n_q, d), dtype=torch.float32, device=dev)

    def score(self, q_win, q_pos):
        se_window_score(self.cache, q_win, q_pos, self.scores, scale=self.scale, mode=SE_SCORE_CAUSAL,
                        n_query=self.wq, status=self.status)

    def select(self):
        se_topk_select(self.cache, self.scores, self.idx, self.count, mode=SE_TOPK_LARGEST, unit=SE_UNIT_SLOT,
                       k=self.keep, protect=self.protect, status=self.status)

    def compact(self):
        se_compact_evict(self.cache, self.idx, self.count, mode=SE_COMPACT_GATHER, status=self.status)

    def decode(self, q_dec):
        se_sparse_decode_attn(self.cache, q_dec, self.out, scale=self.scale, max_slots=self.keep + self.protect,
                              status=self.status)

    def run(self, q_win, q_pos, q_dec):
        self.score(q_win, q_pos)
        self.select()
        self.compact()
        self.decode(q_dec)
        return self.out


class PruneRange:
    """Sparse prefix-cache pruning over an application's position range [L, R) (SparseEngine page, "How it
    differs"): causal window scores of the last queries -> the best `keep` slots of the range among idle blocks,
    every other resident slot kept -> the dropped slots freed onto the slot stacks (no data moves, so blocks with
    references are never written)."""

    def __init__(self, cache, *, wq, scale, status=None):
        B, G, S, d = _dims(cache)
        dev = cache.device
        self.cache, self.wq, self.scale, self.status = cache, wq, scale, status
        self.scores = torch.zeros((B, G, S), dtype=torch.float32, device=dev)
        self.drop = torch.zeros((B, G, S), dtype=torch.int32, device=dev)
        self.count = torch.zeros((B, G), dtype=torch.int32, device=dev)

    def score(self, q_win, q_pos):
        se_window_score(self.cache, q_win, q_pos, self.scores, scale=self.scale, mode=SE_SCORE_CAUSAL,
                        n_query=self.wq, status=self.status)

    def select(self, lo, hi, keep, block_refs=None):
        se_topk_select(self.cache, self.scores, self.drop, self.count, mode=SE_TOPK_LARGEST, unit=SE_UNIT_SLOT,
                       k=keep, prune_range=(lo, hi), block_refs=block_refs, emit_dropped=True, status=self.status)

    def evict(self):
        se_compact_evict(self.cache, self.drop, self.count, mode=SE_COMPACT_EVICT_SLOTS, status=self.status)

    def run(self, q_win, q_pos, lo, hi, keep, block_refs=None):
        self.score(q_win, q_pos)
        self.select(lo, hi, keep, block_refs)
        self.evict()


class H2OPrefillChunk:
    """H2O at the end of a prefill chunk (SparseEngine page, "What it is" and "How it works"): the chunk's keys and
    values are appended -> its queries add their causal attention weights to the cumulative scores -> while the
    context exceeds the budget, the lowest scores outside the most recent positions go. The cache is compacted
    after every chunk, so its last `recent` slots are the most recent positions and the choice is: keep them plus
    the best `budget - recent` of the rest (in-place gather), leaving the next chunk a dense cache to score."""

    def __init__(self, cache, *, chunk, budget, recent, scale, status=None):
        B, G, S, d = _dims(cache)
        self.cache, self.chunk, self.budget, self.recent, self.scale, self.status = (
            cache, chunk, budget, recent, scale, status)
        self.keep = torch.zeros((B, G, budget), dtype=torch.int32, device=cache.device)
        self.count = torch.zeros((B, G), dtype=torch.int32, device=cache.device)

    def append(self, k_chunk, v_chunk, pos0):
        se_cache_append_chunk(self.cache, k_chunk, v_chunk, pos0, status=self.status)

    def score(self, q_chunk, q_pos):
        se_window_score(self.cache, q_chunk, q_pos, self.cache.cum_score, scale=self.scale, mode=SE_SCORE_CAUSAL,
                        n_query=self.chunk, accumulate=True, status=self.status)

    def select(self):
        se_topk_select(self.cache, self.cache.cum_score, self.keep, self.count, mode=SE_TOPK_LARGEST,
                       unit=SE_UNIT_SLOT, k=self.budget - self.recent, protect=self.recent, status=self.status)

    def compact(self):
        se_compact_evict(self.cache, self.keep, self.count, mode=SE_COMPACT_GATHER, status=self.status)

    def run(self, q_chunk, q_pos, k_chunk=None, v_chunk=None, pos0=None):
        if k_chunk is not None:  # the first chunk of a prompt may already be in the cache
            self.append(k_chunk, v_chunk, pos0)
        self.score(q_chunk, q_pos)
        self.select()
        self.compact()


class KaraEvent:
    """Bidirectional scores of the trailing window -> top-K candidates -> Token2Chunk -> trailing compaction."""

    def __init__(self, cache, *, window, protect, n_cand, budget, max_gap, scale, status=None):
        B, G, S, d = _dims(cache)
        dev = cache.device
        self.cache, self.window, self.protect, self.n_cand, self.budget, self.max_gap = (
            cache, window, protect, n_cand, budget, max_gap)
        self.scale, self.status = scale, status
        R = window - protect
        self.scores = torch.zeros((B, G, R), dtype=torch.float32, device=dev)
        self.cand = torch.zeros((B, G, n_cand + protect), dtype=torch.int32, device=dev)
        self.cand_count = torch.zeros((B, G), dtype=torch.int32, device=dev)
        self.keep = torch.zeros((B, G, max(budget, n_cand) + protect), dtype=torch.int32, device=dev)
        self.keep_count = torch.zeros((B, G), dtype=torch.int32, device=dev)

    def run(self, q_win):
        se_window_score(self.cache, q_win, None, self.scores, scale=self.scale, mode=SE_SCORE_BIDIR,
                        n_query=self.window, window=self.window, protect=self.protect, status=self.status)
        se_topk_select(self.cache, self.scores, self.cand, self.cand_count, mode=SE_TOPK_LARGEST, unit=SE_UNIT_SLOT,
                       k=self.n_cand, window=self.window, protect=self.protect, status=self.status)
        se_token2chunk(self.cache, self.cand, self.cand_count, self.scores, self.keep, self.keep_count,
                       max_gap=self.max_gap, budget=self.budget, window=self.window, protect=self.protect,
                       status=self.status)
        se_compact_evict(self.cache, self.keep, self.keep_count, mode=SE_COMPACT_GATHER, window=self.window,
                         status=self.status)


class CompressionLoop:
    """A decode loop whose compression follows a policy (KARA page, "Method" part 3: KvLLM compresses the
    trailing blocks of selected sequences every fixed number of decode steps; "Problem" point 1: threshold-
    triggered policies compress a sequence when its cache reaches a threshold, and fire more and more often as
    concurrency grows).

    Each step appends every sequence's token and attends over its resident slots, the whole batch at once. Then
    the sequences the policy names are compressed by Kara's event (bidirectional window scores, top-K candidates,
    Token2Chunk, trailing-window compaction) on a view of each run of consecutive sequences, so the other
    sequences are not touched.
      periodic:  every sequence after every ``period``-th step (one batched event);
      threshold: sequence b joins with an uncompressed tail of (b * period) // B tokens and is compressed when
                 the tail reaches ``period`` tokens, so events of a few sequences fall at almost every step.
    The caller supplies each event's window queries (those of the sequences' ``window`` most recent tokens).
    """

    POLICIES = ("periodic", "threshold")

    def __init__(self, cache, *, policy, period, window, protect, n_cand, budget, max_gap, scale, status=None):
        if policy not in self.POLICIES:
            raise ValueError(f"policy must be one of {self.POLICIES}")
        B, G, S, d = _dims(cache)
        dev = cache.device
        self.cache, self.policy, self.period = cache, policy, int(period)
        self.window, self.protect, self.n_cand, self.budget, self.max_gap = window, protect, n_cand, budget, max_gap
        self.scale, self.status, self.B = scale, status, B
        R = window - protect
        self.scores = torch.zeros((B, G, R), dtype=torch.float32, device=dev)
        self.cand = torch.zeros((B, G, n_cand + protect), dtype=torch.int32, device=dev)
        self.cand_count = torch.zeros((B, G), dtype=torch.int32, device=dev)
        self.keep = torch.zeros((B, G, max(budget, n_cand) + protect), dtype=torch.int32, device=dev)
        self.keep_count = torch.zeros((B, G), dtype=torch.int32, device=dev)
        self.out = torch.zeros((B, cache.n_q, d), dtype=torch.float32, device=dev)

    def due(self, t):
        """Runs [b0, b1) of consecutive sequences to compress after decode step t (0-based)."""
        P, B = self.period, self.B
        if self.policy == "periodic":
            seqs = range(B) if (t + 1) % P == 0 else ()
        else:
            seqs = [b for b in range(B) if (t + 1 + (b * P) // B) % P == 0]
        runs = []
        for b in seqs:
            if runs and runs[-1][1] == b:
                runs[-1][1] = b + 1
            else:
                runs.append([b, b + 1])
        return [tuple(r) for r in runs]

    def decode(self, k_new, v_new, pos, q):
        se_cache_append(self.cache, k_new, v_new, pos, status=self.status)
        se_sparse_decode_attn(self.cache, q, self.out, scale=self.scale, status=self.status)
        return self.out

    def compress(self, b0, b1, q_win):
        """Kara's event on sequences [b0, b1); q_win [b1-b0][n_q][window][d]."""
        view = self.cache.seq_view(b0, b1)
        sc, cand, cc = self.scores[b0:b1], self.cand[b0:b1], self.cand_count[b0:b1]
        keep, kc = self.keep[b0:b1], self.keep_count[b0:b1]
        w, pr = self.window, self.protect
        se_window_score(view, q_win, None, sc, scale=self.scale, mode=SE_SCORE_BIDIR, n_query=w, window=w,
                        protect=pr, status=self.status)
        se_topk_select(view, sc, cand, cc, mode=SE_TOPK_LARGEST, unit=SE_UNIT_SLOT, k=self.n_cand, window=w,
                       protect=pr, status=self.status)
        se_token2chunk(view, cand, cc, sc, keep, kc, max_gap=self.max_gap, budget=self.budget, window=w, protect=pr,
                       status=self.status)
        se_compact_evict(view, keep, kc, mode=SE_COMPACT_GATHER, window=w, status=self.status)

    def step(self, t, k_new, v_new, pos, q, window_queries):
        """Decode step t, then the events it triggers; window_queries(b0, b1) gives an event's queries.
        Returns the step's attention output and the runs compressed."""
        out = self.decode(k_new, v_new, pos, q)
        runs = self.due(t)
        for b0, b1 in runs:
            self.compress(b0, b1, window_queries(b0, b1))
        return out, runs


class DecodeStep:
    """Append this step's token, then attend over every resident slot (optionally accumulating H2O scores)."""

    def __init__(self, cache, *, scale, accumulate=False, status=None):
        B, G, S, d = _dims(cache)
        self.cache, self.scale, self.accumulate, self.status = cache, scale, accumulate, status
        self.out = torch.zeros((B, cache.n_q, d), dtype=torch.float32, device=cache.device)

    def run(self, k_new, v_new, pos, q):
        se_cache_append(self.cache, k_new, v_new, pos, status=self.status)
        se_sparse_decode_attn(self.cache, q, self.out, scale=self.scale, accumulate=self.accumulate,
                              status=self.status)
        return self.out


class H2OStep(DecodeStep):
    """Append -> decode with cumulative scores -> evict the lowest score outside the recent positions.

    The last three are one call, se_h2o_decode_evict; with fused=False they are made as se_sparse_decode_attn,
    se_topk_select and se_compact_evict (the same results)."""

    def __init__(self, cache, *, scale, budget, recent, status=None, fused=True):
        super().__init__(cache, scale=scale, accumulate=True, status=status)
        B, G, S, d = _dims(cache)
        self.budget, self.recent, self.fused = budget, recent, fused
        self.evict = torch.zeros((B, G, 1), dtype=torch.int32, device=cache.device)
        self.evict_count = torch.zeros((B, G), dtype=torch.int32, device=cache.device)

    def run(self, k_new, v_new, pos, q):
        if self.fused:
            se_cache_append(self.cache, k_new, v_new, pos, status=self.status)
            se_h2o_decode_evict(self.cache, q, self.out, self.evict, self.evict_count, scale=self.scale,
                                budget=self.budget, recent=self.recent, status=self.status)
            return self.out
        super().run(k_new, v_new, pos, q)
        se_topk_select(self.cache, self.cache.cum_score, self.evict, self.evict_count, mode=SE_TOPK_SMALLEST,
                       unit=SE_UNIT_SLOT, k=1, budget=self.budget, recent=self.recent, status=self.status)
        se_compact_evict(self.cache, self.evict, self.evict_count, mode=SE_COMPACT_EVICT_SLOTS, status=self.status)
        return self.out


class H2OGraph:
    """H2O's decode loop captured as one HIP graph: `steps` steps of append, accumulating decode, bottom-1 and slot
    eviction (SparseEngine page, "What it is": continuous scores during generation), each with its own token, position
    and query (k_new, v_new, q, pos: sequences of per-step device tensors). One replay runs every step with no host
    launch between kernels. Capture records the kernels only; the cache is changed by replays, in stream order.

    With `record` (a list of batch indices), each step also copies that step's evicted slots [steps][B][n_kv],
    eviction counts and the recorded sequences' outputs [steps][len(record)][n_q][d] into device buffers (small
    elementwise kernels inside the graph), so a replay can be checked afterwards step by step. None of the calls
    allocates or clears memory inside the graph."""

    def __init__(self, cache, k_new, v_new, pos, q, *, scale, budget, recent, record=None, status=None):
        steps = len(q)
        B, G, S, d = _dims(cache)
        dev = cache.device
        self.step = H2OStep(cache, scale=scale, budget=budget, recent=recent, status=status)
        self.steps = steps
        self.evict = self.evict_count = self.out = None
        if record is not None:
            self.evict = torch.zeros((steps, B, G), dtype=torch.int32, device=dev)
            self.evict_count = torch.zeros((steps, B, G), dtype=torch.int32, device=dev)
            self.out = torch.zeros((steps, len(record), cache.n_q, d), dtype=torch.float32, device=dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for s in range(steps):
                self.step.run(k_new[s], v_new[s], pos[s], q[s])
                if record is not None:  # elementwise kernels, not copy engines
                    torch.add(self.step.evict[:, :, 0], 0, out=self.evict[s])
                    torch.add(self.step.evict_count, 0, out=self.evict_count[s])
                    for i, b in enumerate(record):
                        torch.add(self.step.out[b], 0, out=self.out[s, i])

    def replay(self):
        self.graph.replay()


class QuestStep:
    """Page bounds of the cache (built once) -> page scores -> top pages + first/last -> decode over them."""

    def __init__(self, cache, *, top_pages, scale, status=None):
        B, G, S, d = _dims(cache)
        dev = cache.device
        self.cache, self.top_pages, self.scale, self.status = cache, top_pages, scale, status
        nb = cache.block_table.shape[1]
        self.page_scores = torch.zeros((B, G, nb), dtype=torch.float32, device=dev)
        self.pages = torch.zeros((B, G, top_pages + 2), dtype=torch.int32, device=dev)
        self.count = torch.zeros((B, G), dtype=torch.int32, device=dev)
        self.out = torch.zeros((B, cache.n_q, d), dtype=torch.float32, device=dev)

    def build(self):
        se_page_bounds(self.cache, SE_PAGES_BUILD, status=self.status)

    def refresh_last_page(self):
        """After a high-water append: the metadata of the page it wrote."""
        se_page_bounds_refresh(self.cache, SE_REFRESH_LAST_PAGE, status=self.status)

    def refresh_from(self, page_lo=None, max_pages=0):
        """After a compaction: the metadata of pages [page_lo, end) of every unit (page_lo None = 0)."""
        se_page_bounds_refresh(self.cache, SE_REFRESH_FROM_PAGE, page_lo, max_pages, status=self.status)

    def run(self, q):
        se_page_bounds(self.cache, SE_PAGES_SCORE, q, self.page_scores, status=self.status)
        se_topk_select(self.cache, self.page_scores, self.pages, self.count, mode=SE_TOPK_LARGEST, unit=SE_UNIT_PAGE,
                       k=self.top_pages, forced_ends=1, status=self.status)
        se_sparse_decode_attn(self.cache, q, self.out, scale=self.scale, sel_pages=self.pages, sel_count=self.count,
                              status=self.status)
        return self.out


class ChainCacheIndex:
    """Cross-request reuse of an evicted cache (SparseEngine page, "How it differs": Chain Cache lets eviction
    methods reuse their compressed state across turns; ChainCacheIndex links a session to its retained KV, its
    method metadata and its logical token prefix; a request resumes from the retained state and prefills only the
    unprocessed suffix; idle chains are reclaimed in least-recently-used order).

    Host-side bookkeeping over a DeviceCache whose B sequence slots are the places sessions live. A finished
    session stays parked in its slot (retained KV, positions, cumulative scores and page metadata untouched)
    under its chain id and logical prefix. acquire() finds the parked chain whose prefix is the longest prefix of
    a request's tokens and hands back its slot; otherwise a free slot; otherwise it reclaims the least recently
    used chain: a gather that keeps nothing, on a view of the victim's sequence alone, returns its blocks to the
    free stack. The caller appends the suffix (se_cache_append_chunk) and runs the method on the slot, then parks
    it again."""

    def __init__(self, cache, status=None):
        self.cache, self.status = cache, status
        self.free = list(range(cache.block_table.shape[0]))
        self.chains = OrderedDict()  # chain id -> (slot, logical prefix), least recently used first

    def park(self, chain_id, slot, prefix):
        self.chains[chain_id] = (slot, tuple(prefix))
        self.chains.move_to_end(chain_id)
        if slot in self.free:
            self.free.remove(slot)

    def acquire(self, tokens):
        """(slot, number of tokens already in it, chain id or None) for a request with these logical tokens."""
        tokens = tuple(tokens)
        best = None
        for cid, (slot, prefix) in self.chains.items():
            if len(prefix) <= len(tokens) and tokens[:len(prefix)] == prefix:
                if best is None or len(prefix) > len(self.chains[best][1]):
                    best = cid
        if best is not None:
            slot, prefix = self.chains.pop(best)
            return slot, len(prefix), best
        if self.free:
            return self.free.pop(0), 0, None
        victim, (slot, _) = self.chains.popitem(last=False)
        self.reclaim(slot)
        return slot, 0, None

    def reclaim(self, slot):
        """Free every block of one sequence slot (its resident set becomes empty): a gather that keeps nothing,
        on a view of that sequence alone, so the other sequences are neither read nor written."""
        view = self.cache.seq_view(slot, slot + 1)
        G = view.pos_map.shape[1]
        dev = view.device
        keep = torch.zeros((1, G, 1), dtype=torch.int32, device=dev)
        count = torch.zeros((1, G), dtype=torch.int32, device=dev)
        se_compact_evict(view, keep, count, mode=SE_COMPACT_GATHER, status=self.status)
