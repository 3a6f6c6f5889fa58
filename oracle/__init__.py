"""CPU oracle for the sparse-KV hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import or call
anything in this package. The product path (the HIP library and its Python binding) never imports it and
shares no code with it; the only thing the two sides share is the seeded input generator in ``workloads.py``,
which holds none of the method's arithmetic.

What is computed follows three web pages:

* "SparseEngine ..." (onedev.kr/papers/824), section "How it works": the lifecycle contract — H2O
  cumulative-score eviction and SnapKV selection/eviction at the prefill ``finish_step`` hook, Quest's
  query-dependent page selection at ``build_decode_selection``, the CacheManager's physical eviction (slot map
  and context length updated, discarded slots returned to the allocator) versus logical selection, and the
  AttentionView ``View = BuildView(C, I)``, ``o = Attention(q, View)``.
* "KARA: Efficient Reasoning LLM Serving via Sliding-Window KV Cache Compression" (gist.science/ko/paper/
  2607.01237), section "Method": bidirectional window scoring, top-K candidates, Token2Chunk, and KvLLM's
  periodic compression of trailing blocks.
* The five benchmark workloads that make those steps concrete (formulas for SnapKV scoring, Quest page bounds,
  H2O cumulative scores and the Token2Chunk priority are only fixed there).

Arithmetic is float64 on the exact values of the stored inputs (bf16 bit patterns are widened exactly), except
where a step fixes float32: the H2O cumulative scores are float32 storage, and the Token2Chunk priority is an
IEEE float32 quotient. Every function below loops over independent (sequence, KV head) units and uses numpy
vector operations only as the textbook primitives (dot products, exp, sort).

Parity pins: see ``tests/test_oracle_pins.py`` and ``tests/test_golden.py``. No function here is "parity
unpinned".
"""
from .cache_ops import (cache_append, cache_append_chunk, compact_gather, evict_slots, put_sequence_range,
                        sequence_range)
from .decode import decode_attn
from .pages import page_bounds_build, page_bounds_refresh, page_bounds_score
from .score import window_score_bidir, window_score_causal
from .select import token2chunk, topk_largest, topk_smallest

__all__ = [
    "window_score_causal", "window_score_bidir", "topk_largest", "topk_smallest", "token2chunk",
    "compact_gather", "evict_slots", "cache_append", "cache_append_chunk", "page_bounds_build", "page_bounds_refresh",
    "page_bounds_score",
    "decode_attn", "sequence_range", "put_sequence_range",
]
