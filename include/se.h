/*
 * se.h — sparse KV selection, eviction and sparse decode attention on MI355X (gfx950).
 *
 * C ABI of libse.so. The calls follow the lifecycle contract of the SparseEngine page
 * (onedev.kr/papers/824, section "How it works"): a persistent cache state C owned by a cache manager
 * (KV layout, position mapping, allocate / write / update / free, metadata kept beside the KV), a set of
 * selected token or page ids I, a view View = BuildView(C, I) and o = Attention(q, View). Here C is an
 * se_cache_t, I is an (idx, count) pair, BuildView is implicit in passing both to se_sparse_decode_attn.
 *
 * Conventions shared by every call
 *  - Every pointer in a descriptor or argument is a DEVICE pointer unless stated otherwise; descriptor and
 *    parameter structs themselves are host memory and are read before the call returns. The caller owns all
 *    memory: pools, maps, scores, index lists, outputs and workspaces. The library allocates nothing and keeps
 *    no per-cache state.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream) and mutates its outputs
 *    in stream order. Calls on different streams must not touch the same buffers concurrently.
 *  - Return value: SE_OK, or a host-detected error (SE_ERR_*) in which case nothing was launched.
 *  - Errors only the device can see (bad indices, exhausted free lists) are OR-ed into the caller's sticky
 *    device word `status` (may be NULL to ignore them) as SE_DEV_* bits; read it with se_status_read.
 *  - `ws`/`ws_bytes`: caller-provided device workspace of at least the size the matching *_workspace_size
 *    function reports (NULL/0 when it reports 0). Its contents need not be initialised and are clobbered.
 *
 * Paged cache layout (se_cache_t): K and V live in pools of physical blocks; block p holds, for every KV
 * head g, `page` consecutive slots of `d` elements: k_pool[p][g][i][e]. A sequence b maps logical block L to
 * physical block block_table[b][L] (-1 = none; allocated entries form a prefix). Slot s of (b, g) is row
 * s % page of block block_table[b][s / page]. pos_map[b][g][s] is the original token position held in slot s
 * (-1 = free). Slots at or beyond n_slots[b][g] are unused (their pos_map entries are unspecified). Inside
 * [0, n_slots) the free slots are exactly the entries of the (b, g) slot stack, and ctx_len counts the
 * resident ones. All calls keep these invariants.
 */
#ifndef SE_H
#define SE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------------------------------ */
enum {
  SE_OK = 0,
  SE_ERR_NULL = 1,        /* a required pointer is NULL */
  SE_ERR_SHAPE = 2,       /* sizes that do not fit together (strides, dims, group size) */
  SE_ERR_DTYPE = 3,       /* unsupported element type or head dimension */
  SE_ERR_PARAM = 4,       /* a parameter outside its domain */
  SE_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  SE_ERR_UNSUPPORTED = 6, /* a combination the library does not implement */
  SE_ERR_HIP = 7,         /* a HIP runtime call failed */
  SE_ERR_SCRATCH_LIMIT = 8, /* the call needs more scratch than the allocation-free entry point holds */
  /* device status bits, OR-ed into *status */
  SE_DEV_INDEX = 1 << 8,    /* an index list entry out of range, unsorted, duplicated or not resident */
  SE_DEV_CAPACITY = 1 << 9  /* free block stack, slot stack or slot range exhausted */
};

enum { SE_DTYPE_F32 = 0, SE_DTYPE_BF16 = 1 };

typedef void *se_stream_t; /* a hipStream_t */

/* ---- the persistent cache state C ------------------------------------------------------------------------ */
typedef struct se_cache {
  void *k_pool, *v_pool;  /* [num_blocks][n_kv][page][d] of dtype */
  int32_t *block_table;   /* [B][max_blocks] physical block id, -1 = none */
  int32_t *pos_map;       /* [B][n_kv][max_blocks * page] original position, -1 = free slot */
  int32_t *ctx_len;       /* [B][n_kv] resident tokens */
  int32_t *n_slots;       /* [B][n_kv] high-water slot count */
  int32_t *free_blocks;   /* [num_blocks] LIFO stack of free physical blocks */
  int32_t *free_top;      /* [1] number of entries on free_blocks */
  int32_t *slot_stack;    /* [B][n_kv][slot_cap] LIFO of free slots below n_slots (may be NULL if slot_cap = 0) */
  int32_t *slot_top;      /* [B][n_kv] entries on each slot stack (may be NULL if slot_cap = 0) */
  void *page_meta;        /* optional [B][n_kv][max_blocks][2][d] of dtype: per-page key min ([..][0][..]) and
                             max ([..][1][..]) (Quest metadata) */
  float *cum_score;       /* optional [B][n_kv][max_blocks * page] per-slot cumulative attention (H2O metadata) */
  int32_t B, n_kv, n_q, d, page, num_blocks, max_blocks, slot_cap, dtype;
} se_cache_t;

/* ---- window scores ------------------------------------------------------------------------------------------
 * SnapKV observation-window scoring (SparseEngine page, "How it works": selection after the last prompt
 * chunk) and Kara's bidirectional window scoring (KARA page, gist.science/ko/paper/2607.01237, "Method"
 * part 1). For every KV head g of sequence b and every query head h of its group (h / (n_q / n_kv) == g):
 *   CAUSAL: q_win [B][n_q][n_query][d] are the queries of the window tokens, q_pos [B][n_query] their
 *     positions. Each query row is a softmax over the resident slots s < n_slots with pos_map[s] <= q_pos.
 *     scores[(b*n_kv+g)*score_stride + s] = sum over h, t of that row's weight on s, for s < n_slots
 *     (0 where no query sees the slot).
 *   BIDIR: the window is the last `window` slots [w0, n_slots), w0 = n_slots - window, and the region its first
 *     window - protect slots. q_win [B][n_q][window][d] holds the queries of the window's tokens; q_pos is
 *     unused. Each query row is a softmax over the resident region slots (no mask);
 *     scores[(b*n_kv+g)*score_stride + (s - w0)] for s in the region. A unit with n_slots < window raises
 *     SE_DEV_INDEX and its scores are not written.
 *   Nothing outside these entries is written.
 * accumulate != 0: every score is added to the value the output already holds instead of replacing it, so with
 *   scores = cum_score (score_stride = max_blocks * page) the causal scores of a prefill chunk's queries are added to
 *   H2O's cumulative scores (SparseEngine page, "What it is": H2O keeps cumulative attention scores).
 * Arithmetic: products of stored values exact, fp32 accumulation, fp32 output.
 * Errors: SE_ERR_UNSUPPORTED when num_blocks * n_kv * page >= 2^31 (pool rows are addressed with 32-bit ids).
 */
enum { SE_SCORE_CAUSAL = 0, SE_SCORE_BIDIR = 1 };
typedef struct {
  float scale;          /* logit scale, usually 1/sqrt(d) */
  int32_t mode;         /* SE_SCORE_CAUSAL or SE_SCORE_BIDIR */
  int32_t n_query;      /* queries per (sequence, head) in q_win; BIDIR requires n_query == window */
  int32_t window;       /* BIDIR only */
  int32_t protect;      /* BIDIR only: trailing window slots outside the key region */
  int32_t score_stride; /* floats between consecutive (b, g) rows of scores */
  int32_t accumulate;   /* 0: scores = the window's scores; else scores += them */
} se_window_params_t;

size_t se_window_score_workspace_size(const se_cache_t *c, const se_window_params_t *p);
int32_t se_window_score(const se_cache_t *c, const void *q_win, const int32_t *q_pos, const se_window_params_t *p,
                        float *scores, int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- top-K retention / bottom eviction ---------------------------------------------------------------------
 * KARA page "Method" part 1 (top-K discrete pairs become candidates), SparseEngine page "How it works"
 * (SnapKV selection; Quest build_decode_selection) and "What it is" (H2O eviction by continuous scores).
 * Output per (b, g): idx[(b*n_kv+g)*out_stride + i], i < count[b*n_kv+g], ascending item ids.
 *  LARGEST / SLOT: items are slots. Candidates are the resident slots of [base, n_slots - protect), with base = 0
 *    (scores indexed by slot) or, if window > 0, base = n_slots - window (scores indexed by slot - base; a
 *    window longer than n_slots raises SE_DEV_INDEX and gives count 0). The min(k, #candidates) best by
 *    (score desc, position asc) are returned together with the resident slots of the protected tail
 *    [n_slots - protect, n_slots).
 *  LARGEST / PAGE: items are logical pages [0, ceil(n_slots/page)), scores indexed by page. With forced_ends
 *    the first and last page are always returned and are not candidates. Order (score desc, page asc).
 *  SMALLEST / SLOT: if ctx_len > budget, returns min(k, ctx_len - budget) slots with the lowest score among the
 *    resident slots whose position is <= (max resident position - recent); order (score asc, position desc).
 *    Otherwise count = 0.
 *  Range-restricted pruning (LARGEST / SLOT; SparseEngine page, "How it differs", sparse prefix-cache pruning:
 *    the application names a 0-based position range [L, R), a scoring policy keeps part of it, the mask applies
 *    to idle blocks only and the resident set becomes R' = (R minus T) plus I): with range_hi > range_lo a
 *    resident slot is a candidate only if range_lo <= position < range_hi and, when block_refs is given (device
 *    [num_blocks], > 0 = the block has active references or transfers), its physical block is idle. Every other
 *    resident slot of the region is kept. emit_dropped != 0 returns the candidates that were not chosen, ascending
 *    (the list SE_COMPACT_EVICT_SLOTS frees) instead of the kept list. Needs out_stride >= the item count.
 *    block_refs needs a range; range and emit_dropped need LARGEST / SLOT (else SE_ERR_PARAM).
 * Scores must not be NaN.
 */
enum { SE_TOPK_LARGEST = 0, SE_TOPK_SMALLEST = 1 };
enum { SE_UNIT_SLOT = 0, SE_UNIT_PAGE = 1 };
typedef struct {
  int32_t mode, unit, k;
  int32_t window, protect; /* LARGEST / SLOT */
  int32_t forced_ends;     /* LARGEST / PAGE */
  int32_t budget, recent;  /* SMALLEST */
  int32_t score_stride, out_stride;
  int32_t range_lo, range_hi, emit_dropped; /* range-restricted pruning (0, 0, 0: off) */
  const int32_t *block_refs;                /* NULL: every block idle */
} se_topk_params_t;

size_t se_topk_select_workspace_size(const se_cache_t *c, const se_topk_params_t *p);
int32_t se_topk_select(const se_cache_t *c, const float *scores, const se_topk_params_t *p, int32_t *idx,
                       int32_t *count, int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- Token2Chunk -------------------------------------------------------------------------------------------
 * KARA page, "Method" part 2. Input per (b, g): an ascending slot list (as returned by se_topk_select with a
 * window): entries below n_slots - protect are the candidates c_1 < ... < c_m, the rest the protected tail.
 * For consecutive candidates a < b with 1 <= b - a - 1 <= max_gap the gap's priority is the IEEE fp32 quotient
 * (s_a + s_b) / (b - a), s read from scores[(b*n_kv+g)*score_stride + (slot - (n_slots - window))]. Gaps are
 * taken by priority (ties: lower a); a gap is filled whole if the count of candidates plus filled slots stays
 * <= budget, otherwise skipped; filling stops at the budget. Output: ascending candidates and fills, then the
 * tail.
 */
typedef struct {
  int32_t max_gap, budget, window, protect;
  int32_t score_stride, in_stride, out_stride;
} se_t2c_params_t;

int32_t se_token2chunk(const se_cache_t *c, const int32_t *idx, const int32_t *count, const float *scores,
                       const se_t2c_params_t *p, int32_t *idx_out, int32_t *count_out, int32_t *status, void *ws,
                       size_t ws_bytes, se_stream_t stream);

/* ---- physical compaction and slot eviction ------------------------------------------------------------------
 * SparseEngine page, "How it works": physical eviction updates the retained slot mapping and the context
 * length and returns discarded slots to the allocator. KARA page, "Method" part 3: trailing blocks are
 * compacted periodically.
 *  GATHER: per (b, g) the ascending, distinct, resident slots idx[..][0..count) inside [w0, n_slots) are kept,
 *    w0 = 0 (window = 0) or n_slots - window. The j-th moves to slot w0 + j with its K, V, position and (if
 *    present) cumulative score; n_slots = w0 + count; ctx_len drops the window's other resident slots; free
 *    slots at or above w0 leave the slot stack. Sequence b keeps logical blocks [0, ceil(max_g n_slots / page))
 *    (same physical ids); the rest of its allocated blocks are pushed on free_blocks in order of sequence, then
 *    logical block, and their table entries become -1. In place; bit-exact.
 *  EVICT_SLOTS: per (b, g) each listed resident slot is freed: position -1, cumulative score 0, pushed on the
 *    slot stack (in list order), ctx_len - 1. No data moves. The list must be ascending and distinct (as
 *    se_topk_select returns it); an entry that is out of order, out of range or not resident raises SE_DEV_INDEX
 *    and is skipped; entries beyond the slot stack's capacity are not evicted and raise SE_DEV_CAPACITY.
 * GATHER needs a workspace of se_compact_evict_workspace_size bytes ((2 B + 1) int32, rounded up); EVICT_SLOTS
 * needs none.
 */
enum { SE_COMPACT_GATHER = 0, SE_COMPACT_EVICT_SLOTS = 1 };
typedef struct {
  int32_t mode, window, idx_stride;
} se_compact_params_t;

size_t se_compact_evict_workspace_size(const se_cache_t *c, const se_compact_params_t *p);
int32_t se_compact_evict(se_cache_t *c, const int32_t *idx, const int32_t *count, const se_compact_params_t *p,
                         int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- append one decode token per (sequence, KV head) --------------------------------------------------------
 * CacheManager allocate/write (SparseEngine page, "How it works"). Per (b, g): the slot is popped from the
 * slot stack if it is not empty, else slot = n_slots++. When a slot lies in a logical block sequence b lacks,
 * one block is popped from free_blocks for it (pops in sequence order). k_new, v_new [B][n_kv][d] of dtype are
 * written, pos_map = pos[b] (pos: device [B]), ctx_len + 1, and the cumulative score (if present) set to 0. All or
 * nothing: if the free stack or a sequence's slot range cannot serve the whole call, nothing changes and
 * SE_DEV_CAPACITY is raised. Workspace: se_cache_append_workspace_size bytes (one int32 per (sequence, KV head):
 * the pool row each new token goes to, handed from the planning kernel to the copying one).
 */
size_t se_cache_append_workspace_size(const se_cache_t *c);
int32_t se_cache_append(se_cache_t *c, const void *k_new, const void *v_new, const int32_t *pos, int32_t *status,
                        void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- append a chunk of tokens per (sequence, KV head) -------------------------------------------------------
 * CacheManager allocate/write for a prefill chunk (SparseEngine page, "How it works"). Sequence b appends
 * T_b = counts[b] tokens (counts: device [B], each in [0, T]; NULL = T for every sequence). Per (b, g) they take
 * the slots [n_slots, n_slots + T_b) (the high-water mark; freed slots on the slot stack are left for single-
 * token appends): k_new, v_new [B][n_kv][T][d] of dtype (rows t < T_b are read) are written there,
 * pos_map = pos0[b] + t (pos0: device [B]), cumulative scores (if present) 0, n_slots and ctx_len + T_b. Logical blocks the new slots need beyond a
 * sequence's allocated prefix are popped from free_blocks in order of sequence, then logical block. All or
 * nothing: if the free stack or a unit's slot range cannot take the whole call (or a count is outside [0, T]),
 * nothing changes and SE_DEV_CAPACITY is raised (SE_DEV_INDEX for a block table entry out of range). B <= 2048.
 * Workspace:
 * se_cache_append_chunk_workspace_size bytes (one int32).
 */
size_t se_cache_append_chunk_workspace_size(const se_cache_t *c, int32_t T);
int32_t se_cache_append_chunk(se_cache_t *c, const void *k_new, const void *v_new, const int32_t *pos0, int32_t T,
                              const int32_t *counts, int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- Quest page bounds ---------------------------------------------------------------------------------------
 * SparseEngine page, "What it is"/"How it works": Quest's query-dependent page selection. Needs page_meta.
 *  BUILD: page_meta[b][g][p][0][e] / [1][e] = min / max over the resident keys of page p (exact). Every page
 *    p < max_blocks is written; pages without a resident key hold +inf / -inf.
 *  SCORE: page_scores[(b*n_kv+g)*score_stride + p] = max over h in G(g) of sum_e max(q[b][h][e]*min_e,
 *    q[b][h][e]*max_e) for p < ceil(n_slots/page) (fp32 accumulation; -inf for empty pages). q [B][n_q][d].
 */
enum { SE_PAGES_BUILD = 0, SE_PAGES_SCORE = 1 };
int32_t se_page_bounds(se_cache_t *c, int32_t op, const void *q, float *page_scores, int32_t score_stride,
                       int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- Quest metadata maintenance -------------------------------------------------------------------------------
 * The metadata Quest keeps beside the KV (SparseEngine page, "How it works") must follow the cache: an append
 * changes the page it writes, a compaction rewrites the kept prefix. This call writes, for the chosen logical
 * pages of every unit u = b*n_kv + g, exactly what BUILD writes for them (min / max over the page's resident
 * keys, +inf / -inf without any), from the cache as it is now. Other pages are not touched. Needs page_meta.
 *  LAST_PAGE: page ceil(n_slots/page) - 1 of each unit (the page a high-water append wrote; none if n_slots = 0).
 *    page_lo and max_pages are ignored.
 *  FROM_PAGE: pages [page_lo[u], ceil(n_slots/page)) (page_lo: device [B][n_kv]; NULL = page 0 for every unit),
 *    at most max_pages (>= 1) of them per unit: a longer range raises SE_DEV_CAPACITY and only its first
 *    max_pages pages are written; page_lo[u] outside [0, max_blocks] raises SE_DEV_INDEX and skips the unit.
 * A slot reused from the slot stack (H2O) can lie in any page: refresh from that page, or BUILD. No workspace.
 */
enum { SE_REFRESH_LAST_PAGE = 0, SE_REFRESH_FROM_PAGE = 1 };
int32_t se_page_bounds_refresh(se_cache_t *c, int32_t mode, const int32_t *page_lo, int32_t max_pages,
                               int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- decode attention over the view ---------------------------------------------------------------------------
 * o = Attention(q, View), View = BuildView(C, I) (SparseEngine page, "How it works"). For each query head h of
 * KV head g: out[b][h][e] = sum over slots s in View(b, g) of softmax_s(scale * q[b][h] . k_s) v_s[e], fp32
 * output [B][n_q][d]. View(b, g) = the resident slots below n_slots, or, when sel_pages is given, the resident
 * slots of the logical pages sel_pages[(b*n_kv+g)*sel_stride + i], i < sel_count[b*n_kv+g] (ascending,
 * distinct, < ceil(n_slots/page)). An empty view gives 0. With accumulate != 0 (needs cum_score; H2O, the
 * SparseEngine page "What it is"): cum_score[b][g][s] += sum over h in G(g) of that head's weight on s.
 */
typedef struct {
  float scale;
  int32_t sel_stride; /* ignored without sel_pages */
  int32_t max_sel;    /* with sel_pages: upper bound on sel_count (sizes the launch); counts above it raise
                         SE_DEV_CAPACITY and only the first max_sel pages are read */
  int32_t max_slots;  /* without sel_pages: upper bound on n_slots (0 = max_blocks * page); larger n_slots raise
                         SE_DEV_CAPACITY and only the first max_slots slots are read */
  int32_t accumulate;
} se_decode_params_t;

size_t se_sparse_decode_attn_workspace_size(const se_cache_t *c, const se_decode_params_t *p, int32_t has_sel);
int32_t se_sparse_decode_attn(se_cache_t *c, const void *q, const int32_t *sel_pages, const int32_t *sel_count,
                              const se_decode_params_t *p, float *out, int32_t *status, void *ws, size_t ws_bytes,
                              se_stream_t stream);

/* ---- H2O decode step: accumulate, then evict the lowest cumulative score ---------------------------------------
 * SparseEngine page, "What it is": H2O keeps cumulative attention scores during generation and evicts physically by
 * them. One call computes what these three calls in order compute, with the same results bit for bit:
 *   se_sparse_decode_attn (every resident slot, accumulate != 0, max_slots = 0),
 *   se_topk_select (SE_TOPK_SMALLEST, SE_UNIT_SLOT, k = 1, budget, recent, scores = cum_score,
 *                   out_stride = 1) into evict_idx [B*n_kv] and evict_count [B*n_kv] (0 or 1),
 *   se_compact_evict (SE_COMPACT_EVICT_SLOTS) of that list.
 * When the unit's logits fit the single-workgroup decode (max_blocks * page * (n_q / n_kv) <= 38912 and
 * max_blocks * page <= 9984), the choice and the eviction happen inside the decode's own workgroup, from the scores
 * it has just updated (one launch instead of four); otherwise the three calls are made in turn. Needs cum_score and
 * a slot stack (slot_cap > 0). Workspace: se_h2o_decode_evict_workspace_size bytes (0 on the single-workgroup path).
 * Errors: those of the three calls.
 */
typedef struct {
  float scale;
  int32_t budget; /* evict only while ctx_len > budget */
  int32_t recent; /* slots within `recent` positions of the newest resident one are never evicted */
} se_h2o_params_t;

size_t se_h2o_decode_evict_workspace_size(const se_cache_t *c, const se_h2o_params_t *p);
int32_t se_h2o_decode_evict(se_cache_t *c, const void *q, const se_h2o_params_t *p, float *out, int32_t *evict_idx,
                            int32_t *evict_count, int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream);

/* ---- decode attention without allocation -----------------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Computes exactly what se_sparse_decode_attn computes (the same kernels, the same
 * results bit for bit), but its scratch (split partials and, when accumulating, the logits) lives in a static
 * device array of SE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process ends,
 * instead of a caller workspace. The caller still passes every input and output. The array's address is looked
 * up (hipGetSymbolAddress) at the first call on each device, with that device current; the call allocates
 * nothing, with HIP or otherwise.
 * Errors: as se_sparse_decode_attn, plus SE_ERR_SCRATCH_LIMIT (nothing launched) when the call's workspace
 * (se_sparse_decode_attn_workspace_size) exceeds SE_NOALLOC_SCRATCH_BYTES, and SE_ERR_HIP if the lookup fails.
 * Every call on a GPU shares that GPU's one array: calls that may overlap on one GPU (different streams, or
 * different threads without ordering) race and must not be issued; calls in order on one stream are safe. The
 * array keeps the last call's contents; nothing in it needs an initial value.
 */
#define SE_NOALLOC_SCRATCH_BYTES (16u << 20) /* 16 MiB per GPU: e.g. 1024 units x 16 chunks of split partials */
int32_t se_sparse_decode_attn_noalloc(se_cache_t *c, const void *q, const int32_t *sel_pages,
                                      const int32_t *sel_count, const se_decode_params_t *p, float *out,
                                      int32_t *status, se_stream_t stream);

/* ---- utilities ----------------------------------------------------------------------------------------------- */
/* Synchronise `stream`, copy the device status word to *host_value and (if reset) clear it. */
int32_t se_status_read(int32_t *status, int32_t *host_value, int32_t reset, se_stream_t stream);
const char *se_error_string(int32_t code);
const char *se_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SE_H */
