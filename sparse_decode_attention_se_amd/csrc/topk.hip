// Top-K retention and bottom eviction per (sequence, KV head) unit (KARA page "Method" part 1: the top-K
// discrete pairs become retention candidates; SparseEngine page "How it works": SnapKV selection and Quest's
// page selection; "What it is": H2O eviction by continuous attention scores).
//
// One workgroup per unit. Scores become order-preserving 32-bit keys (for the smallest mode the complement),
// and an MSB-first radix select over 8-bit digits of key - min (from the highest differing bit) finds the K-th
// key T with LDS histograms. Items with key T are then resolved by a second radix select over their tie key
// (position, or page id; the complement of the position for the smallest mode), so the result is exactly "K
// best by (score, tie key)". Per-wave ballots and one scan over them write the ascending output. Given
// identical fp32 scores the result is exact.
//
// Range-restricted pruning (SparseEngine page, "How it differs": the application names a position range, a scoring
// policy keeps part of it, and the mask applies to idle blocks only): with a range, only resident slots whose
// position lies in it and whose block has no references are candidates; the others are kept. The output can be
// the dropped candidates instead, the list slot eviction frees.
#include "common.hpp"

namespace se {
namespace {

// workgroup sizes: 1024 threads, or 256 for units of at most 1024 items (fewer waves to meet at each barrier)
constexpr int kThreadsBig = 1024, kThreadsSmall = 256;
#ifndef SE_TOPK_ONE_THREADS
#define SE_TOPK_ONE_THREADS 512  // workgroup size for k = 1 over more than 1024 items (fewer waves per barrier)
#endif

struct TopkArgs {
  const float *scores;
  const int32_t *pos, *n_slots, *ctx;
  const int32_t *bt, *refs;  // block table and per-block reference counts (refs may be NULL: all idle)
  int32_t *idx, *count, *status;
  int32_t mode, unit_kind, k, window, protect, forced_ends, budget, recent, score_stride, out_stride;
  int32_t range_lo, range_hi, emit_dropped;  // range active when range_hi > range_lo
  int32_t n_kv, page, max_slots, max_blocks, num_blocks;
};

// One workgroup per unit; item i lives in thread i % NTH, register j = i / NTH (coalesced loads).

// block-wide reductions (every thread gets the result); s_red holds one value per wave
template <int NTH>
SE_DEV uint32_t block_min_u(uint32_t x, uint32_t *s_red) {
  constexpr int kWaves = NTH / 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = s_red[0];
  for (int w = 1; w < kWaves; ++w) x = min(x, s_red[w]);
  return x;
}
template <int NTH>
SE_DEV uint32_t block_max_u(uint32_t x, uint32_t *s_red) {
  constexpr int kWaves = NTH / 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = s_red[0];
  for (int w = 1; w < kWaves; ++w) x = max(x, s_red[w]);
  return x;
}
template <int NTH>
SE_DEV uint64_t block_max_u64(uint64_t x, uint64_t *s_red) {
  constexpr int kWaves = NTH / 64;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, o), hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), o);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y > x ? y : x;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = s_red[0];
  for (int w = 1; w < kWaves; ++w) x = s_red[w] > x ? s_red[w] : x;
  return x;
}
template <int NTH>
SE_DEV int block_sum_i(int x, uint32_t *s_red) {
  constexpr int kWaves = NTH / 64;
  x = wave_sum_i(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = (uint32_t)x;
  __syncthreads();
  x = 0;
  for (int w = 0; w < kWaves; ++w) x += (int)s_red[w];
  return x;
}

// Among the items of `mask` (bit j: register j), the `want`-th largest value T of v (1 <= want <= #items). On
// return `want` is the number of items equal to T still to be taken (those above T are all taken). Radix select
// over 8-bit digits of v - min, starting at the highest bit in which the items differ, so the first histogram
// already spreads over many bins.
template <int PER, int NTH>
SE_DEV uint32_t radix_kth(const uint32_t (&v)[PER], uint32_t mask, int &want, uint32_t *s_hist, uint32_t *s_red,
                          int *s_res) {
  constexpr int kThreads = NTH;
  uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if ((mask >> j) & 1u) {
      lo = min(lo, v[j]);
      hi = max(hi, v[j]);
    }
  lo = block_min_u<NTH>(lo, s_red);
  hi = block_max_u<NTH>(hi, s_red);
  if (lo >= hi) return hi;  // all equal
  int top = 32 - __clz(hi - lo);
  uint32_t prefix = 0;  // digits of (T - lo) above bit `top` found so far
  const int lane = threadIdx.x & 63;
  while (top > 0) {
    const int w = top < 8 ? top : 8, sh = top - w;
    const uint32_t dmask = (1u << w) - 1u;
    for (int i = threadIdx.x; i < 256; i += kThreads) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!((mask >> j) & 1u)) continue;
      const uint32_t x = v[j] - lo;
      if ((top >= 32 ? 0u : x >> top) == prefix) atomicAdd(&s_hist[(x >> sh) & dmask], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins 4l..4l+3; counts strictly above each bin, from the top digit down
      uint32_t c[4], t = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = s_hist[4 * lane + q];
        t += c[q];
      }
      uint32_t incl = t;  // sum over lanes >= l
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_down((int)incl, o);
        if (lane + o < 64) incl += y;
      }
      uint32_t above = incl - t;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (above < (uint32_t)want && (uint32_t)want <= above + c[q]) {
          s_res[0] = 4 * lane + q;
          s_res[1] = (int)above;
        }
        above += c[q];
      }
    }
    __syncthreads();
    const uint32_t d = (uint32_t)s_res[0];
    want -= s_res[1];
    prefix = (prefix << w) | d;
    top = sh;
    __syncthreads();
  }
  return lo + prefix;
}

template <int PER, bool ONE, int NTH>  // ONE: k == 1, selected by one arg-max instead of radix passes
__global__ __launch_bounds__(NTH) void topk_kernel(TopkArgs a) {
  constexpr int kThreads = NTH, kWaves = NTH / 64;
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_red[kWaves];
  __shared__ uint64_t s_red64[ONE ? kWaves : 1];
  __shared__ int s_res[2];
  __shared__ int s_cnt[PER * kWaves];
  __shared__ uint32_t s_busy[(PER * kThreads + 31) / 32];  // range pruning: logical pages in busy blocks
  const int unit = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int n = a.n_slots[unit];
  n = n < 0 ? 0 : (n > a.max_slots ? a.max_slots : n);
  const int32_t *pos = a.pos + (int64_t)unit * a.max_slots;
  const float *sc = a.scores + (int64_t)unit * a.score_stride;
  const bool page_unit = a.unit_kind == SE_UNIT_PAGE;
  // with a window, the items are the window's slots [base, n); otherwise all slots (or pages) from 0
  const bool win = !page_unit && a.window > 0;
  const int base = win ? n - a.window : 0;
  if (base < 0) {  // a window longer than the cache
    if (t == 0) {
      raise(a.status, SE_DEV_INDEX);
      a.count[unit] = 0;
    }
    return;
  }
  const int n_items = page_unit ? (n + a.page - 1) / a.page : n - base;
  if (n_items > PER * kThreads) {
    if (t == 0) {
      raise(a.status, SE_DEV_CAPACITY);
      a.count[unit] = 0;
    }
    return;
  }

  // Positions (slot units) and scores, every load issued up front and unconditionally (clamped to index 0 where
  // the item does not exist or has no score) so that all are in flight together; selects drop what is not needed.
  const int n_scored = win ? a.window - a.protect : n_items;  // scores exist for items [0, n_scored)
  int pv[PER];
  float sv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kThreads + t;
    pv[j] = pos[base + (i < n_items ? i : 0)];
    sv[j] = sc[i < n_scored && i < n_items ? i : 0];
  }
  int mx = -1;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kThreads + t;
    if (page_unit || i >= n_items) pv[j] = -1;
    mx = max(mx, pv[j]);
  }
  int limit = 0;
  if (a.mode == SE_TOPK_SMALLEST) limit = (int)block_max_u<NTH>((uint32_t)(mx + 1), s_red) - 1 - a.recent;

  // range-restricted pruning: a bit per logical page of the items (pages from the one holding slot `base`) whose
  // block has references, in LDS (threads load block-table entries and counts cooperatively); an item looks up
  // its page's bit. The items span at most PER * kThreads pages, the bitmap's size.
  const bool rng = !page_unit && a.range_hi > a.range_lo;
  const bool gate = rng && a.refs;
  const int p_lo = base / a.page;
  if (gate) {
    const int n_lp = (n + a.page - 1) / a.page;
    for (int i = t; i < (PER * kThreads + 31) / 32; i += kThreads) s_busy[i] = 0u;
    __syncthreads();
    const int32_t *btb = a.bt + (int64_t)(unit / a.n_kv) * a.max_blocks;
    for (int lp = p_lo + t; lp < n_lp && lp - p_lo < PER * kThreads; lp += kThreads) {
      const int blk = btb[lp];
      const int q = lp - p_lo;
      if (blk_ok(blk, a.num_blocks) && a.refs[blk] > 0) atomicOr(&s_busy[q >> 5], 1u << (q & 31));
    }
    __syncthreads();
  }

  // keys of the candidates (tie keys, which order equal scores, are recomputed in the rare tie path below)
  uint32_t key[PER], cand = 0, keep = 0;
  int ncand_local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kThreads + t;
    key[j] = 0;
    if (i >= n_items) continue;
    bool c = false, k = false;
    if (page_unit) {
      const bool end = a.forced_ends && (i == 0 || i == n_items - 1);
      k = end;
      c = !end;
    } else {
      const int p = pv[j];
      if (p < 0) continue;
      if (a.mode == SE_TOPK_SMALLEST) {
        c = p <= limit;
      } else {
        k = base + i >= n - a.protect;
        if (!k && rng) {
          const int lp = (base + i) / a.page - p_lo;
          if (p < a.range_lo || p >= a.range_hi || (gate && ((s_busy[lp >> 5] >> (lp & 31)) & 1u))) k = true;
        }
        c = !k;
      }
    }
    if (c) {
      const float x = sv[j];
      key[j] = a.mode == SE_TOPK_SMALLEST ? ~orderable(x) : orderable(x);
      cand |= 1u << j;
      ++ncand_local;
    }
    if (k) keep |= 1u << j;
  }
  // k = 1 needs no candidate count: its selection below finds nothing when there is no candidate
  const int ncand = ONE ? 0 : block_sum_i<NTH>(ncand_local, s_red);

  int want = a.k;
  if (a.mode == SE_TOPK_SMALLEST) {
    const int over = a.ctx[unit] - a.budget;
    want = min(want, over < 0 ? 0 : over);
  }
  if (!ONE) want = min(want, ncand);

  uint32_t sel = 0;
  uint64_t best = 0;  // k = 1: the chosen item's (key, complemented tie key); 0 when nothing is chosen
  if (ONE) {
    // one item (H2O evicts one per step): the largest key, then the smallest tie key among the items holding it,
    // as the largest pair (key, ~tie key) in one reduction. Tie keys are below 2^31, so a candidate's pair is never 0.
    if (want > 0) {
      auto tie_of = [&](int j) {
        const int i = j * kThreads + t;
        return page_unit ? (uint32_t)i : (a.mode == SE_TOPK_SMALLEST ? 0x7fffffffu - (uint32_t)pv[j] : (uint32_t)pv[j]);
      };
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const uint64_t v = ((uint64_t)key[j] << 32) | (uint32_t)~tie_of(j);
        if (((cand >> j) & 1u) && v > best) best = v;
      }
      best = block_max_u64<NTH>(best, s_red64);
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (((cand >> j) & 1u) && best != 0 && ((uint64_t)key[j] << 32 | (uint32_t)~tie_of(j)) == best) sel |= 1u << j;
    }
    if (a.mode == SE_TOPK_SMALLEST) {
      // nothing is kept besides the chosen item: its thread writes it, with no ordering pass
      if (best != 0 && a.out_stride < 1) {
        if (t == 0) {
          raise(a.status, SE_DEV_CAPACITY);
          a.count[unit] = 0;
        }
        return;
      }
      if (sel) a.idx[(int64_t)unit * a.out_stride] = base + __builtin_ctz(sel) * kThreads + t;
      if (t == 0) a.count[unit] = best != 0 ? 1 : 0;
      return;
    }
  } else if (want == ncand) {
    sel = cand;
  } else if (want > 0) {
    int w = want;
    const uint32_t T = radix_kth<PER, NTH>(key, cand, w, s_hist, s_red, s_res);
    uint32_t eq = 0;
    int n_eq_local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!((cand >> j) & 1u)) continue;
      if (key[j] > T) sel |= 1u << j;
      else if (key[j] == T) {
        eq |= 1u << j;
        ++n_eq_local;
      }
    }
    const int n_eq = block_sum_i<NTH>(n_eq_local, s_red);
    if (n_eq == w) {
      sel |= eq;
    } else {
      // the w smallest tie keys among the tied items: the w largest complements (tie keys are distinct). The tie
      // key is the page id, the position (largest mode) or 0x7fffffff - position (smallest mode: the higher
      // position goes first).
      uint32_t inv[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = j * kThreads + t;
        uint32_t tie = 0;
        if ((eq >> j) & 1u) {
          if (page_unit) tie = (uint32_t)i;
          else {
            const int p = pos[base + i];
            tie = a.mode == SE_TOPK_SMALLEST ? 0x7fffffffu - (uint32_t)p : (uint32_t)p;
          }
        }
        inv[j] = ~tie;
      }
      const uint32_t T2 = radix_kth<PER, NTH>(inv, eq, w, s_hist, s_red, s_res);
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (((eq >> j) & 1u) && inv[j] >= T2) sel |= 1u << j;
    }
  }

  // ascending output: items are ordered by (register j, wave, lane); per (j, wave) counts from ballots, one
  // exclusive scan over them, then each selected item's rank inside its wave
  const uint32_t out = a.emit_dropped ? (cand & ~sel) : (sel | keep);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint64_t b = __ballot((out >> j) & 1u);
    if (lane == 0) s_cnt[j * kWaves + wave] = __popcll(b);
  }
  __syncthreads();
  if (t < 64) {
    constexpr int E = (PER * kWaves + 63) / 64;  // entries per lane
    int v[E], sum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = lane * E + e;
      v[e] = x < PER * kWaves ? s_cnt[x] : 0;
      sum += v[e];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int run = incl - sum;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int x = lane * E + e;
      if (x < PER * kWaves) s_cnt[x] = run;
      run += v[e];
    }
    if (lane == 63) s_res[0] = incl;
  }
  __syncthreads();
  const int total = s_res[0];
  if (total > a.out_stride) {
    if (t == 0) {
      raise(a.status, SE_DEV_CAPACITY);
      a.count[unit] = 0;
    }
    return;
  }
  int32_t *dst = a.idx + (int64_t)unit * a.out_stride;
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint64_t b = __ballot((out >> j) & 1u);
    if ((out >> j) & 1u) dst[s_cnt[j * kWaves + wave] + __popcll(b & lt)] = base + j * kThreads + t;
  }
  if (t == 0) a.count[unit] = total;
}

}  // namespace
}  // namespace se

extern "C" size_t se_topk_select_workspace_size(const se_cache_t *, const se_topk_params_t *) { return 0; }

extern "C" int32_t se_topk_select(const se_cache_t *c, const float *scores, const se_topk_params_t *p, int32_t *idx,
                                  int32_t *count, int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!scores || !p || !idx || !count) return SE_ERR_NULL;
  if (p->k < 0 || p->window < 0 || p->protect < 0 || p->recent < 0) return SE_ERR_PARAM;
  if (p->mode != SE_TOPK_LARGEST && p->mode != SE_TOPK_SMALLEST) return SE_ERR_PARAM;
  if (p->unit != SE_UNIT_SLOT && p->unit != SE_UNIT_PAGE) return SE_ERR_PARAM;
  if (p->mode == SE_TOPK_SMALLEST && p->unit != SE_UNIT_SLOT) return SE_ERR_PARAM;
  if (p->window > 0 && p->protect > p->window) return SE_ERR_PARAM;
  const bool rng = p->range_hi > p->range_lo;
  if ((rng || p->emit_dropped || p->block_refs) && (p->mode != SE_TOPK_LARGEST || p->unit != SE_UNIT_SLOT))
    return SE_ERR_PARAM;
  if (p->block_refs && !rng) return SE_ERR_PARAM;
  const int max_slots = c->max_blocks * c->page;
  const int n_items = p->unit == SE_UNIT_PAGE ? c->max_blocks
                      : (p->mode == SE_TOPK_LARGEST && p->window > 0 && p->window < max_slots) ? p->window
                                                                                                : max_slots;
  long long need = p->k;
  if (p->mode == SE_TOPK_LARGEST) need += p->unit == SE_UNIT_PAGE ? (p->forced_ends ? 2 : 0) : p->protect;
  if (p->out_stride < need && p->out_stride < n_items) return SE_ERR_SHAPE;
  if ((rng || p->emit_dropped) && p->out_stride < n_items) return SE_ERR_SHAPE;  // kept or dropped: up to every slot
  if (p->unit == SE_UNIT_SLOT && p->window == 0 && p->score_stride < max_slots) return SE_ERR_SHAPE;
  if (p->unit == SE_UNIT_SLOT && p->window > 0 && p->score_stride < p->window - p->protect) return SE_ERR_SHAPE;
  if (p->unit == SE_UNIT_PAGE && p->score_stride < c->max_blocks) return SE_ERR_SHAPE;
  se::TopkArgs a;
  a.scores = scores;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.ctx = c->ctx_len;
  a.bt = c->block_table;
  a.refs = p->block_refs;
  a.range_lo = p->range_lo;
  a.range_hi = p->range_hi;
  a.emit_dropped = p->emit_dropped;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.idx = idx;
  a.count = count;
  a.status = status;
  a.mode = p->mode;
  a.unit_kind = p->unit;
  a.k = p->k;
  a.window = p->mode == SE_TOPK_SMALLEST ? 0 : p->window;
  a.protect = p->protect;
  a.forced_ends = p->forced_ends;
  a.budget = p->budget;
  a.recent = p->recent;
  a.score_stride = p->score_stride;
  a.out_stride = p->out_stride;
  a.n_kv = c->n_kv;
  a.page = c->page;
  a.max_slots = max_slots;
  const int units = c->B * c->n_kv;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(units);
#define SE_TOPK_LAUNCH(P, N)                                                                                   \
  do {                                                                                                         \
    if (p->k == 1) hipLaunchKernelGGL((se::topk_kernel<P, true, N>), grid, dim3(N), 0, st, a);                \
    else hipLaunchKernelGGL((se::topk_kernel<P, false, N>), grid, dim3(N), 0, st, a);                          \
  } while (0)
  if (n_items <= 4 * se::kThreadsSmall) {
    if (n_items <= se::kThreadsSmall) SE_TOPK_LAUNCH(1, se::kThreadsSmall);
    else SE_TOPK_LAUNCH(4, se::kThreadsSmall);
  } else if (SE_TOPK_ONE_THREADS != se::kThreadsBig && p->k == 1 && n_items <= 32 * SE_TOPK_ONE_THREADS) {
    constexpr int N = SE_TOPK_ONE_THREADS;
    const int per = (n_items + N - 1) / N;
    if (per <= 4) hipLaunchKernelGGL((se::topk_kernel<4, true, N>), grid, dim3(N), 0, st, a);
    else if (per <= 8) hipLaunchKernelGGL((se::topk_kernel<8, true, N>), grid, dim3(N), 0, st, a);
    else if (per <= 16) hipLaunchKernelGGL((se::topk_kernel<16, true, N>), grid, dim3(N), 0, st, a);
    else hipLaunchKernelGGL((se::topk_kernel<32, true, N>), grid, dim3(N), 0, st, a);
  } else {
    const int per = (n_items + se::kThreadsBig - 1) / se::kThreadsBig;
    if (per <= 4) SE_TOPK_LAUNCH(4, se::kThreadsBig);
    else if (per <= 8) SE_TOPK_LAUNCH(8, se::kThreadsBig);
    else if (per <= 16) SE_TOPK_LAUNCH(16, se::kThreadsBig);
    else if (per <= 32) SE_TOPK_LAUNCH(32, se::kThreadsBig);
    else return SE_ERR_UNSUPPORTED;
  }
#undef SE_TOPK_LAUNCH
  return se_host::launch_status();
}
