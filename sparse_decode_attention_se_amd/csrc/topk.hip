// Top-K retention and bottom eviction per (sequence, KV head) unit (KARA page "Method" part 1: the top-K
// discrete pairs become retention candidates; SparseEngine page "How it works": SnapKV selection and Quest's
// page selection; "What it is": H2O eviction by continuous attention scores).
//
// One workgroup per unit. Scores become order-preserving 32-bit keys (for the smallest mode the complement),
// and an MSB-first radix select over 8-bit digits finds the K-th key T with LDS histograms. Items with key T
// are then resolved by a second radix select over their tie key (position, or page id; the complement of the
// position for the smallest mode), so the result is exactly "K best by (score, tie key)". A workgroup-wide
// scan over items in order writes the ascending output. Given identical fp32 scores the result is exact.
#include "common.hpp"

namespace se {
namespace {

constexpr int kThreads = 1024;

SE_DEV uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkArgs {
  const float *scores;
  const int32_t *pos, *n_slots, *ctx;
  int32_t *idx, *count, *status;
  int32_t mode, unit_kind, k, window, protect, forced_ends, budget, recent, score_stride, out_stride;
  int32_t n_kv, page, max_slots;
};

// candidate item state of one thread: PER contiguous items
template <int PER>
struct Items {
  uint32_t key[PER];
  uint32_t tie[PER];
  uint32_t cand_mask;  // bit j: item is a candidate
  uint32_t keep_mask;  // bit j: item is always kept
};

// find, among items with (v & mask) == prefix and the given candidate mask, the digit at `shift` such that
// `want` items lie at or above it; returns the updated prefix and decrements want by the count above.
template <int PER>
SE_DEV void radix_pass(const uint32_t (&v)[PER], uint32_t sel, uint32_t &prefix, uint32_t &mask, int shift,
                       int &want, uint32_t *s_hist, int *s_res) {
  for (int i = threadIdx.x; i < 256; i += kThreads) s_hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (((sel >> j) & 1u) && (v[j] & mask) == prefix) atomicAdd(&s_hist[(v[j] >> shift) & 255u], 1u);
  __syncthreads();
  // inclusive scan from the top digit: c(t) = #items with digit >= 255 - t
  if (threadIdx.x < 256) s_hist[256 + threadIdx.x] = s_hist[255 - threadIdx.x];
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    uint32_t x = 0;
    if (threadIdx.x < 256 && threadIdx.x >= off) x = s_hist[256 + threadIdx.x - off];
    __syncthreads();
    if (threadIdx.x < 256) s_hist[256 + threadIdx.x] += x;
    __syncthreads();
  }
  if (threadIdx.x < 256) {
    uint32_t c = s_hist[256 + threadIdx.x];
    uint32_t cprev = threadIdx.x ? s_hist[256 + threadIdx.x - 1] : 0u;
    if (cprev < (uint32_t)want && (uint32_t)want <= c) {
      s_res[0] = 255 - threadIdx.x;
      s_res[1] = (int)cprev;
    }
  }
  __syncthreads();
  const int digit = s_res[0];
  want -= s_res[1];
  prefix |= (uint32_t)digit << shift;
  mask |= 255u << shift;
  __syncthreads();
}

template <int PER>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t s_hist[512];
  __shared__ int s_res[2];
  __shared__ int s_scan[kThreads];
  __shared__ int s_red[kThreads / 64];
  const int unit = blockIdx.x;
  const int t = threadIdx.x;
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

  // the smallest mode needs the largest resident position first
  int limit = 0;
  if (a.mode == SE_TOPK_SMALLEST) {
    int mx = -1;
    for (int j = 0; j < PER; ++j) {
      int i = t * PER + j;
      if (i < n_items) mx = max(mx, pos[i]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
    if ((t & 63) == 0) s_red[t >> 6] = mx;
    __syncthreads();
    mx = -1;
    for (int w = 0; w < kThreads / 64; ++w) mx = max(mx, s_red[w]);
    limit = mx - a.recent;
    __syncthreads();
  }

  // gather keys
  Items<PER> it;
  it.cand_mask = 0;
  it.keep_mask = 0;
  int ncand_local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = t * PER + j;
    it.key[j] = 0;
    it.tie[j] = 0;
    if (i >= n_items) continue;
    bool cand = false, keep = false;
    if (page_unit) {
      bool end = a.forced_ends && (i == 0 || i == n_items - 1);
      keep = end;
      cand = !end;
      it.tie[j] = (uint32_t)i;
    } else {
      const int p = pos[base + i];
      if (p < 0) continue;
      if (a.mode == SE_TOPK_SMALLEST) {
        cand = p <= limit;
        it.tie[j] = 0x7fffffffu - (uint32_t)p;
      } else {
        keep = base + i >= n - a.protect;
        cand = !keep;
        it.tie[j] = (uint32_t)p;
      }
    }
    if (cand) {
      const float s = sc[i];
      it.key[j] = a.mode == SE_TOPK_SMALLEST ? ~orderable(s) : orderable(s);
      it.cand_mask |= 1u << j;
      ++ncand_local;
    }
    if (keep) it.keep_mask |= 1u << j;
  }
  // total candidates
  int ncand = ncand_local;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ncand += __shfl_xor(ncand, o);
  if ((t & 63) == 0) s_red[t >> 6] = ncand;
  __syncthreads();
  ncand = 0;
  for (int w = 0; w < kThreads / 64; ++w) ncand += s_red[w];
  __syncthreads();

  int want = a.k;
  if (a.mode == SE_TOPK_SMALLEST) {
    int over = a.ctx[unit] - a.budget;
    want = min(want, over < 0 ? 0 : over);
  }
  want = min(want, ncand);

  uint32_t sel_mask = 0;
  if (want == ncand) {
    sel_mask = it.cand_mask;
  } else if (want > 0) {
    uint32_t prefix = 0, mask = 0;
    int w = want;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) radix_pass<PER>(it.key, it.cand_mask, prefix, mask, shift, w, s_hist, s_res);
    const uint32_t T = prefix;  // the want-th largest key; w items with key == T still to take
    uint32_t eq_mask = 0;
    int n_eq_local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (!((it.cand_mask >> j) & 1u)) continue;
      if (it.key[j] > T) sel_mask |= 1u << j;
      else if (it.key[j] == T) {
        eq_mask |= 1u << j;
        ++n_eq_local;
      }
    }
    int n_eq = n_eq_local;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n_eq += __shfl_xor(n_eq, o);
    if ((t & 63) == 0) s_red[t >> 6] = n_eq;
    __syncthreads();
    n_eq = 0;
    for (int ww = 0; ww < kThreads / 64; ++ww) n_eq += s_red[ww];
    __syncthreads();
    if (n_eq == w) {
      sel_mask |= eq_mask;
    } else {
      // the w smallest tie keys among the tied items: radix select the largest complements
      uint32_t inv[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) inv[j] = ~it.tie[j];
      uint32_t p2 = 0, m2 = 0;
      int w2 = w;
#pragma unroll 1
      for (int shift = 24; shift >= 0; shift -= 8) radix_pass<PER>(inv, eq_mask, p2, m2, shift, w2, s_hist, s_res);
      // tie keys are distinct among resident items, so exactly one item holds the threshold and w2 == 1
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (((eq_mask >> j) & 1u) && inv[j] >= p2) sel_mask |= 1u << j;
    }
  }

  // ascending output: scan of per-thread counts over contiguous item ranges
  const uint32_t out_mask = sel_mask | it.keep_mask;
  const int mine = __popc(out_mask);
  s_scan[t] = mine;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int x = t >= off ? s_scan[t - off] : 0;
    __syncthreads();
    s_scan[t] += x;
    __syncthreads();
  }
  int o = s_scan[t] - mine;
  const int total = s_scan[kThreads - 1];
  int32_t *out = a.idx + (int64_t)unit * a.out_stride;
  if (total > a.out_stride) {
    if (t == 0) {
      raise(a.status, SE_DEV_CAPACITY);
      a.count[unit] = 0;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if ((out_mask >> j) & 1u) out[o++] = base + t * PER + j;
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
  const int max_slots = c->max_blocks * c->page;
  const int n_items = p->unit == SE_UNIT_PAGE ? c->max_blocks
                      : (p->mode == SE_TOPK_LARGEST && p->window > 0 && p->window < max_slots) ? p->window
                                                                                                : max_slots;
  long long need = p->k;
  if (p->mode == SE_TOPK_LARGEST) need += p->unit == SE_UNIT_PAGE ? (p->forced_ends ? 2 : 0) : p->protect;
  if (p->out_stride < need && p->out_stride < n_items) return SE_ERR_SHAPE;
  if (p->unit == SE_UNIT_SLOT && p->window == 0 && p->score_stride < max_slots) return SE_ERR_SHAPE;
  if (p->unit == SE_UNIT_SLOT && p->window > 0 && p->score_stride < p->window - p->protect) return SE_ERR_SHAPE;
  if (p->unit == SE_UNIT_PAGE && p->score_stride < c->max_blocks) return SE_ERR_SHAPE;
  se::TopkArgs a;
  a.scores = scores;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.ctx = c->ctx_len;
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
  const int per = (n_items + se::kThreads - 1) / se::kThreads;
  if (per <= 1) hipLaunchKernelGGL(se::topk_kernel<1>, dim3(units), dim3(se::kThreads), 0, st, a);
  else if (per <= 4) hipLaunchKernelGGL(se::topk_kernel<4>, dim3(units), dim3(se::kThreads), 0, st, a);
  else if (per <= 8) hipLaunchKernelGGL(se::topk_kernel<8>, dim3(units), dim3(se::kThreads), 0, st, a);
  else if (per <= 16) hipLaunchKernelGGL(se::topk_kernel<16>, dim3(units), dim3(se::kThreads), 0, st, a);
  else if (per <= 32) hipLaunchKernelGGL(se::topk_kernel<32>, dim3(units), dim3(se::kThreads), 0, st, a);
  else return SE_ERR_UNSUPPORTED;
  return se_host::launch_status();
}
