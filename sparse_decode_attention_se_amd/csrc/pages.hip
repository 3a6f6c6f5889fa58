// Quest page metadata and page upper bounds (SparseEngine page, "What it is" / "How it works": Quest's
// query-dependent page selection at build_decode_selection; the metadata is kept beside the KV).
//   BUILD  page_meta[b][g][p] = (elementwise min, elementwise max) of the resident keys of page p
//   SCORE  U[b][g][p] = max over the group's query heads of sum_e max(q_e * min_e, q_e * max_e)
//   REFRESH (se_page_bounds_refresh) BUILD's values for the pages an append or a compaction changed
// All are HBM streams: a page's key tile for one head is 16 rows x 256 B contiguous, read by 16 lanes.
#include "common.hpp"

namespace se {
namespace {

constexpr int kThreads = 256;
constexpr int kPagesPerWG = kThreads / 16;

struct PagesArgs {
  const char *k;
  const int32_t *bt, *pos, *n_slots;
  char *meta;
  const char *q;
  float *scores;
  int32_t *status;
  int32_t n_kv, page, max_blocks, num_blocks, score_stride, R;
  const int32_t *page_lo;     // refresh: first page per unit (NULL = 0)
  int32_t refresh_last, max_pages;
};

template <int DTYPE>
SE_DEV void unpack(const u32x4 &w, float *x) {
  if (DTYPE == SE_DTYPE_BF16) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y); x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
}

template <int DTYPE>
SE_DEV u32x4 pack(const float *x) {
  u32x4 w;
  if (DTYPE == SE_DTYPE_BF16) {  // values are bf16 already: truncation is exact
    w.x = (__float_as_uint(x[0]) >> 16) | (__float_as_uint(x[1]) & 0xffff0000u);
    w.y = (__float_as_uint(x[2]) >> 16) | (__float_as_uint(x[3]) & 0xffff0000u);
    w.z = (__float_as_uint(x[4]) >> 16) | (__float_as_uint(x[5]) & 0xffff0000u);
    w.w = (__float_as_uint(x[6]) >> 16) | (__float_as_uint(x[7]) & 0xffff0000u);
  } else {
    w.x = __float_as_uint(x[0]); w.y = __float_as_uint(x[1]); w.z = __float_as_uint(x[2]); w.w = __float_as_uint(x[3]);
  }
  return w;
}

// page p of unit (b, g) with n slots: (min, max) over its resident keys into page_meta (+inf / -inf without any),
// by the 16 lanes of one row, lane cl holding bytes [16 cl, 16 cl + 16) of the key
template <int DTYPE>
SE_DEV void build_page(const PagesArgs &a, int unit, int b, int g, int p, int cl, int n) {
  constexpr int EPL = DTYPE == SE_DTYPE_BF16 ? 8 : 4;
  float lo[EPL], hi[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    lo[e] = INFINITY;
    hi[e] = -INFINITY;
  }
  const int blk = (p * a.page < n) ? a.bt[(int64_t)b * a.max_blocks + p] : -1;
  if (blk_ok(blk, a.num_blocks)) {
    const int32_t *pos = a.pos + (int64_t)unit * a.max_blocks * a.page + p * a.page;
    const char *tile = a.k + ((int64_t)blk * a.n_kv + g) * a.page * 256 + cl * 16;
    const int rows = min(a.page, n - p * a.page);
    // eight rows at a time: their positions and key pieces all in flight (past the page's last row: that row
    // again, not counted)
    for (int i0 = 0; i0 < rows; i0 += 8) {
      int pv[8];
      u32x4 w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = min(i0 + j, rows - 1);
        pv[j] = pos[i];
        w[j] = ld16_stream(tile + i * 256);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (i0 + j >= rows || pv[j] < 0) continue;
        float x[EPL];
        unpack<DTYPE>(w[j], x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          lo[e] = fminf(lo[e], x[e]);
          hi[e] = fmaxf(hi[e], x[e]);
        }
      }
    }
  } else if (p * a.page < n) {
    raise(a.status, SE_DEV_INDEX);
  }
  char *m = a.meta + ((int64_t)unit * a.max_blocks + p) * 2 * 256 + cl * 16;
  st16(m, pack<DTYPE>(lo));
  st16(m + 256, pack<DTYPE>(hi));
}

template <int DTYPE>
__global__ __launch_bounds__(kThreads) void pages_build(PagesArgs a) {
  const int unit = blockIdx.y;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int p = blockIdx.x * kPagesPerWG + (threadIdx.x >> 4);
  if (p >= a.max_blocks) return;
  int n = a.n_slots[unit];
  n = min(max(n, 0), a.max_blocks * a.page);
  build_page<DTYPE>(a, unit, b, g, p, threadIdx.x & 15, n);
}

// the unit's pages [lo, ceil(n_slots / page)), lo = page_lo[unit] (0 without page_lo), or only its last page;
// at most max_pages of them
template <int DTYPE>
__global__ __launch_bounds__(kThreads) void pages_refresh(PagesArgs a) {
  const int unit = blockIdx.y;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  int n = a.n_slots[unit];
  n = min(max(n, 0), a.max_blocks * a.page);
  const int n_pages = (n + a.page - 1) / a.page;
  int lo, hi;
  if (a.refresh_last) {
    lo = n_pages - 1;
    hi = n_pages;
  } else {
    lo = a.page_lo ? a.page_lo[unit] : 0;
    hi = n_pages;
    if (lo < 0 || lo > a.max_blocks) {
      if (blockIdx.x == 0 && threadIdx.x == 0) raise(a.status, SE_DEV_INDEX);
      return;
    }
    if (hi - lo > a.max_pages) {
      if (blockIdx.x == 0 && threadIdx.x == 0) raise(a.status, SE_DEV_CAPACITY);
      hi = lo + a.max_pages;
    }
  }
  const int p = lo + blockIdx.x * kPagesPerWG + (threadIdx.x >> 4);
  if (p < 0 || p >= hi) return;
  build_page<DTYPE>(a, unit, b, g, p, threadIdx.x & 15, n);
}

template <int DTYPE, int R>
__global__ __launch_bounds__(kThreads) void pages_score(PagesArgs a) {
  constexpr int EPL = DTYPE == SE_DTYPE_BF16 ? 8 : 4;
  const int unit = blockIdx.y;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int p = blockIdx.x * kPagesPerWG + (threadIdx.x >> 4);
  const int cl = threadIdx.x & 15;
  int n = a.n_slots[unit];
  n = min(max(n, 0), a.max_blocks * a.page);
  const int n_pages = (n + a.page - 1) / a.page;
  float q[R][EPL];
#pragma unroll
  for (int h = 0; h < R; ++h) unpack<DTYPE>(ld16(a.q + (((int64_t)b * a.n_kv + g) * R + h) * 256 + cl * 16), q[h]);
  const bool live = p < n_pages;  // uniform within the 16-lane row
  float lo[EPL], hi[EPL];
  if (live) {
    const char *m = a.meta + ((int64_t)unit * a.max_blocks + p) * 2 * 256 + cl * 16;
    unpack<DTYPE>(ld16_stream(m), lo);  // read once per call: non-temporal
    unpack<DTYPE>(ld16_stream(m + 256), hi);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) lo[e] = hi[e] = 0.f;
  }
  float best = -INFINITY;
#pragma unroll
  for (int h = 0; h < R; ++h) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s += fmaxf(q[h][e] * lo[e], q[h][e] * hi[e]);
    best = fmaxf(best, row16_sum(s));
  }
  const float empty = row16_max(lo[0] > hi[0] ? 1.f : 0.f);
  if (live && cl == 0) a.scores[(int64_t)unit * a.score_stride + p] = empty > 0.f ? -INFINITY : best;
}

}  // namespace
}  // namespace se

extern "C" int32_t se_page_bounds(se_cache_t *c, int32_t op, const void *q, float *page_scores, int32_t score_stride,
                                  int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!c->page_meta) return SE_ERR_NULL;
  const bool ok_shape = (c->dtype == SE_DTYPE_BF16 && c->d == 128) || (c->dtype == SE_DTYPE_F32 && c->d == 64);
  if (!ok_shape) return SE_ERR_DTYPE;
  se::PagesArgs a;
  a.k = (const char *)c->k_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.meta = (char *)c->page_meta;
  a.q = (const char *)q;
  a.scores = page_scores;
  a.status = status;
  a.n_kv = c->n_kv;
  a.page = c->page;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.score_stride = score_stride;
  a.R = c->n_q / c->n_kv;
  a.page_lo = nullptr;
  a.refresh_last = 0;
  a.max_pages = 0;
  const dim3 grid((c->max_blocks + se::kPagesPerWG - 1) / se::kPagesPerWG, c->B * c->n_kv);
  hipStream_t st = (hipStream_t)stream;
  if (op == SE_PAGES_BUILD) {
    if (c->dtype == SE_DTYPE_BF16) hipLaunchKernelGGL(se::pages_build<SE_DTYPE_BF16>, grid, dim3(se::kThreads), 0, st, a);
    else hipLaunchKernelGGL(se::pages_build<SE_DTYPE_F32>, grid, dim3(se::kThreads), 0, st, a);
    return se_host::launch_status();
  }
  if (op != SE_PAGES_SCORE) return SE_ERR_PARAM;
  if (!q || !page_scores) return SE_ERR_NULL;
  if (score_stride < c->max_blocks) return SE_ERR_SHAPE;
#define SE_PAGES_R(RR)                                                                                         \
  case RR:                                                                                                     \
    if (c->dtype == SE_DTYPE_BF16)                                                                             \
      hipLaunchKernelGGL((se::pages_score<SE_DTYPE_BF16, RR>), grid, dim3(se::kThreads), 0, st, a);            \
    else                                                                                                       \
      hipLaunchKernelGGL((se::pages_score<SE_DTYPE_F32, RR>), grid, dim3(se::kThreads), 0, st, a);             \
    break;
  switch (a.R) {
    SE_PAGES_R(1)
    SE_PAGES_R(2)
    SE_PAGES_R(4)
    SE_PAGES_R(8)
    default: return SE_ERR_UNSUPPORTED;
  }
#undef SE_PAGES_R
  return se_host::launch_status();
}

extern "C" int32_t se_page_bounds_refresh(se_cache_t *c, int32_t mode, const int32_t *page_lo, int32_t max_pages,
                                          int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!c->page_meta) return SE_ERR_NULL;
  const bool ok_shape = (c->dtype == SE_DTYPE_BF16 && c->d == 128) || (c->dtype == SE_DTYPE_F32 && c->d == 64);
  if (!ok_shape) return SE_ERR_DTYPE;
  if (mode != SE_REFRESH_LAST_PAGE && mode != SE_REFRESH_FROM_PAGE) return SE_ERR_PARAM;
  if (mode == SE_REFRESH_FROM_PAGE && max_pages < 1) return SE_ERR_PARAM;
  se::PagesArgs a;
  a.k = (const char *)c->k_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.meta = (char *)c->page_meta;
  a.q = nullptr;
  a.scores = nullptr;
  a.status = status;
  a.n_kv = c->n_kv;
  a.page = c->page;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.score_stride = 0;
  a.R = c->n_q / c->n_kv;
  a.page_lo = mode == SE_REFRESH_FROM_PAGE ? page_lo : nullptr;
  a.refresh_last = mode == SE_REFRESH_LAST_PAGE;
  const int pages = a.refresh_last ? 1 : (max_pages < c->max_blocks ? max_pages : c->max_blocks);
  a.max_pages = pages;
  const dim3 grid((pages + se::kPagesPerWG - 1) / se::kPagesPerWG, c->B * c->n_kv);
  hipStream_t st = (hipStream_t)stream;
  if (c->dtype == SE_DTYPE_BF16) hipLaunchKernelGGL(se::pages_refresh<SE_DTYPE_BF16>, grid, dim3(se::kThreads), 0, st, a);
  else hipLaunchKernelGGL(se::pages_refresh<SE_DTYPE_F32>, grid, dim3(se::kThreads), 0, st, a);
  return se_host::launch_status();
}
