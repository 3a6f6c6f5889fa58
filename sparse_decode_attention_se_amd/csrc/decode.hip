// Decode attention over a view of the paged cache: o = Attention(q, View), View = BuildView(C, I)
// (SparseEngine page, "How it works"), optionally adding each step's softmax weights to per-slot cumulative
// scores (H2O, SparseEngine page "What it is").
//
// The op is HBM-bound (each KV byte is used for one query group), so it runs on the vector ALU, not MFMA.
// Split-K: workgroup (chunk, unit) streams `chunk_rows` view rows of one (sequence, KV head) unit. A row of
// K or V is 256 bytes (bf16 d=128 or fp32 d=64) = 16 lanes x 16 B, so a wave reads four rows per load and the
// per-row dot products reduce inside a 16-lane DPP row. Each lane-row keeps an online softmax (max, sum,
// weighted V) for the R query heads of the group; lane-rows and waves merge at the end and the workgroup
// writes one (m, l, acc[d]) partial per head. A second kernel merges the chunks and, when asked, turns the
// stored logits into probabilities and adds them to cum_score. Accumulating decode over all slots of views that
// fit in LDS takes a one-launch path instead (decode_unit).
#include <atomic>
#include <mutex>

#include "common.hpp"

namespace se {
namespace {

constexpr int kThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// out[h] = x of lane h of the lane's row of 16, h < N
template <int N>
SE_DEV void bcast_r(float x, float (&out)[N]) {
  out[0] = row16_bcast<0>(x);
  if constexpr (N > 1) out[1 % N] = row16_bcast<1 % N>(x);
  if constexpr (N > 2) out[2 % N] = row16_bcast<2 % N>(x), out[3 % N] = row16_bcast<3 % N>(x);
  if constexpr (N > 4) {
    out[4 % N] = row16_bcast<4 % N>(x), out[5 % N] = row16_bcast<5 % N>(x);
    out[6 % N] = row16_bcast<6 % N>(x), out[7 % N] = row16_bcast<7 % N>(x);
  }
}
constexpr int kUnroll = 4;  // wave-loads in flight per lane-row

template <int DTYPE>
struct Vec;

template <>
struct Vec<SE_DTYPE_BF16> {
  static constexpr int EPL = 8;  // elements per lane (16 B)
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  SE_DEV static float dot(const u32x4 &q, const u32x4 &k, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.x), __builtin_bit_cast(bf2, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.y), __builtin_bit_cast(bf2, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.z), __builtin_bit_cast(bf2, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q.w), __builtin_bit_cast(bf2, k.w), acc, false);
    return acc;
  }
  SE_DEV static void widen(const u32x4 &w, float *x) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
};

template <>
struct Vec<SE_DTYPE_F32> {
  static constexpr int EPL = 4;
  SE_DEV static float dot(const u32x4 &q, const u32x4 &k, float acc) {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  SE_DEV static void widen(const u32x4 &w, float *x) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y); x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};

struct DecodeArgs {
  const char *k, *v;
  const int32_t *bt, *pos, *n_slots;
  const char *q;
  const int32_t *sel, *sel_count;
  float *out, *part, *logits, *cum;
  float *mil;  // with accumulate: per (unit, head) the merged max and 1/sum, written by decode_merge
  int32_t *status;
  int32_t n_kv, page, max_blocks, num_blocks, sel_stride, rows_bound, chunk_rows, nchunk;
  float scale_log2;
  // H2O's eviction inside decode_unit: the cache's mutable maps, the chosen slot and count per unit
  int32_t *ev_pos, *ev_stack, *ev_top, *ev_ctx, *ev_idx, *ev_count;
  int32_t ev_cap, ev_budget, ev_recent;
};

// number of view rows of a unit, and the slot of view row r (-1 if the row is not in the view)
struct ViewMap {
  const DecodeArgs &a;
  int unit, n, rows;
  SE_DEV ViewMap(const DecodeArgs &a_, int unit_) : a(a_), unit(unit_) {
    n = a.n_slots[unit];
    int cap = a.max_blocks * a.page;
    n = n < 0 ? 0 : (n > cap ? cap : n);
    if (a.sel) {
      int cnt = a.sel_count[unit];
      int bound = a.rows_bound / a.page;
      rows = (cnt < 0 ? 0 : (cnt > bound ? bound : cnt)) * a.page;
    } else {
      rows = n < a.rows_bound ? n : a.rows_bound;
    }
  }
  SE_DEV int slot(int r) const {
    if (r >= rows) return -1;
    if (!a.sel) return r;
    const int32_t *list = a.sel + (int64_t)unit * a.sel_stride;
    int i = r / a.page;
    int p = list[i];
    int n_pages = (n + a.page - 1) / a.page;
    if (p < 0 || p >= n_pages || (i > 0 && list[i - 1] >= p)) return -2;  // invalid selection entry
    int s = p * a.page + r % a.page;
    return s < n ? s : -1;
  }
};

// Running maxima move only when a logit exceeds them by more than kLazy (log2 units): until then the weights are
// exp2 of at most kLazy, which fp32 sums hold without loss, and the rescale of l and acc is skipped.
constexpr float kLazy = 8.f;
constexpr int kMaxChunkRows = 2048;
#ifndef SE_DECODE_WG_PER_CU
#define SE_DECODE_WG_PER_CU 2  // occupancy hint of the split kernel (the compiler settles at three waves per SIMD)
#endif
#ifndef SE_DECODE_MIN_WGS
#define SE_DECODE_MIN_WGS 512
#endif
constexpr int kMinWGs = SE_DECODE_MIN_WGS;
#ifndef SE_DECODE_HOT_ROWS
#define SE_DECODE_HOT_ROWS 4096
#endif
constexpr int kHotRows = SE_DECODE_HOT_ROWS;  // a unit's most recent rows, read with plain loads
constexpr int kUnitHotRows = 2048;              // the same for the single-workgroup decode

template <int DTYPE, int R>
__global__ __launch_bounds__(kThreads, SE_DECODE_WG_PER_CU) void decode_partial(DecodeArgs a) {
  using V = Vec<DTYPE>;
  constexpr int EPL = V::EPL;
  constexpr int D = 16 * EPL;
  constexpr int RB = 256;  // row bytes
  const int unit = blockIdx.y, chunk = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane >> 4, cl = lane & 15;
  __shared__ int s_row[kMaxChunkRows];

  // the group's query heads, this lane's 16-byte slice of each
  u32x4 q[R];
#pragma unroll
  for (int h = 0; h < R; ++h) q[h] = ld16(a.q + (((int64_t)b * a.n_kv + g) * R + h) * RB + cl * 16);
  // bf16, d = 128: the step's logits come from MFMA. S^T = K Q^T per 16 keys (v_mfma_f32_16x16x32_bf16, four
  // k-steps): A = 16 keys x 32 dims (lane l: key l % 16, dims 32 t + 8 (l / 16)), B = 32 dims x 16 columns, the
  // group's R query heads and zeros (lane l: head l % 16). Lane l receives keys 4 (l / 16) + v of head l % 16:
  // in lane-row lr, lanes 0..R-1 hold the logits of keys 4 lr .. 4 lr + 3, the keys whose V slices that lane-row
  // accumulates, so the weights reach them by broadcasts inside the row.
  constexpr bool kMfma = DTYPE == SE_DTYPE_BF16 && EPL == 8;
  bf16x8 qf[4];
  if constexpr (kMfma) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[t] = __builtin_bit_cast(
          bf16x8, cl < R ? ld16(a.q + (((int64_t)b * a.n_kv + g) * R + (cl < R ? cl : 0)) * RB + t * 64 + lrow * 16)
                         : z);
    }
  }

  // Resolve the chunk's view rows to pool rows (-1: outside the view or not resident) into LDS. Loads are
  // issued speculatively (only their addresses are range-checked), so the chain is two rounds deep.
  const int cap = a.max_blocks * a.page;
  int n = a.n_slots[unit];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int32_t *list = a.sel ? a.sel + (int64_t)unit * a.sel_stride : nullptr;
  int rows;
  if (list) {
    const int cnt = a.sel_count[unit], bound = a.rows_bound / a.page;
    if (chunk == 0 && threadIdx.x == 0 && cnt > bound) raise(a.status, SE_DEV_CAPACITY);
    rows = (cnt < 0 ? 0 : (cnt > bound ? bound : cnt)) * a.page;
  } else {
    if (chunk == 0 && threadIdx.x == 0 && n > a.rows_bound) raise(a.status, SE_DEV_CAPACITY);
    rows = n < a.rows_bound ? n : a.rows_bound;
  }
  const int row0 = chunk * a.chunk_rows;
  const int n_pages = (n + a.page - 1) / a.page;
  const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  const int32_t *pos = a.pos + (int64_t)unit * cap;
  bool bad = false;
  for (int i = threadIdx.x; i < a.chunk_rows; i += kThreads) {
    const int r = row0 + i;
    int v = -1;
    if (r < a.rows_bound) {
      const int pi = r / a.page, off = r - pi * a.page;
      const int p = list ? list[pi] : pi;
      const int prev = list && pi > 0 ? list[pi - 1] : -1;
      const bool p_safe = p >= 0 && p < a.max_blocks;
      const int s = (p_safe ? p : 0) * a.page + off;
      const int blk = bt[p_safe ? p : 0];
      const int ps = pos[s];
      if (r < rows) {
        const bool p_ok = p_safe && p < n_pages && prev < p;
        if (!p_ok) {
          bad = true;
        } else if (s < n && ps >= 0) {
          if (blk_ok(blk, a.num_blocks)) v = (blk * a.n_kv + g) * a.page + off;
          else bad = true;
        }
      }
    }
    s_row[i] = v;
  }
  if (bad) raise(a.status, SE_DEV_INDEX);

  float m[R], l[R], acc[R][EPL];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -1e30f;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  __syncthreads();

  // each wave streams a contiguous quarter of the chunk, 16 rows (4 lane-rows x 4) per step, double-buffered
  const int per_wave = a.chunk_rows / 4;
  const int w0 = wave * per_wave;
  int lim = rows - row0 - w0;
  lim = lim < 0 ? 0 : (lim > per_wave ? per_wave : lim);
  const int nit = (lim + 15) / 16;

  // Chunks away from the unit's most recent rows (which the step's other calls have just written or read, so
  // that the last-level cache may hold them) stream their rows with non-temporal loads.
  const bool cold = list != nullptr || row0 + a.chunk_rows <= n - kHotRows;
  auto load = [&](int it, u32x4 (&kb)[kUnroll], u32x4 (&vb)[kUnroll], int (&rv)[kUnroll]) {
    if constexpr (kMfma) {
      // K in the MFMA layout (key cl of the step, k-step t at byte 64 t); V of keys 4 lrow + u, slice cl
      const int ik = it * 16 + cl;
      const int vk = ik < lim ? s_row[w0 + ik] : -1;
      const char *kr = a.k + (int64_t)(vk >= 0 ? vk : 0) * RB + lrow * 16;
      const char *vr[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = it * 16 + lrow * 4 + u;
        const int v = i < lim ? s_row[w0 + i] : -1;
        vr[u] = a.v + (int64_t)(v >= 0 ? v : 0) * RB + cl * 16;
        rv[u] = v;
      }
      if (cold) {  // uniform
#pragma unroll
        for (int t = 0; t < 4; ++t) kb[t] = ld16_stream(kr + t * 64);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) vb[u] = ld16_stream(vr[u]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) kb[t] = ld16(kr + t * 64);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) vb[u] = ld16(vr[u]);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = it * 16 + u * 4 + lrow;
      const int v = i < lim ? s_row[w0 + i] : -1;
      const int64_t off = (int64_t)(v >= 0 ? v : 0) * RB + cl * 16;
      kb[u] = ld16(a.k + off);
      vb[u] = ld16(a.v + off);
      rv[u] = v;
    }
  };
  // With R x kUnroll = 16 logits per lane-row and step, one per lane (the GQA group of four heads): the partial dot
  // products are reduce-scattered over the row's 16 lanes, so lane cl holds the logit of row u = cl / R of the
  // step, head h = cl % R, and does that logit's softmax work alone. Each lane keeps the running max ml and the sum
  // ll of its head (the four lanes of a head move ml together: their maximum is shared); the weights are then
  // broadcast to the row for the V accumulation.
  constexpr bool kOne = R * kUnroll == 16;
  float ml = -1e30f, ll = 0.f;
  auto step1 = [&](int it, const u32x4 (&kb)[kUnroll], const u32x4 (&vb)[kUnroll], const int (&rv)[kUnroll])
      __attribute__((always_inline)) {
    float d[16];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int h = 0; h < R; ++h) d[(u * R + h) & 15] = V::dot(q[h], kb[u], 0.f);
    float s = row16_reduce_scatter(d);
    const int ul = cl / R, hl = cl % R;
    const int rvl = ul == 0 ? rv[0] : ul == 1 ? rv[1 % kUnroll] : ul == 2 ? rv[2 % kUnroll] : rv[3 % kUnroll];
    s = rvl >= 0 ? s * a.scale_log2 : -INFINITY;
    if (a.logits) {
      const int i = it * 16 + ul * 4 + lrow;
      if (i < lim) a.logits[((int64_t)unit * a.rows_bound + row0 + w0 + i) * R + hl] = s;
    }
    float mx = fmaxf(s, dpp_f<kRowRor4>(s));  // the head's maximum over the step's rows of this lane-row
    if constexpr (R == 4) mx = fmaxf(mx, dpp_f<kRowRor8>(mx));
    if (__builtin_amdgcn_ballot_w64(mx > ml + kLazy)) {  // uniform, rare
      const float mn = mx > ml + kLazy ? mx : ml;
      const float f = __builtin_amdgcn_exp2f(ml - mn);
      ml = mn;
      ll *= f;
      float fh[R];
      fh[0] = row16_bcast<0>(f);
      if constexpr (R > 1) fh[1 % R] = row16_bcast<1 % R>(f);
      if constexpr (R > 2) fh[2 % R] = row16_bcast<2 % R>(f), fh[3 % R] = row16_bcast<3 % R>(f);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= fh[h];
    }
    const float p = __builtin_amdgcn_exp2f(s - ml);
    ll += p;
    float pj[16];
    pj[0] = row16_bcast<0>(p), pj[1] = row16_bcast<1>(p), pj[2] = row16_bcast<2>(p), pj[3] = row16_bcast<3>(p);
    pj[4] = row16_bcast<4>(p), pj[5] = row16_bcast<5>(p), pj[6] = row16_bcast<6>(p), pj[7] = row16_bcast<7>(p);
    pj[8] = row16_bcast<8>(p), pj[9] = row16_bcast<9>(p), pj[10] = row16_bcast<10>(p);
    pj[11] = row16_bcast<11>(p), pj[12] = row16_bcast<12>(p), pj[13] = row16_bcast<13>(p);
    pj[14] = row16_bcast<14>(p), pj[15] = row16_bcast<15>(p);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool ok = rv[u] >= 0;  // rows outside the view read row 0 of the pool: drop its values
      const u32x4 w = {ok ? vb[u].x : 0u, ok ? vb[u].y : 0u, ok ? vb[u].z : 0u, ok ? vb[u].w : 0u};
      float x[EPL];
      V::widen(w, x);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pj[(u * R + h) & 15], x[e], acc[h][e]);
    }
  };
  // The MFMA step: lane (lr, c) with c < R holds the logits of keys 4 lr + v, head c, and does their softmax work:
  // the head's maximum over the step's 16 keys (in-lane, then across the four lane-rows), its running max ml
  // (shared by the head's four lanes) and its lane-row's sum ll.
  auto stepm = [&](int it, const u32x4 (&kb)[kUnroll], const u32x4 (&vb)[kUnroll], const int (&rv)[kUnroll])
      __attribute__((always_inline)) {
    floatx4 lg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) lg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[t]), qf[t],
                                                                           lg, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sv[v] = rv[v] >= 0 ? lg[v] * a.scale_log2 : -INFINITY;
    if (a.logits && cl < R) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = it * 16 + lrow * 4 + v;
        if (i < lim) a.logits[((int64_t)unit * a.rows_bound + row0 + w0 + i) * R + cl] = sv[v];
      }
    }
    const float mx = cross_row_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (__builtin_amdgcn_ballot_w64(mx > ml + kLazy)) {  // uniform, rare
      const float mn = mx > ml + kLazy ? mx : ml;
      const float f = __builtin_amdgcn_exp2f(ml - mn);
      ml = mn;
      ll *= f;
      float fh[R];
      bcast_r<R>(f, fh);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= fh[h];
    }
    float pv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) pv[v] = __builtin_amdgcn_exp2f(sv[v] - ml);
    ll += (pv[0] + pv[1]) + (pv[2] + pv[3]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float ph[R];
      bcast_r<R>(pv[u], ph);
      const bool ok = rv[u] >= 0;  // rows outside the view read row 0 of the pool: drop its values
      const u32x4 w = {ok ? vb[u].x : 0u, ok ? vb[u].y : 0u, ok ? vb[u].z : 0u, ok ? vb[u].w : 0u};
      float x[EPL];
      V::widen(w, x);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(ph[h], x[e], acc[h][e]);
    }
  };
  auto step = [&](int it, const u32x4 (&kb)[kUnroll], const u32x4 (&vb)[kUnroll], const int (&rv)[kUnroll]) {
    if constexpr (kMfma) {
      stepm(it, kb, vb, rv);
      return;
    } else if constexpr (kOne) {
      step1(it, kb, vb, rv);
      return;
    }
    float sc[kUnroll][R];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float d = row16_sum(V::dot(q[h], kb[u], 0.f));
        sc[u][h] = rv[u] >= 0 ? d * a.scale_log2 : -INFINITY;
      }
    }
    if (a.logits) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int i = it * 16 + u * 4 + lrow;
        if (cl == 0 && i < lim) {
          float *dst = a.logits + ((int64_t)unit * a.rows_bound + row0 + w0 + i) * R;
#pragma unroll
          for (int h = 0; h < R; ++h) dst[h] = sc[u][h];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mx = sc[0][h];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, sc[u][h]);
      if (mx > m[h] + kLazy) {
        const float f = __builtin_amdgcn_exp2f(m[h] - mx);
        m[h] = mx;
        l[h] *= f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool ok = rv[u] >= 0;  // rows outside the view read row 0 of the pool: drop its values
      const u32x4 w = {ok ? vb[u].x : 0u, ok ? vb[u].y : 0u, ok ? vb[u].z : 0u, ok ? vb[u].w : 0u};
      float x[EPL];
      V::widen(w, x);
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float p = __builtin_amdgcn_exp2f(sc[u][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
      }
    }
  };

  u32x4 ka[kUnroll], va[kUnroll], kb2[kUnroll], vb2[kUnroll];
  int ra[kUnroll], rb2[kUnroll];
  if (nit > 0) load(0, ka, va, ra);
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load(it + 1, kb2, vb2, rb2);
    step(it, ka, va, ra);
    if (it + 1 >= nit) break;
    if (it + 2 < nit) load(it + 2, ka, va, ra);
    step(it + 1, kb2, vb2, rb2);
  }

  if constexpr (kMfma) {
    // per head and lane-row: the head's max and the row's sum, from lane h of the row, in every lane of the row
    bcast_r<R>(ml, m);
    bcast_r<R>(ll, l);
  } else if constexpr (kOne) {
    // per head: the max every lane of the head holds, the sum over the head's four lanes, in every lane of the row
    float lsum = ll + dpp_f<kRowRor4>(ll);
    if constexpr (R == 4) lsum += dpp_f<kRowRor8>(lsum);
    m[0] = row16_bcast<0>(ml), l[0] = row16_bcast<0>(lsum);
    if constexpr (R > 1) m[1 % R] = row16_bcast<1 % R>(ml), l[1 % R] = row16_bcast<1 % R>(lsum);
    if constexpr (R > 2) {
      m[2 % R] = row16_bcast<2 % R>(ml), l[2 % R] = row16_bcast<2 % R>(lsum);
      m[3 % R] = row16_bcast<3 % R>(ml), l[3 % R] = row16_bcast<3 % R>(lsum);
    }
  }
  // merge the four lane-rows of the wave
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mo = __shfl_xor(m[h], off), lo = __shfl_xor(l[h], off);
      float mn = fmaxf(m[h], mo);
      float fa = __builtin_amdgcn_exp2f(m[h] - mn), fb = __builtin_amdgcn_exp2f(mo - mn);
      l[h] = l[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * fa + __shfl_xor(acc[h][e], off) * fb;
      m[h] = mn;
    }
  }
  // merge the waves through LDS and write the chunk's partial
  __shared__ float s_ml[4][R][2];
  __shared__ float s_acc[4][R][D];
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][cl * EPL + e] = acc[h][e];
      if (lane == 0) {
        s_ml[wave][h][0] = m[h];
        s_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  float *part = a.part + ((int64_t)unit * a.nchunk + chunk) * R * (D + 2);
  for (int i = threadIdx.x; i < R * D; i += kThreads) {
    int h = i / D, e = i % D;
    float mm = fmaxf(fmaxf(s_ml[0][h][0], s_ml[1][h][0]), fmaxf(s_ml[2][h][0], s_ml[3][h][0]));
    float ll = 0.f, oo = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float f = __builtin_amdgcn_exp2f(s_ml[w][h][0] - mm);
      ll += s_ml[w][h][1] * f;
      oo += s_acc[w][h][e] * f;
    }
    part[h * (D + 2) + 2 + e] = oo;
    if (e == 0) {
      part[h * (D + 2)] = mm;
      part[h * (D + 2) + 1] = ll;
    }
  }
}

constexpr int kMaxChunks = 4096;

// (max, sum) of head h over the chunks of a unit, computed by one full wave; lanes stride over chunks. When w is
// given, the per-chunk weights exp2(m_c - max) are stored there.
SE_DEV void merge_ml(const float *part, int nchunk, int R, int D, int h, float &mm, float &ll, float *w) {
  const int lane = threadIdx.x & 63;
  mm = -1e30f;
  for (int c = lane; c < nchunk; c += 64) mm = fmaxf(mm, part[(c * R + h) * (D + 2)]);
  mm = wave_max(mm);
  ll = 0.f;
  for (int c = lane; c < nchunk; c += 64) {
    const float wc = __builtin_amdgcn_exp2f(part[(c * R + h) * (D + 2)] - mm);
    if (w) w[c] = wc;
    ll += part[(c * R + h) * (D + 2) + 1] * wc;
  }
  ll = wave_sum(ll);
}

// one workgroup per (unit, head): merge the chunks' partial softmax states into the output row
template <int DTYPE, int R>
__global__ __launch_bounds__(128) void decode_merge(DecodeArgs a) {
  constexpr int D = 16 * Vec<DTYPE>::EPL;
  const int unit = blockIdx.x / R, h = blockIdx.x % R;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const float *part = a.part + (int64_t)unit * a.nchunk * R * (D + 2);
  __shared__ float s_w[kMaxChunks];
  __shared__ float s_l, s_m;
  if (threadIdx.x < 64) {
    float mm, ll;
    merge_ml(part, a.nchunk, R, D, h, mm, ll, s_w);
    if (threadIdx.x == 0) {
      s_l = ll;
      s_m = mm;
    }
  }
  __syncthreads();
  const float inv = s_l > 0.f ? 1.f / s_l : 0.f;
  if (a.mil && threadIdx.x == 0) {  // for decode_cum
    a.mil[((int64_t)unit * R + h) * 2] = s_m;
    a.mil[((int64_t)unit * R + h) * 2 + 1] = inv;
  }
  for (int e = threadIdx.x; e < D; e += 128) {
    float o = 0.f;
#pragma unroll 4
    for (int c = 0; c < a.nchunk; ++c) o += s_w[c] * part[(c * R + h) * (D + 2) + 2 + e];
    a.out[(((int64_t)b * a.n_kv + g) * R + h) * D + e] = o * inv;
  }
}

// cumulative scores: cum[slot] += sum over the group's heads of that head's softmax weight on the slot, from the
// stored logits and the merged (max, 1/sum) of each head
template <int DTYPE, int R>
__global__ __launch_bounds__(kThreads) void decode_cum(DecodeArgs a) {
  const int unit = blockIdx.y;
  float mm[R], il[R];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    mm[h] = a.mil[((int64_t)unit * R + h) * 2];
    il[h] = a.mil[((int64_t)unit * R + h) * 2 + 1];
  }
  ViewMap vm(a, unit);
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= vm.rows) return;
  const int s = vm.slot(r);
  if (s < 0) return;
  const float *lg = a.logits + ((int64_t)unit * a.rows_bound + r) * R;
  float x[R];
#pragma unroll
  for (int h = 0; h < R; ++h) x[h] = lg[h];
  if (x[0] == -INFINITY) return;  // free slot: not in the view
  float sum = 0.f;
#pragma unroll
  for (int h = 0; h < R; ++h) sum += __builtin_amdgcn_exp2f(x[h] - mm[h]) * il[h];
  a.cum[(int64_t)unit * a.max_blocks * a.page + s] += sum;
}

// Accumulating decode with the unit's logits kept in LDS: one workgroup of kUnitThreads per unit streams the
// whole view (each wave a contiguous run of 16-row steps), so the merged (max, sum) of every head is known inside
// the workgroup and the cumulative scores are updated from LDS: no partials, no logits in HBM, one launch. Used
// when the view is not page-selected and rows_bound * R logits fit kUnitLdsFloats. With one workgroup per CU,
// each wave keeps twice the split kernel's rows in flight.
constexpr int kUnitThreads = 512;
constexpr int kUnitWaves = kUnitThreads / 64;
constexpr int kUnitLdsFloats = 38912;  // 152 KiB
constexpr int kUnitMaxRows = 9984;     // and at most this many rows: 20 cumulative scores per thread
constexpr int U = 4;   // wave-loads per lane-row and step: 16 rows (8 KiB of K and V) per wave
constexpr int UG = 4;  // rows per lane-row whose scores are live at once
constexpr int NB = 4;  // K/V buffers: three steps in flight while one is computed

// With EV, H2O's eviction follows in the same workgroup (se_h2o_decode_evict): from the scores just updated, the
// resident slot with the lowest cumulative score among those at least `recent` positions below the newest resident
// one (ties: the higher position) is freed when the unit holds more than `budget` tokens: the selection of top-K's
// smallest mode with k = 1 and the slot eviction, on the same values.
template <int DTYPE, int R, bool EV>
SE_DEV void decode_unit_body(const DecodeArgs &a) {
  using V = Vec<DTYPE>;
  constexpr int EPL = V::EPL;
  constexpr int D = 16 * EPL;
  constexpr int RB = 256;
  constexpr int kMaxRows = kUnitLdsFloats / R < kUnitMaxRows ? kUnitLdsFloats / R : kUnitMaxRows;
  constexpr int kCum = (kMaxRows + kUnitThreads - 1) / kUnitThreads;
  constexpr int SR = 4 * U;  // rows per step: 4 lane-rows x U
  constexpr int SUB = NB * SR;  // rows per sub-chunk (NB steps), resolved one per lane
  const int unit = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lrow = lane >> 4, cl = lane & 15;
  __shared__ float s_lg[kUnitLdsFloats];
  __shared__ float s_ml[kUnitWaves][R][2];
  __shared__ float s_acc[R][D];
  __shared__ int s_evmx[EV ? kUnitWaves : 1];
  __shared__ uint64_t s_ev64[EV ? kUnitWaves : 1];

  u32x4 q[R];
#pragma unroll
  for (int h = 0; h < R; ++h) q[h] = ld16(a.q + (((int64_t)b * a.n_kv + g) * R + h) * RB + cl * 16);
  // bf16, d = 128: logits from MFMA in decode_partial's layout (lane-row lr's lanes 0..R-1 hold keys 4 lr + v)
  constexpr bool kMfma = DTYPE == SE_DTYPE_BF16 && EPL == 8;
  bf16x8 qf[4];
  if constexpr (kMfma) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qf[t] = __builtin_bit_cast(
          bf16x8, cl < R ? ld16(a.q + (((int64_t)b * a.n_kv + g) * R + (cl < R ? cl : 0)) * RB + t * 64 + lrow * 16)
                         : z);
    }
  }

  const int cap = a.max_blocks * a.page;
  int n = a.n_slots[unit];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  if (threadIdx.x == 0 && n > a.rows_bound) raise(a.status, SE_DEV_CAPACITY);
  const int rows = n < a.rows_bound ? n : a.rows_bound;
  const int nit_all = (rows + SR - 1) / SR;
  const int it0 = wave * nit_all / kUnitWaves, it1 = (wave + 1) * nit_all / kUnitWaves;
  const int nst = it1 - it0;  // this wave's steps: rows [wr0, wr1)
  const int wr0 = it0 * SR, wr1 = it1 * SR < rows ? it1 * SR : rows;
  const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  const int32_t *pos = a.pos + (int64_t)unit * cap;
  float *cum = a.cum + (int64_t)unit * cap;
  // EV: the unit's token count and slot-stack top, which only this workgroup changes during the call
  int ctxv = 0, topv = 0;
  if constexpr (EV) {
    ctxv = a.ev_ctx[unit];
    topv = a.ev_top[unit];
  }

  // Rows are resolved SUB at a time, lane i holding row wr0 + SUB k + i of sub-chunk k (pool row, or -1 when not
  // resident); a step takes its rows from that register with ds_bpermute. The block-table and position loads of
  // sub-chunk k + 2 go out while sub-chunk k streams (clamped addresses, no branch).
  bool bad = false;
  auto res_issue = [&](int k, int &blk, int &ps) {
    const int r = wr0 + SUB * k + lane;
    const int rr = lane < SUB && r < wr1 ? r : 0;
    blk = bt[rr / a.page];
    ps = pos[rr];
  };
  int mxp = -1;  // EV: the newest position among this lane's resolved rows
  auto res_make = [&](int k, int blk, int ps) {
    const int r = wr0 + SUB * k + lane;
    int v = -1;
    if (EV && lane < SUB && r < wr1) mxp = max(mxp, ps);
    if (lane < SUB && r < wr1 && ps >= 0) {
      if (blk_ok(blk, a.num_blocks)) v = (blk * a.n_kv + g) * a.page + r % a.page;
      else bad = true;
    }
    return v;
  };
  // rv[u]: the pool row of the step's row u * 4 + lrow (MFMA: of row lrow * 4 + u, the V rows, and rv[U] that of
  // row cl, the lane's key for the K fragments)
  auto rows_from = [&](int vs, int half, int (&rv)[U + 1]) {
    if constexpr (kMfma) {
#pragma unroll
      for (int u = 0; u < U; ++u) rv[u] = __builtin_amdgcn_ds_bpermute((half * SR + lrow * 4 + u) * 4, vs);
      rv[U] = __builtin_amdgcn_ds_bpermute((half * SR + cl) * 4, vs);
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) rv[u] = __builtin_amdgcn_ds_bpermute((half * SR + u * 4 + lrow) * 4, vs);
  };
  // waves whose rows end at least kUnitHotRows before the view's last row load non-temporally; the waves over the
  // most recent rows load plain (measured: a mix streams faster than either kind alone)
  const bool cold = wr1 <= rows - kUnitHotRows;  // uniform per wave
  auto load = [&](const int (&rv)[U + 1], u32x4 (&kb)[U], u32x4 (&vb)[U]) {
    if constexpr (kMfma) {
      const char *kr = a.k + (int64_t)(rv[U] >= 0 ? rv[U] : 0) * RB + lrow * 16;
      if (cold) {
#pragma unroll
        for (int t = 0; t < 4; ++t) kb[t] = ld16_stream(kr + t * 64);
#pragma unroll
        for (int u = 0; u < U; ++u) vb[u] = ld16_stream(a.v + (int64_t)(rv[u] >= 0 ? rv[u] : 0) * RB + cl * 16);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) kb[t] = ld16(kr + t * 64);
#pragma unroll
        for (int u = 0; u < U; ++u) vb[u] = ld16(a.v + (int64_t)(rv[u] >= 0 ? rv[u] : 0) * RB + cl * 16);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (int64_t)(rv[u] >= 0 ? rv[u] : 0) * RB + cl * 16;
      kb[u] = ld16_stream(a.k + off);
      vb[u] = ld16_stream(a.v + off);
    }
  };

  float m[R], l[R], acc[R][EPL];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -1e30f;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  // With R x U = 16, one logit per lane as in decode_partial (lane cl: row u = cl / R of the step, head cl % R),
  // which also writes it to LDS for the cumulative scores.
  constexpr bool kOne = R * U == 16;
  float ml = -1e30f, ll = 0.f;
  auto step1 = [&](int rbase, const u32x4 (&kb)[U], const u32x4 (&vb)[U], const int (&rv)[U + 1])
      __attribute__((always_inline)) {
    float d[16];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < R; ++h) d[(u * R + h) & 15] = V::dot(q[h], kb[u], 0.f);
    float s = row16_reduce_scatter(d);
    const int ul = cl / R, hl = cl % R;
    const int rvl = ul == 0 ? rv[0] : ul == 1 ? rv[1 % U] : ul == 2 ? rv[2 % U] : rv[3 % U];
    s = rvl >= 0 ? s * a.scale_log2 : -INFINITY;
    const int r = rbase + ul * 4 + lrow;
    if (r < rows) s_lg[r * R + hl] = s;
    float mx = fmaxf(s, dpp_f<kRowRor4>(s));
    if constexpr (R == 4) mx = fmaxf(mx, dpp_f<kRowRor8>(mx));
    if (__builtin_amdgcn_ballot_w64(mx > ml + kLazy)) {  // uniform, rare
      const float mn = mx > ml + kLazy ? mx : ml;
      const float f = __builtin_amdgcn_exp2f(ml - mn);
      ml = mn;
      ll *= f;
      float fh[R];
      fh[0] = row16_bcast<0>(f);
      if constexpr (R > 1) fh[1 % R] = row16_bcast<1 % R>(f);
      if constexpr (R > 2) fh[2 % R] = row16_bcast<2 % R>(f), fh[3 % R] = row16_bcast<3 % R>(f);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= fh[h];
    }
    const float p = __builtin_amdgcn_exp2f(s - ml);
    ll += p;
    float pj[16];
    pj[0] = row16_bcast<0>(p), pj[1] = row16_bcast<1>(p), pj[2] = row16_bcast<2>(p), pj[3] = row16_bcast<3>(p);
    pj[4] = row16_bcast<4>(p), pj[5] = row16_bcast<5>(p), pj[6] = row16_bcast<6>(p), pj[7] = row16_bcast<7>(p);
    pj[8] = row16_bcast<8>(p), pj[9] = row16_bcast<9>(p), pj[10] = row16_bcast<10>(p);
    pj[11] = row16_bcast<11>(p), pj[12] = row16_bcast<12>(p), pj[13] = row16_bcast<13>(p);
    pj[14] = row16_bcast<14>(p), pj[15] = row16_bcast<15>(p);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = rv[u] >= 0;
      const u32x4 w = {ok ? vb[u].x : 0u, ok ? vb[u].y : 0u, ok ? vb[u].z : 0u, ok ? vb[u].w : 0u};
      float x[EPL];
      V::widen(w, x);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pj[(u * R + h) & 15], x[e], acc[h][e]);
    }
  };
  auto stepm = [&](int rbase, const u32x4 (&kb)[U], const u32x4 (&vb)[U], const int (&rv)[U + 1])
      __attribute__((always_inline)) {
    floatx4 lg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) lg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[t]), qf[t],
                                                                           lg, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sv[v] = rv[v] >= 0 ? lg[v] * a.scale_log2 : -INFINITY;
    if (cl < R) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = rbase + lrow * 4 + v;
        if (r < rows) s_lg[r * R + cl] = sv[v];
      }
    }
    const float mx = cross_row_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    if (__builtin_amdgcn_ballot_w64(mx > ml + kLazy)) {  // uniform, rare
      const float mn = mx > ml + kLazy ? mx : ml;
      const float f = __builtin_amdgcn_exp2f(ml - mn);
      ml = mn;
      ll *= f;
      float fh[R];
      bcast_r<R>(f, fh);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= fh[h];
    }
    float pv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) pv[v] = __builtin_amdgcn_exp2f(sv[v] - ml);
    ll += (pv[0] + pv[1]) + (pv[2] + pv[3]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float ph[R];
      bcast_r<R>(pv[u], ph);
      const bool ok = rv[u] >= 0;
      const u32x4 w = {ok ? vb[u].x : 0u, ok ? vb[u].y : 0u, ok ? vb[u].z : 0u, ok ? vb[u].w : 0u};
      float x[EPL];
      V::widen(w, x);
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(ph[h], x[e], acc[h][e]);
    }
  };
  // one step in groups of UG rows per lane-row (fewer live scores)
  auto step = [&](int rbase, const u32x4 (&kb)[U], const u32x4 (&vb)[U], const int (&rv)[U + 1]) {
    if constexpr (kMfma) {
      stepm(rbase, kb, vb, rv);
      return;
    } else if constexpr (kOne) {
      step1(rbase, kb, vb, rv);
      return;
    }
#pragma unroll
    for (int hf = 0; hf < U / UG; ++hf) {
      float sc[UG][R];
#pragma unroll
      for (int uu = 0; uu < UG; ++uu) {
        const int u = hf * UG + uu;
#pragma unroll
        for (int h = 0; h < R; ++h) {
          const float d = row16_sum(V::dot(q[h], kb[u], 0.f));
          sc[uu][h] = rv[u] >= 0 ? d * a.scale_log2 : -INFINITY;
        }
        const int r = rbase + u * 4 + lrow;
        if (cl == 0 && r < rows) {
#pragma unroll
          for (int h = 0; h < R; ++h) s_lg[r * R + h] = sc[uu][h];
        }
      }
#pragma unroll
      for (int h = 0; h < R; ++h) {
        float mx = sc[0][h];
#pragma unroll
        for (int uu = 1; uu < UG; ++uu) mx = fmaxf(mx, sc[uu][h]);
        if (mx > m[h] + kLazy) {
          const float f = __builtin_amdgcn_exp2f(m[h] - mx);
          m[h] = mx;
          l[h] *= f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
        }
      }
#pragma unroll
      for (int uu = 0; uu < UG; ++uu) {
        const int u = hf * UG + uu;
        const bool ok = rv[u] >= 0;
        const u32x4 w = {ok ? vb[u].x : 0u, ok ? vb[u].y : 0u, ok ? vb[u].z : 0u, ok ? vb[u].w : 0u};
        float x[EPL];
        V::widen(w, x);
#pragma unroll
        for (int h = 0; h < R; ++h) {
          const float p = __builtin_amdgcn_exp2f(sc[uu][h] - m[h]);
          l[h] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
        }
      }
    }
  };

  // steps 4k .. 4k+3 form sub-chunk k and use buffers 0 .. 3; the K/V loads of the next three steps are in
  // flight while a step is computed
  static_assert(NB == 4, "the loop below is written for four buffers");
  int r0[U + 1], r1[U + 1], r2[U + 1], r3[U + 1], vcur = -1, rbk = 0, rpk = 0, rbn = 0, rpn = 0;
  u32x4 k0[U], v0[U], k1[U], v1[U], k2[U], v2[U], k3[U], v3[U];
  if (nst > 0) {
    res_issue(0, rbk, rpk);
    res_issue(1, rbn, rpn);
    vcur = res_make(0, rbk, rpk);
    rows_from(vcur, 0, r0);
    load(r0, k0, v0);
    if (nst > 1) {
      rows_from(vcur, 1, r1);
      load(r1, k1, v1);
    }
    if (nst > 2) {
      rows_from(vcur, 2, r2);
      load(r2, k2, v2);
    }
  }
  for (int k = 0; NB * k < nst; ++k) {
    const int j = NB * k;
    res_issue(k + 2, rbk, rpk);
    if (j + 3 < nst) {
      rows_from(vcur, 3, r3);
      load(r3, k3, v3);
    }
    step(wr0 + j * SR, k0, v0, r0);
    if (j + 1 >= nst) break;
    const int vnext = res_make(k + 1, rbn, rpn);
    if (j + 4 < nst) {
      rows_from(vnext, 0, r0);
      load(r0, k0, v0);
    }
    step(wr0 + (j + 1) * SR, k1, v1, r1);
    if (j + 2 >= nst) break;
    if (j + 5 < nst) {
      rows_from(vnext, 1, r1);
      load(r1, k1, v1);
    }
    step(wr0 + (j + 2) * SR, k2, v2, r2);
    if (j + 3 >= nst) break;
    if (j + 6 < nst) {
      rows_from(vnext, 2, r2);
      load(r2, k2, v2);
    }
    step(wr0 + (j + 3) * SR, k3, v3, r3);
    vcur = vnext;
    rbn = rbk;
    rpn = rpk;
  }
  if (bad) raise(a.status, SE_DEV_INDEX);

  if constexpr (kMfma) {
    bcast_r<R>(ml, m);
    bcast_r<R>(ll, l);
  } else if constexpr (kOne) {
    float lsum = ll + dpp_f<kRowRor4>(ll);
    if constexpr (R == 4) lsum += dpp_f<kRowRor8>(lsum);
    m[0] = row16_bcast<0>(ml), l[0] = row16_bcast<0>(lsum);
    if constexpr (R > 1) m[1 % R] = row16_bcast<1 % R>(ml), l[1 % R] = row16_bcast<1 % R>(lsum);
    if constexpr (R > 2) {
      m[2 % R] = row16_bcast<2 % R>(ml), l[2 % R] = row16_bcast<2 % R>(lsum);
      m[3 % R] = row16_bcast<3 % R>(ml), l[3 % R] = row16_bcast<3 % R>(lsum);
    }
  }
  // this thread's cumulative scores, loaded while the waves merge (with EV also its slots' positions, -1 past the
  // view, and the unit's token count)
  float cv[kCum];
#pragma unroll
  for (int k = 0; k < kCum; ++k) {
    const int r = k * kUnitThreads + threadIdx.x;
    cv[k] = cum[r < rows ? r : 0];
  }
  int pv[EV ? kCum : 1];
  if constexpr (EV) {
#pragma unroll
    for (int k = 0; k < kCum; ++k) {
      const int r = k * kUnitThreads + threadIdx.x;
      const int p = pos[r < rows ? r : 0];
      pv[k] = r < rows ? p : -1;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mxp = max(mxp, __shfl_xor(mxp, o));
    if (lane == 0) s_evmx[wave] = mxp;  // published with the waves' statistics below
  }

  // merge the four lane-rows of each wave, then the waves: max and sum first, then acc one wave at a time
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float mo = __shfl_xor(m[h], off), lo = __shfl_xor(l[h], off);
      float mn = fmaxf(m[h], mo);
      float fa = __builtin_amdgcn_exp2f(m[h] - mn), fb = __builtin_amdgcn_exp2f(mo - mn);
      l[h] = l[h] * fa + lo * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * fa + __shfl_xor(acc[h][e], off) * fb;
      m[h] = mn;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      s_ml[wave][h][0] = m[h];
      s_ml[wave][h][1] = l[h];
    }
  }
  __syncthreads();
  float M[R], iL[R];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    float mm = s_ml[0][h][0];
#pragma unroll
    for (int w = 1; w < kUnitWaves; ++w) mm = fmaxf(mm, s_ml[w][h][0]);
    float ll = 0.f;
#pragma unroll
    for (int w = 0; w < kUnitWaves; ++w) ll += s_ml[w][h][1] * __builtin_amdgcn_exp2f(s_ml[w][h][0] - mm);
    M[h] = mm;
    iL[h] = ll > 0.f ? 1.f / ll : 0.f;
  }
  for (int w = 0; w < kUnitWaves; ++w) {
    if (wave == w && lane < 16) {
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float f = __builtin_amdgcn_exp2f(m[h] - M[h]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float &dst = s_acc[h][cl * EPL + e];
          dst = (w == 0 ? 0.f : dst) + acc[h][e] * f;
        }
      }
    }
    __syncthreads();
  }
  float *out = a.out + (((int64_t)b * a.n_kv + g) * R) * D;
  for (int i = threadIdx.x; i < R * D; i += kUnitThreads) out[i] = s_acc[i / D][i % D] * iL[i / D];

  // cum[slot] += the group's summed weight on the slot; free slots (logit -inf) keep their value. With EV the
  // stores wait until the eviction has been chosen from the new values (the chosen slot's score becomes 0), so no
  // barrier below waits for them.
  uint32_t inview = 0;  // bit k: slot k * kUnitThreads + threadIdx.x gets a new score
#pragma unroll
  for (int k = 0; k < kCum; ++k) {
    const int r = k * kUnitThreads + threadIdx.x;
    if (r >= rows) break;
    if (s_lg[r * R] == -INFINITY) continue;
    float sum = 0.f;
#pragma unroll
    for (int h = 0; h < R; ++h) sum += __builtin_amdgcn_exp2f(s_lg[r * R + h] - M[h]) * iL[h];
    cv[k] += sum;
    if constexpr (EV) inview |= 1u << k;
    else cum[r] = cv[k];
  }
  if constexpr (EV) {
    // the newest resident position over every slot below n_slots (as in top-K), from the rows the waves resolved
    int mx = -1;
#pragma unroll
    for (int w = 0; w < kUnitWaves; ++w) mx = max(mx, s_evmx[w]);
    const int limit = mx - a.ev_recent;
    // this thread's candidate with the lowest score (ties: the higher position), by float comparisons (scores are
    // not NaN, and -0 equals +0 as in top-K's keys); then the largest (~key, ~tie key) pair over the workgroup,
    // packed as top-K's k = 1 path packs it (a candidate's pair is never 0)
    const bool over = ctxv - a.ev_budget > 0;
    float bv = 0.f;
    int bp = -1, br = -1;
#pragma unroll
    for (int k = 0; k < kCum; ++k) {
      const bool cand = over && pv[k] >= 0 && pv[k] <= limit;
      const bool better = bp < 0 || cv[k] < bv || (cv[k] == bv && pv[k] > bp);
      if (cand && better) {
        bv = cv[k];
        bp = pv[k];
        br = k * kUnitThreads + threadIdx.x;
      }
    }
    const uint64_t mine = bp >= 0 ? ((uint64_t)~orderable(bv) << 32) | (uint32_t)~(0x7fffffffu - (uint32_t)bp) : 0;
    uint64_t best = mine;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, o);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), o);
      const uint64_t y = ((uint64_t)hi << 32) | lo;
      best = y > best ? y : best;
    }
    if (lane == 0) s_ev64[wave] = best;
    // only LDS is exchanged here: wait for this wave's LDS write, not for its global accesses, then meet
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int w = 0; w < kUnitWaves; ++w) best = s_ev64[w] > best ? s_ev64[w] : best;
    // the chosen slot's thread frees it under the slot eviction's rules for one entry (a stack top outside
    // [0, cap) raises SE_DEV_CAPACITY and changes nothing); every other new score is stored as it is
    const bool room = topv >= 0 && topv < a.ev_cap;
    const int chosen_r = best != 0 && mine == best ? br : -1;  // this thread's slot, if it is the one chosen
#pragma unroll
    for (int k = 0; k < kCum; ++k) {
      const int r = k * kUnitThreads + threadIdx.x;
      const bool chosen = r == chosen_r;
      if ((inview >> k) & 1u) cum[r] = chosen && room ? 0.f : cv[k];
      if (!chosen) continue;
      a.ev_idx[unit] = r;
      if (!room) {
        raise(a.status, SE_DEV_CAPACITY);
      } else {
        a.ev_pos[(int64_t)unit * cap + r] = -1;
        if (!((inview >> k) & 1u)) cum[r] = 0.f;
        a.ev_stack[(int64_t)unit * a.ev_cap + topv] = r;
        a.ev_top[unit] = topv + 1;
        a.ev_ctx[unit] = ctxv - 1;
      }
    }
    if (threadIdx.x == 0) a.ev_count[unit] = best != 0 ? 1 : 0;
  }
}

template <int DTYPE, int R>
__global__ __launch_bounds__(kUnitThreads) void decode_unit(DecodeArgs a) {
  decode_unit_body<DTYPE, R, false>(a);
}
// the same with H2O's bottom-1 eviction after the cumulative scores (se_h2o_decode_evict)
template <int DTYPE, int R>
__global__ __launch_bounds__(kUnitThreads) void h2o_decode_unit(DecodeArgs a) {
  decode_unit_body<DTYPE, R, true>(a);
}

struct Plan {
  int rows_bound, chunk_rows, nchunk, units;
  bool unit_path;  // decode_unit: accumulate over all slots, logits fit in LDS
  size_t part_bytes, logit_bytes;
};

Plan make_plan(const se_cache_t *c, const se_decode_params_t *p, int has_sel) {
  Plan pl;
  int cap = c->max_blocks * c->page;
  if (has_sel) {
    pl.rows_bound = p->max_sel * c->page;
  } else {
    pl.rows_bound = p->max_slots > 0 && p->max_slots < cap ? p->max_slots : cap;
  }
  pl.units = c->B * c->n_kv;
  // the largest chunk (<= kMaxChunkRows) that still gives >= kMinWGs workgroups, else the smallest (64 rows)
  int ch = kMaxChunkRows;
  while (ch > 64 && (long long)pl.units * ((pl.rows_bound + ch - 1) / ch) < kMinWGs) ch /= 2;
  pl.chunk_rows = ch;
  pl.nchunk = (pl.rows_bound + ch - 1) / ch;
  if (pl.nchunk < 1) pl.nchunk = 1;
  int R = c->n_q / c->n_kv;
  pl.part_bytes = se_host::align_up((size_t)pl.units * pl.nchunk * R * (c->d + 2) * sizeof(float));
  pl.logit_bytes = p->accumulate ? se_host::align_up((size_t)pl.units * pl.rows_bound * R * sizeof(float)) +
                                       se_host::align_up((size_t)pl.units * R * 2 * sizeof(float))
                                 : 0;
  pl.unit_path = p->accumulate && !has_sel && (long long)pl.rows_bound * R <= kUnitLdsFloats &&
                 pl.rows_bound <= kUnitMaxRows;
  if (pl.unit_path) pl.part_bytes = pl.logit_bytes = 0;
  return pl;
}

template <int DTYPE, int R>
void launch(const DecodeArgs &a, int units, int nchunk, bool unit_path, hipStream_t st) {
  if (unit_path) {
    if (a.ev_idx) hipLaunchKernelGGL((h2o_decode_unit<DTYPE, R>), dim3(units), dim3(kUnitThreads), 0, st, a);
    else hipLaunchKernelGGL((decode_unit<DTYPE, R>), dim3(units), dim3(kUnitThreads), 0, st, a);
    return;
  }
  hipLaunchKernelGGL((decode_partial<DTYPE, R>), dim3(nchunk, units), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((decode_merge<DTYPE, R>), dim3(units * R), dim3(128), 0, st, a);
  if (a.cum)
    hipLaunchKernelGGL((decode_cum<DTYPE, R>), dim3((a.rows_bound + kThreads - 1) / kThreads, units), dim3(kThreads),
                       0, st, a);
}

template <int DTYPE>
int32_t dispatch_r(int R, const DecodeArgs &a, int units, int nchunk, bool unit_path, hipStream_t st) {
  switch (R) {
    case 1: launch<DTYPE, 1>(a, units, nchunk, unit_path, st); break;
    case 2: launch<DTYPE, 2>(a, units, nchunk, unit_path, st); break;
    case 4: launch<DTYPE, 4>(a, units, nchunk, unit_path, st); break;
    case 8: launch<DTYPE, 8>(a, units, nchunk, unit_path, st); break;
    default: return SE_ERR_UNSUPPORTED;
  }
  return se_host::launch_status();
}

}  // namespace
}  // namespace se

extern "C" size_t se_sparse_decode_attn_workspace_size(const se_cache_t *c, const se_decode_params_t *p,
                                                        int32_t has_sel) {
  if (se_host::check_cache(c) != SE_OK || !p) return 0;
  se::Plan pl = se::make_plan(c, p, has_sel);
  return pl.part_bytes + pl.logit_bytes;
}

namespace {

// H2O's eviction after an accumulating decode (se_h2o_decode_evict); null for a plain decode call
struct EvictSpec {
  int32_t budget, recent;
  int32_t *idx, *count;
};

int32_t decode_call(se_cache_t *c, const void *q, const int32_t *sel_pages, const int32_t *sel_count,
                    const se_decode_params_t *p, float *out, int32_t *status, void *ws, size_t ws_bytes,
                    se_stream_t stream, const EvictSpec *ev = nullptr) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!q || !out || !p) return SE_ERR_NULL;
  const int has_sel = sel_pages != nullptr;
  if (has_sel && !sel_count) return SE_ERR_NULL;
  if (has_sel && (p->max_sel <= 0 || p->sel_stride < p->max_sel)) return SE_ERR_SHAPE;
  if (p->max_slots < 0) return SE_ERR_PARAM;
  if (p->accumulate && !c->cum_score) return SE_ERR_NULL;
  const bool ok_shape = (c->dtype == SE_DTYPE_BF16 && c->d == 128) || (c->dtype == SE_DTYPE_F32 && c->d == 64);
  if (!ok_shape) return SE_ERR_DTYPE;
  se::Plan pl = se::make_plan(c, p, has_sel);
  if (pl.nchunk > se::kMaxChunks) return SE_ERR_UNSUPPORTED;  // views beyond 4M slots per (sequence, head)
  if ((long long)c->num_blocks * c->n_kv * c->page >= (1ll << 31)) return SE_ERR_UNSUPPORTED;
  if (pl.part_bytes + pl.logit_bytes > 0 && (ws_bytes < pl.part_bytes + pl.logit_bytes || !ws))
    return SE_ERR_WORKSPACE;
  se::DecodeArgs a;
  a.k = (const char *)c->k_pool;
  a.v = (const char *)c->v_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.q = (const char *)q;
  a.sel = sel_pages;
  a.sel_count = sel_count;
  a.out = out;
  a.part = (float *)ws;
  a.logits = p->accumulate ? (float *)((char *)ws + pl.part_bytes) : nullptr;
  a.cum = p->accumulate ? c->cum_score : nullptr;
  a.mil = p->accumulate ? (float *)((char *)ws + pl.part_bytes +
                                    se_host::align_up((size_t)pl.units * pl.rows_bound * (c->n_q / c->n_kv) * sizeof(float)))
                        : nullptr;
  a.status = status;
  a.n_kv = c->n_kv;
  a.page = c->page;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.sel_stride = has_sel ? p->sel_stride : 0;
  a.rows_bound = pl.rows_bound;
  a.chunk_rows = pl.chunk_rows;
  a.nchunk = pl.nchunk;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  const bool fused = ev && pl.unit_path;  // the eviction inside the single-workgroup decode
  a.ev_pos = fused ? c->pos_map : nullptr;
  a.ev_stack = fused ? c->slot_stack : nullptr;
  a.ev_top = fused ? c->slot_top : nullptr;
  a.ev_ctx = fused ? c->ctx_len : nullptr;
  a.ev_idx = fused ? ev->idx : nullptr;
  a.ev_count = fused ? ev->count : nullptr;
  a.ev_cap = fused ? c->slot_cap : 0;
  a.ev_budget = fused ? ev->budget : 0;
  a.ev_recent = fused ? ev->recent : 0;
  const int R = c->n_q / c->n_kv;
  hipStream_t st = (hipStream_t)stream;
  rc = c->dtype == SE_DTYPE_BF16 ? se::dispatch_r<SE_DTYPE_BF16>(R, a, pl.units, pl.nchunk, pl.unit_path, st)
                                 : se::dispatch_r<SE_DTYPE_F32>(R, a, pl.units, pl.nchunk, pl.unit_path, st);
  if (rc != SE_OK || !ev || fused) return rc;
  // the view is too long for one workgroup's LDS: bottom-1 and the slot eviction as their own calls
  se_topk_params_t tp{};
  tp.mode = SE_TOPK_SMALLEST;
  tp.unit = SE_UNIT_SLOT;
  tp.k = 1;
  tp.budget = ev->budget;
  tp.recent = ev->recent;
  tp.score_stride = c->max_blocks * c->page;
  tp.out_stride = 1;
  rc = se_topk_select(c, c->cum_score, &tp, ev->idx, ev->count, status, nullptr, 0, stream);
  if (rc != SE_OK) return rc;
  se_compact_params_t cp{};
  cp.mode = SE_COMPACT_EVICT_SLOTS;
  cp.idx_stride = 1;
  return se_compact_evict(c, ev->idx, ev->count, &cp, status, nullptr, 0, stream);
}

}  // namespace

extern "C" int32_t se_sparse_decode_attn(se_cache_t *c, const void *q, const int32_t *sel_pages,
                                         const int32_t *sel_count, const se_decode_params_t *p, float *out,
                                         int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream) {
  return decode_call(c, q, sel_pages, sel_count, p, out, status, ws, ws_bytes, stream);
}

namespace {
se_decode_params_t h2o_decode_params(const se_h2o_params_t *p) {
  se_decode_params_t d{};
  d.scale = p->scale;
  d.accumulate = 1;
  return d;
}
}  // namespace

extern "C" size_t se_h2o_decode_evict_workspace_size(const se_cache_t *c, const se_h2o_params_t *p) {
  if (!p) return 0;
  const se_decode_params_t d = h2o_decode_params(p);
  return se_sparse_decode_attn_workspace_size(c, &d, 0);
}

extern "C" int32_t se_h2o_decode_evict(se_cache_t *c, const void *q, const se_h2o_params_t *p, float *out,
                                       int32_t *evict_idx, int32_t *evict_count, int32_t *status, void *ws,
                                       size_t ws_bytes, se_stream_t stream) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!p || !evict_idx || !evict_count) return SE_ERR_NULL;
  if (!c->cum_score || !c->slot_stack || !c->slot_top || c->slot_cap <= 0) return SE_ERR_NULL;
  if (p->budget < 0 || p->recent < 0) return SE_ERR_PARAM;
  const se_decode_params_t d = h2o_decode_params(p);
  const EvictSpec ev{p->budget, p->recent, evict_idx, evict_count};
  return decode_call(c, q, nullptr, nullptr, &d, out, status, ws, ws_bytes, stream, &ev);
}

// ---- the allocation-free variant ------------------------------------------------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving loops): the split partials and the
// logits live in one file-scope device array per GPU, of SE_NOALLOC_SCRATCH_BYTES. Its device address is looked
// up once per device (the array's name in host code is only a stand-in for the symbol) and kept. Decode's
// scratch needs no initial value: every partial and logit is written before it is read.
static __device__ __align__(256) char scratch[SE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// the scratch array's device address on the current device (looked up at the first call there)
int32_t scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SE_ERR_UNSUPPORTED;
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SE_ERR_HIP;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return SE_OK;
}

}  // namespace

extern "C" int32_t se_sparse_decode_attn_noalloc(se_cache_t *c, const void *q, const int32_t *sel_pages,
                                                 const int32_t *sel_count, const se_decode_params_t *p, float *out,
                                                 int32_t *status, se_stream_t stream) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!p) return SE_ERR_NULL;
  const size_t need = se_sparse_decode_attn_workspace_size(c, p, sel_pages != nullptr);
  if (need > (size_t)SE_NOALLOC_SCRATCH_BYTES) return SE_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  if (need > 0 && (rc = scratch_address(&ws)) != SE_OK) return rc;
  return decode_call(c, q, sel_pages, sel_count, p, out, status, ws, need, stream);
}
