// CacheManager state changes (SparseEngine page, "How it works": physical eviction updates the retained
// slot mapping and context length and returns discarded slots to the allocator; KARA page, "Method" part 3:
// periodic compaction of trailing blocks):
//   se_compact_evict  GATHER       in-place keep-prefix compaction + block freeing
//                     EVICT_SLOTS  slot eviction onto the per-head slot stack
//   se_cache_append   one decode token per (sequence, KV head)
//   se_cache_append_chunk  T tokens per (sequence, KV head) at the high-water slots (a prefill chunk)
//
// In-place gather hazard. Output j of a (sequence, head) unit copies slot s_j to slot w0 + j, with s ascending
// and s_j >= w0 + j. Writing slot w0 + j destroys a source only if some output k < j reads s_k = w0 + j. Let
// h = #{j : s_j < w0 + cnt}; those outputs form a prefix, and so do the identity outputs (s_j = w0 + j,
// nothing to move), [0, i0). The only conflicting pairs are (reader k in [i0, h), writer s_k - w0). Workgroup
// 0 of each unit moves exactly that set S in ascending tiles (all reads of a tile before its writes); every
// other output reads a slot >= w0 + cnt, which nobody writes, and writes a slot no reader needs, so the other
// workgroups move them with no ordering at all (a unit with a single tile: workgroup 0, after S). Bit-exact,
// deterministic, one pass over the data.
#include "common.hpp"

namespace se {
namespace {

constexpr int kMoveRowsMax = 256;  // output rows per workgroup tile (rows <= 256 B; 128 rows for 512-B rows)
constexpr int kMoveThreads = 1024;
constexpr int kMovePer = 4;        // 16-byte K and V chunks held per thread in a tile
constexpr int kMaxBitmapWords = 2048;  // hazard bitmap: 65536 outputs per unit
constexpr int kIdxLds = 4096;          // retained-index lists up to this length are searched in LDS
constexpr int kWindowWords = 256;      // hazard outputs are listed 8192 at a time

struct GatherArgs {
  char *k, *v;
  const int32_t *bt;
  int32_t *pos;
  float *cum;
  const int32_t *n_slots, *idx, *count;
  int32_t *status;
  int32_t n_kv, page, max_blocks, num_blocks, row_bytes, window, idx_stride;
  int32_t fold;  // 1: a unit's outputs fit one tile, which workgroup 0 moves after the hazard set
};

struct UnitPlan {
  int n, cnt, w0, i0, h;
  bool ok;
};

// first j in [0, cnt) with pred(j) true, for a monotone predicate (cnt if none)
template <class F>
SE_DEV int lower_bound_pred(int cnt, F pred) {
  int lo = 0, hi = cnt;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (pred(mid)) hi = mid; else lo = mid + 1;
  }
  return lo;
}

SE_DEV UnitPlan plan_unit(const GatherArgs &a, int unit, const int32_t *s) {
  UnitPlan u;
  const int cap = a.max_blocks * a.page;
  u.n = a.n_slots[unit];
  u.cnt = a.count[unit];
  u.w0 = a.window > 0 ? u.n - a.window : 0;
  u.ok = u.n >= 0 && u.n <= cap && u.w0 >= 0 && u.cnt >= 0 && u.cnt <= u.n - u.w0 && u.cnt <= a.idx_stride;
  if (!u.ok) {
    u.cnt = 0;
    u.i0 = u.h = 0;
    return u;
  }
  const int lim = u.w0 + u.cnt, w0 = u.w0;
  u.h = lower_bound_pred(u.cnt, [&](int j) { return s[j] >= lim; });
  u.i0 = lower_bound_pred(u.cnt, [&](int j) { return s[j] - j > w0; });
  if (u.i0 > u.h) u.i0 = u.h;  // only possible for an invalid list, which is flagged below
  return u;
}

// is slot w0 + j the source of a hazardous reader k in [i0, h)?
SE_DEV bool is_hazard_dest(const int32_t *s, const UnitPlan &u, int j) {
  int lo = u.i0, hi = u.h, want = u.w0 + j;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (s[mid] < want) lo = mid + 1; else hi = mid;
  }
  return lo < u.h && s[lo] == want;
}

// Per-row move descriptors of a tile, prepared in LDS: byte offsets of the source and destination rows (-1: skip),
// the destination slot and the source row's position and cumulative score.
struct Tile {
  int64_t soff[kMoveRowsMax], doff[kMoveRowsMax];
  int dslot[kMoveRowsMax], pval[kMoveRowsMax];
  float cval[kMoveRowsMax];
};

// row r of the tile moves source slot ss to destination slot ds (ss < 0: nothing). The block table, position and
// cumulative-score loads depend only on the slots, so they are all in flight together.
SE_DEV void prepare_row(const GatherArgs &a, int b, int g, int unit, int r, int ss, int ds, Tile &t) {
  int64_t so = -1, dof = -1;
  int pv = -1;
  float cv = 0.f;
  if (ss >= 0) {
    const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
    const int64_t base = (int64_t)unit * a.max_blocks * a.page;
    const int sb = bt[ss / a.page], db = bt[ds / a.page];
    pv = a.pos[base + ss];
    if (a.cum) cv = a.cum[base + ss];
    if (blk_ok(sb, a.num_blocks) && blk_ok(db, a.num_blocks)) {
      so = (((int64_t)sb * a.n_kv + g) * a.page + ss % a.page) * a.row_bytes;
      dof = (((int64_t)db * a.n_kv + g) * a.page + ds % a.page) * a.row_bytes;
    }
  }
  t.soff[r] = so;
  t.doff[r] = dof;
  t.dslot[r] = ds;
  t.pval[r] = pv;
  t.cval[r] = cv;
}

// move the prepared rows of a tile; with ORDERED every read of the tile completes before its first write.
// nrows * row_bytes / 16 <= kMovePer * kMoveThreads.
template <bool ORDERED>
SE_DEV void move_tile(const GatherArgs &a, int unit, const Tile &t, int nrows) {
  const int cpr = a.row_bytes / 16;
  const int total = nrows * cpr;
  u32x4 kbuf[kMovePer], vbuf[kMovePer];
#pragma unroll
  for (int i = 0; i < kMovePer; ++i) {
    const int x = threadIdx.x + i * kMoveThreads;
    if (x >= total) continue;
    const int64_t so = t.soff[x / cpr];
    if (so < 0) continue;
    kbuf[i] = ld16_stream(a.k + so + (x % cpr) * 16);
    vbuf[i] = ld16_stream(a.v + so + (x % cpr) * 16);
  }
  if (ORDERED) __syncthreads();
  const int64_t base = (int64_t)unit * a.max_blocks * a.page;
#pragma unroll
  for (int i = 0; i < kMovePer; ++i) {
    const int x = threadIdx.x + i * kMoveThreads;
    if (x >= total) continue;
    const int r = x / cpr, ch = x % cpr;
    const int64_t so = t.soff[r], dof = t.doff[r];
    if (so < 0) continue;
    // plain stores: the decode that follows a compaction reads these rows, and finds them in the last-level cache
    st16(a.k + dof + ch * 16, kbuf[i]);
    st16(a.v + dof + ch * 16, vbuf[i]);
    if (ch == 0) {
      a.pos[base + t.dslot[r]] = t.pval[r];
      if (a.cum) a.cum[base + t.dslot[r]] = t.cval[r];
    }
  }
  if (ORDERED) __syncthreads();
}

template <int kMoveRows>
__global__ __launch_bounds__(kMoveThreads) void gather_move(GatherArgs a) {
  const int unit = blockIdx.y;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  __shared__ UnitPlan s_plan;
  __shared__ int s_idx[kIdxLds];
  __shared__ Tile s_tile;
  __shared__ uint32_t s_bits[kMaxBitmapWords];
  __shared__ int s_list[kWindowWords * 32];
  __shared__ int s_scan[kWindowWords];
  const int32_t *gidx = a.idx + (int64_t)unit * a.idx_stride;
  const int cnt_raw = a.count[unit];
  const bool in_lds = cnt_raw >= 0 && cnt_raw <= kIdxLds && cnt_raw <= a.idx_stride;
  if (in_lds)
    for (int j = threadIdx.x; j < cnt_raw; j += kMoveThreads) s_idx[j] = gidx[j];
  __syncthreads();
  const int32_t *s = in_lds ? s_idx : gidx;
  if (threadIdx.x == 0) s_plan = plan_unit(a, unit, s);
  __syncthreads();
  const UnitPlan u = s_plan;
  if (!u.ok) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise(a.status, SE_DEV_INDEX);
    return;
  }
  const int32_t *pos = a.pos + (int64_t)unit * a.max_blocks * a.page;
  const int lim = u.w0 + u.cnt;

  // free-running movers: outputs j >= h of tile j0 whose destination no hazardous reader needs. They touch no row
  // the hazard set does, so they move in any order with it: workgroup x >= 1 moves tile x - 1, or, when a unit has
  // a single tile, workgroup 0 moves it after the hazard set.
  auto free_tile = [&](int j0) {
    if (j0 >= u.cnt) return;  // uniform
    if (threadIdx.x < kMoveRows) {
      const int j = j0 + threadIdx.x;
      int src = -1;
      if (j < u.cnt && j >= u.h) {
        const int sj = s[j];
        const bool valid = sj >= lim && sj < u.n && (j == 0 || s[j - 1] < sj);
        if (!valid) raise(a.status, SE_DEV_INDEX);
        else if (!is_hazard_dest(s, u, j)) src = sj;
      }
      prepare_row(a, b, g, unit, threadIdx.x, src, u.w0 + j, s_tile);
      if (src >= 0 && s_tile.pval[threadIdx.x] < 0) {  // not resident
        raise(a.status, SE_DEV_INDEX);
        s_tile.soff[threadIdx.x] = -1;
      }
    }
    __syncthreads();
    move_tile<false>(a, unit, s_tile, kMoveRows);
  };
  if (blockIdx.x > 0) {
    free_tile((blockIdx.x - 1) * kMoveRows);
    return;
  }

  // workgroup 0: validate the prefix, mark the hazard set S = readers [i0, h) and their destinations, then move
  // S in ascending order, a tile of up to kMoveRows outputs at a time (reads of a tile before its writes)
  const int words = (u.cnt + 31) / 32;
  for (int i = threadIdx.x; i < words; i += kMoveThreads) s_bits[i] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < u.h; j += kMoveThreads) {
    int sj = s[j];
    bool valid = sj >= u.w0 + j && sj < lim && (j == 0 || s[j - 1] < sj) && pos[sj] >= 0;
    if (!valid) {
      raise(a.status, SE_DEV_INDEX);
      continue;
    }
    if (j >= u.i0 && sj != u.w0 + j) {
      atomicOr(&s_bits[j >> 5], 1u << (j & 31));
      int d = sj - u.w0;
      atomicOr(&s_bits[d >> 5], 1u << (d & 31));
    }
  }
  __syncthreads();
  for (int wbase = u.i0 >> 5; wbase < words; wbase += kWindowWords) {
    // list the marked outputs of this window of words in ascending order
    const int wi = wbase + threadIdx.x;
    const uint32_t bits = (threadIdx.x < kWindowWords && wi < words) ? s_bits[wi] : 0u;
    if (threadIdx.x < kWindowWords) s_scan[threadIdx.x] = __popc(bits);
    __syncthreads();
    for (int off = 1; off < kWindowWords; off <<= 1) {
      int x = (threadIdx.x < kWindowWords && threadIdx.x >= off) ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      if (threadIdx.x < kWindowWords) s_scan[threadIdx.x] += x;
      __syncthreads();
    }
    const int nlist = s_scan[kWindowWords - 1];
    if (threadIdx.x < kWindowWords) {
      int o = s_scan[threadIdx.x] - __popc(bits);
      for (uint32_t x = bits; x; x &= x - 1) s_list[o++] = wi * 32 + __ffs(x) - 1;
    }
    __syncthreads();
    for (int t0 = 0; t0 < nlist; t0 += kMoveRows) {
      if (threadIdx.x < kMoveRows) {
        int src = -1, j = 0;
        if (t0 + threadIdx.x < nlist) {
          j = s_list[t0 + threadIdx.x];
          const int sj = s[j];
          // outputs below h were validated above; an output j >= h listed here (its destination is a hazardous
          // reader's source) gets the free movers' checks: ascending, past the kept prefix, inside the unit
          const bool valid = j < u.h || (sj >= lim && sj < u.n && (j == 0 || s[j - 1] < sj));
          if (!valid) raise(a.status, SE_DEV_INDEX);
          else if (sj >= u.w0 && sj < u.n) src = sj;
        }
        prepare_row(a, b, g, unit, threadIdx.x, src, u.w0 + j, s_tile);
        if (src >= 0 && s_tile.pval[threadIdx.x] < 0) {  // not resident: flagged, not moved
          raise(a.status, SE_DEV_INDEX);
          s_tile.soff[threadIdx.x] = -1;
        }
      }
      __syncthreads();
      move_tile<true>(a, unit, s_tile, kMoveRows);
    }
  }
  if (a.fold) free_tile(0);  // move_tile<true> ended with a barrier: s_tile is free
}

// Small lists: when every unit keeps at most kSmallRows slots (Kara's trailing window: 166), a unit's whole move fits
// one workgroup, which reads every source row before it writes any destination: no order is needed and no hazard
// analysis. The list is checked first (ascending, inside [w0, n), resident, mapped blocks); a unit with a bad entry
// raises SE_DEV_INDEX and moves nothing.
constexpr int kSmallRows = 256;
constexpr int kSmallThreads = 512;
constexpr int kSmallPer = kSmallRows * 16 / kSmallThreads;  // 16-byte pieces of K (and of V) per thread, 256-B rows

__global__ __launch_bounds__(kSmallThreads) void gather_small(GatherArgs a) {
  const int unit = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  __shared__ int64_t s_soff[kSmallRows], s_doff[kSmallRows];  // byte offsets of the rows; -1: nothing to move
  __shared__ int s_pval[kSmallRows];
  __shared__ float s_cval[kSmallRows];
  __shared__ int s_bad, s_cnt, s_w0;
  const int32_t *idx = a.idx + (int64_t)unit * a.idx_stride;
  if (threadIdx.x == 0) {
    const int cap = a.max_blocks * a.page;
    const int n = a.n_slots[unit], cnt = a.count[unit];
    const int w0 = a.window > 0 ? n - a.window : 0;
    const bool ok = n >= 0 && n <= cap && w0 >= 0 && cnt >= 0 && cnt <= n - w0 && cnt <= a.idx_stride &&
                    cnt <= kSmallRows;
    s_bad = ok ? 0 : 1;
    s_cnt = ok ? cnt : 0;
    s_w0 = w0;
  }
  __syncthreads();
  const int cnt = s_cnt, w0 = s_w0, n = a.n_slots[unit];
  const int64_t base = (int64_t)unit * a.max_blocks * a.page;
  if (threadIdx.x < cnt) {
    const int j = threadIdx.x;
    const int sj = idx[j];
    const int prev = j > 0 ? idx[j - 1] : w0 - 1;
    const int dj = w0 + j;
    const bool in = sj >= dj && sj < n && prev < sj;  // ascending and inside the range: sj >= w0 + j follows
    const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
    const int ss = in ? sj : dj;
    const int sb = bt[ss / a.page], db = bt[dj / a.page];
    const int pv = a.pos[base + ss];
    s_pval[j] = pv;
    s_cval[j] = a.cum ? a.cum[base + ss] : 0.f;
    const bool ok = in && pv >= 0 && blk_ok(sb, a.num_blocks) && blk_ok(db, a.num_blocks);
    if (!ok) atomicOr(&s_bad, 1);
    s_soff[j] = ok && sj != dj ? (((int64_t)sb * a.n_kv + g) * a.page + sj % a.page) * a.row_bytes : -1;
    s_doff[j] = (((int64_t)(ok ? db : 0) * a.n_kv + g) * a.page + dj % a.page) * a.row_bytes;
  }
  __syncthreads();
  if (s_bad) {
    if (threadIdx.x == 0) raise(a.status, SE_DEV_INDEX);
    return;
  }
  const int cpr = a.row_bytes / 16, total = cnt * cpr;
  u32x4 kb[kSmallPer], vb[kSmallPer];
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const int x = threadIdx.x + i * kSmallThreads;
    if (x >= total) continue;
    const int64_t so = s_soff[x / cpr];
    if (so < 0) continue;
    kb[i] = ld16_stream(a.k + so + (x % cpr) * 16);
    vb[i] = ld16_stream(a.v + so + (x % cpr) * 16);
  }
  __syncthreads();  // every source row of the unit is read before any destination row is written
#pragma unroll
  for (int i = 0; i < kSmallPer; ++i) {
    const int x = threadIdx.x + i * kSmallThreads;
    if (x >= total) continue;
    const int r = x / cpr, ch = x % cpr;
    if (s_soff[r] < 0) continue;
    st16_stream(a.k + s_doff[r] + ch * 16, kb[i]);
    st16_stream(a.v + s_doff[r] + ch * 16, vb[i]);
  }
  if (threadIdx.x < cnt) {
    a.pos[base + w0 + threadIdx.x] = s_pval[threadIdx.x];
    if (a.cum) a.cum[base + w0 + threadIdx.x] = s_cval[threadIdx.x];
  }
}

struct FinalArgs {
  int32_t *bt, *n_slots, *ctx, *free_blocks, *free_top, *slot_stack, *slot_top;
  const int32_t *count;
  int32_t *ws;  // [0, B): blocks each sequence frees; [B, 2B): its new extent; [2B]: the free-stack top on entry
  int32_t *status;
  int32_t B, n_kv, page, max_blocks, num_blocks, slot_cap, window;
};

constexpr int kFinalThreads = 256;

SE_DEV bool unit_ok(const FinalArgs &a, int n, int cnt, int &w0) {
  const int cap = a.max_blocks * a.page;
  w0 = a.window > 0 ? n - a.window : 0;
  return n >= 0 && n <= cap && w0 >= 0 && cnt >= 0 && cnt <= n - w0;
}

// one workgroup per sequence: its new extent (max over heads of the kept prefix), its allocated extent (first
// unallocated table entry at or after it: allocated entries form a prefix), then the per-head counters and slot
// stacks. Writes how many blocks the sequence frees.
__global__ __launch_bounds__(kFinalThreads) void gather_extents(FinalArgs a) {
  __shared__ int s_new, s_old;
  const int b = blockIdx.x;
  const int cap = a.max_blocks * a.page;
  if (threadIdx.x == 0) {
    s_new = 0;
    s_old = a.max_blocks;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < a.n_kv; g += kFinalThreads) {
    const int unit = b * a.n_kv + g;
    const int n = a.n_slots[unit], cnt = a.count[unit];
    int w0;
    const int ext = unit_ok(a, n, cnt, w0) ? w0 + cnt : min(max(n, 0), cap);
    atomicMax(&s_new, (ext + a.page - 1) / a.page);
  }
  __syncthreads();
  const int new_ext = s_new;
  const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  for (int j = new_ext + threadIdx.x; j < a.max_blocks; j += kFinalThreads)
    if (bt[j] < 0) atomicMin(&s_old, j);
  for (int g = threadIdx.x; g < a.n_kv; g += kFinalThreads) {
    const int unit = b * a.n_kv + g;
    const int n = a.n_slots[unit], cnt = a.count[unit];
    int w0;
    if (!unit_ok(a, n, cnt, w0)) continue;
    int holes = 0;
    if (a.slot_cap > 0 && a.slot_stack) {
      const int top = min(max(a.slot_top[unit], 0), a.slot_cap);
      int kept = 0;
      int32_t *st = a.slot_stack + (int64_t)unit * a.slot_cap;
      for (int i = 0; i < top; ++i) {
        const int sl = st[i];
        if (sl >= w0) ++holes; else st[kept++] = sl;
      }
      a.slot_top[unit] = kept;
    }
    a.ctx[unit] = a.ctx[unit] - ((n - w0) - holes) + cnt;
    a.n_slots[unit] = w0 + cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.ws[b] = max(s_old - new_ext, 0);
    a.ws[a.B + b] = new_ext;
    if (b == 0) a.ws[2 * a.B] = *a.free_top;
  }
}

// one workgroup per sequence: push its freed blocks (ascending logical block) after those of the sequences before
// it; the offset is the sum of their counts. Nothing is pushed if the stack cannot take every freed block.
__global__ __launch_bounds__(kFinalThreads) void gather_push(FinalArgs a) {
  __shared__ int s_red[2][kFinalThreads / 64];
  const int b = blockIdx.x;
  const int top0 = a.ws[2 * a.B];
  if (top0 < 0 || top0 > a.num_blocks) {
    if (b == 0 && threadIdx.x == 0) raise(a.status, SE_DEV_CAPACITY);
    return;
  }
  int before = 0, total = 0;
  for (int i = threadIdx.x; i < a.B; i += kFinalThreads) {
    const int v = a.ws[i];
    total += v;
    if (i < b) before += v;
  }
  before = wave_sum_i(before);
  total = wave_sum_i(total);
  if ((threadIdx.x & 63) == 0) {
    s_red[0][threadIdx.x >> 6] = before;
    s_red[1][threadIdx.x >> 6] = total;
  }
  __syncthreads();
  before = total = 0;
#pragma unroll
  for (int w = 0; w < kFinalThreads / 64; ++w) {
    before += s_red[0][w];
    total += s_red[1][w];
  }
  if (top0 + total > a.num_blocks) {
    if (b == 0 && threadIdx.x == 0) raise(a.status, SE_DEV_CAPACITY);
    return;
  }
  const int mine = a.ws[b], new_ext = a.ws[a.B + b];
  int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  for (int i = threadIdx.x; i < mine; i += kFinalThreads) {
    a.free_blocks[top0 + before + i] = bt[new_ext + i];
    bt[new_ext + i] = -1;
  }
  if (b == 0 && threadIdx.x == 0) *a.free_top = top0 + total;
}

// ---- slot eviction ------------------------------------------------------------------------------------------------
struct EvictArgs {
  int32_t *pos, *ctx, *slot_stack, *slot_top;
  float *cum;
  const int32_t *n_slots, *idx, *count;
  int32_t *status;
  int32_t units, max_slots, slot_cap, idx_stride;
};

// One workgroup per unit; its list (ascending, distinct) in chunks of kEvictThreads x kEvictPer entries, thread t
// taking kEvictPer consecutive entries of a chunk (their loads in flight together). Valid entries are pushed on
// the slot stack in list order (rank by a block scan of per-thread counts); entries past the stack's capacity
// are not evicted and raise SE_DEV_CAPACITY, invalid ones (not resident, out of range, out of order) raise
// SE_DEV_INDEX.
constexpr int kEvictThreads = 256;
constexpr int kEvictPer = 8;
__global__ __launch_bounds__(kEvictThreads) void evict_slots_kernel(EvictArgs a) {
  __shared__ int s_wave[kEvictThreads / 64];
  const int unit = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int cnt = a.count[unit], n = a.n_slots[unit], top = a.slot_top[unit];
  if (cnt < 0 || cnt > a.idx_stride) {
    if (t == 0) raise(a.status, SE_DEV_INDEX);
    return;
  }
  if (top < 0 || top > a.slot_cap) {
    if (t == 0) raise(a.status, SE_DEV_CAPACITY);
    return;
  }
  int32_t *pos = a.pos + (int64_t)unit * a.max_slots;
  int32_t *st = a.slot_stack + (int64_t)unit * a.slot_cap;
  const int32_t *list = a.idx + (int64_t)unit * a.idx_stride;
  int pushed = 0;  // valid entries of the chunks before this one
  for (int c0 = 0; c0 < cnt; c0 += kEvictThreads * kEvictPer) {
    const int i0 = c0 + t * kEvictPer;
    int s[kEvictPer], ps[kEvictPer];
    const int prev = i0 > 0 && i0 < cnt ? list[i0 - 1] : -1;
#pragma unroll
    for (int e = 0; e < kEvictPer; ++e) s[e] = i0 + e < cnt ? list[i0 + e] : -1;
#pragma unroll
    for (int e = 0; e < kEvictPer; ++e) {
      const bool in = s[e] >= 0 && s[e] < n && s[e] < a.max_slots;
      ps[e] = pos[in ? s[e] : 0];
    }
    uint32_t valid = 0;
    int mine = 0;
#pragma unroll
    for (int e = 0; e < kEvictPer; ++e) {
      if (i0 + e >= cnt) continue;
      const int before_e = e == 0 ? prev : s[e - 1];
      const bool ok = s[e] >= 0 && s[e] < n && s[e] < a.max_slots && before_e < s[e] && ps[e] >= 0;
      if (ok) {
        valid |= 1u << e;
        ++mine;
      } else {
        raise(a.status, SE_DEV_INDEX);
      }
    }
    // exclusive rank of this thread's first valid entry among the chunk's valid ones
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = incl - mine, total = 0;
#pragma unroll
    for (int w = 0; w < kEvictThreads / 64; ++w) {
      before += w < wave ? s_wave[w] : 0;
      total += s_wave[w];
    }
    __syncthreads();  // s_wave is rewritten by the next chunk
    int at = top + pushed + before;
#pragma unroll
    for (int e = 0; e < kEvictPer; ++e) {
      if (!((valid >> e) & 1u)) continue;
      if (at < a.slot_cap) {
        pos[s[e]] = -1;
        if (a.cum) a.cum[(int64_t)unit * a.max_slots + s[e]] = 0.f;
        st[at] = s[e];
      } else {
        raise(a.status, SE_DEV_CAPACITY);
      }
      ++at;
    }
    pushed += total;
  }
  if (t == 0) {
    const int done = min(pushed, a.slot_cap - top);
    a.slot_top[unit] = top + done;
    a.ctx[unit] -= done;
  }
}

// ---- append -------------------------------------------------------------------------------------------------------
struct AppendArgs {
  char *k, *v;
  int32_t *bt, *pos, *ctx, *n_slots, *free_blocks, *free_top, *slot_stack, *slot_top;
  float *cum;
  const char *k_new, *v_new;
  const int32_t *pos_new;
  int32_t *dst_row;  // workspace: per unit, the pool row its new token goes to (-1: none)
  int32_t *status;
  int32_t B, n_kv, page, max_blocks, num_blocks, slot_cap, row_bytes;
};

constexpr int kAppendThreads = 1024;  // plan workgroup; 256 threads when the call has at most 256 units or sequences
constexpr int kAppendThreadsSmall = 256;
constexpr int kMaxUnits = 4096;
constexpr int kAppendMaxSeq = 2048;

// Plan and maps, one workgroup: decide every slot and block first, then commit only if the whole call fits, and
// hand each unit's destination pool row to append_copy through the workspace (-1: nothing to copy).
template <int NTH>
__global__ __launch_bounds__(NTH) void append_plan(AppendArgs a) {
  __shared__ int s_slot[kMaxUnits];
  __shared__ int s_lb[kAppendMaxSeq];   // logical block sequence b lacks (-1 = none)
  __shared__ int s_pop[kAppendMaxSeq];  // free-stack index it pops from
  __shared__ int s_wsum[NTH / 64];
  __shared__ int s_fail;
  const int units = a.B * a.n_kv;
  const int cap = a.max_blocks * a.page;
  if (threadIdx.x == 0) s_fail = 0;
  // loads that depend on nothing go out first: the free-stack top and each unit's high-water mark
  const int top0 = *a.free_top;
  __syncthreads();
  for (int unit = threadIdx.x; unit < units; unit += NTH) {
    int top = a.slot_cap > 0 ? a.slot_top[unit] : 0;
    const int hw = a.n_slots[unit];
    if (top < 0 || top > a.slot_cap) {
      atomicOr(&s_fail, 1);
      top = 0;
    }
    int slot = top > 0 ? a.slot_stack[(int64_t)unit * a.slot_cap + top - 1] : hw;
    if (slot < 0 || slot >= cap) {
      atomicOr(&s_fail, 1);
      slot = 0;
    }
    s_slot[unit] = slot;
  }
  __syncthreads();
  // per sequence: the logical block its heads lack, if any (allocated entries form a prefix, so a single
  // token per head can only enter one new block; heads that lack different blocks are an index error). One
  // thread per head; the sequence's answer is gathered with LDS min/max.
  __shared__ int s_lbmin[kAppendMaxSeq];
  for (int b = threadIdx.x; b < a.B; b += NTH) {
    s_lb[b] = -1;
    s_lbmin[b] = 0x7fffffff;
  }
  __syncthreads();
  for (int unit = threadIdx.x; unit < units; unit += NTH) {
    const int b = unit / a.n_kv;
    const int lb = s_slot[unit] / a.page;
    const int cur = a.bt[(int64_t)b * a.max_blocks + lb];
    if (cur >= a.num_blocks) atomicOr(&s_fail, 1);
    if (cur < 0) {
      atomicMax(&s_lb[b], lb);
      atomicMin(&s_lbmin[b], lb);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < a.B; b += NTH)
    if (s_lb[b] >= 0 && s_lbmin[b] != s_lb[b]) atomicOr(&s_fail, 2);
  __syncthreads();
  // exclusive scan of the pops over sequences, in sequence order
  int carry = 0;
  if (top0 < 0 || top0 > a.num_blocks) {
    if (threadIdx.x == 0) raise(a.status, SE_DEV_CAPACITY);
    for (int unit = threadIdx.x; unit < units; unit += NTH) a.dst_row[unit] = -1;
    return;
  }
  for (int base = 0; base < a.B; base += NTH) {
    const int b = base + threadIdx.x;
    const int v = (b < a.B && s_lb[b] >= 0) ? 1 : 0;
    int total;
    const int before = block_exscan<NTH>(v, s_wsum, total);
    if (v) {
      const int idx = top0 - 1 - (carry + before);
      const int blk = idx >= 0 ? a.free_blocks[idx] : -1;
      if (blk < 0 || blk >= a.num_blocks) atomicOr(&s_fail, 4);
      s_pop[b] = blk;
    }
    carry += total;
  }
  __syncthreads();  // s_fail and s_pop complete
  if (s_fail) {
    if (threadIdx.x == 0) raise(a.status, s_fail == 2 ? SE_DEV_INDEX : SE_DEV_CAPACITY);
    for (int unit = threadIdx.x; unit < units; unit += NTH) a.dst_row[unit] = -1;
    return;  // all or nothing: nothing was written
  }
  for (int b = threadIdx.x; b < a.B; b += NTH)
    if (s_lb[b] >= 0) a.bt[(int64_t)b * a.max_blocks + s_lb[b]] = s_pop[b];
  __syncthreads();
  if (threadIdx.x == 0) *a.free_top = top0 - carry;
  // with few units (the 256-thread plan) the rows are copied here as well, with no second launch
  constexpr bool kCopy = NTH == kAppendThreadsSmall;
  __shared__ int s_dst[kCopy ? kAppendThreadsSmall : 1];
  for (int unit = threadIdx.x; unit < units; unit += NTH) {
    int b = unit / a.n_kv;
    int slot = s_slot[unit];
    int top = a.slot_cap > 0 ? a.slot_top[unit] : 0;
    if (top > 0) a.slot_top[unit] = top - 1; else a.n_slots[unit] = slot + 1;
    a.pos[(int64_t)unit * cap + slot] = a.pos_new[b];
    a.ctx[unit] += 1;
    if (a.cum) a.cum[(int64_t)unit * cap + slot] = 0.f;
    const int blk = a.bt[(int64_t)b * a.max_blocks + slot / a.page];
    const int row = (blk * a.n_kv + unit % a.n_kv) * a.page + slot % a.page;
    a.dst_row[unit] = row;
    if constexpr (kCopy) s_dst[unit] = row;
  }
  if constexpr (kCopy) {
    __syncthreads();
    const int cpr = a.row_bytes / 16;
    for (int x = threadIdx.x; x < units * cpr; x += NTH) {
      const int unit = x / cpr, ch = x % cpr;
      const int64_t src = (int64_t)unit * a.row_bytes + ch * 16, dst = (int64_t)s_dst[unit] * a.row_bytes + ch * 16;
      const u32x4 kr = ld16_stream(a.k_new + src), vr = ld16_stream(a.v_new + src);
      st16_stream(a.k + dst, kr);
      st16_stream(a.v + dst, vr);
    }
  }
}

// Data: one thread per 16 bytes of a new K row and V row, to the pool row the plan chose
constexpr int kCopyThreads = 256;
__global__ __launch_bounds__(kCopyThreads) void append_copy(AppendArgs a) {
  const int cpr = a.row_bytes / 16;
  const int t = blockIdx.x * kCopyThreads + threadIdx.x;
  if (t >= a.B * a.n_kv * cpr) return;
  const int unit = t / cpr, ch = t % cpr;
  const int row = a.dst_row[unit];
  if (row < 0) return;
  const int64_t src = (int64_t)unit * a.row_bytes + ch * 16, dst = (int64_t)row * a.row_bytes + ch * 16;
  const u32x4 kr = ld16_stream(a.k_new + src), vr = ld16_stream(a.v_new + src);
  st16_stream(a.k + dst, kr);
  st16_stream(a.v + dst, vr);
}

// ---- chunk append: T tokens per unit at the high-water slots -------------------------------------------------------
struct ChunkArgs {
  char *k, *v;
  int32_t *bt, *pos, *ctx, *n_slots, *free_blocks, *free_top;
  float *cum;
  const char *k_new, *v_new;
  const int32_t *pos0;
  const int32_t *counts;  // tokens of each sequence (<= T), or NULL: T for every sequence
  int32_t *flag;  // workspace: 1 when chunk_plan committed the call
  int32_t *status;
  int32_t B, n_kv, page, max_blocks, num_blocks, row_bytes, T;
};

// tokens appended to sequence b (-1: a count outside [0, T], which fails the call)
SE_DEV int chunk_count(const ChunkArgs &a, int b) {
  if (!a.counts) return a.T;
  const int c = a.counts[b];
  return c >= 0 && c <= a.T ? c : -1;
}

// One workgroup: per sequence the logical blocks its heads' new slots [n, n + T) need beyond the allocated prefix;
// pops for them in (sequence, logical block) order; then, only if everything fits, the commit: block table,
// free-stack top, n_slots and ctx_len. chunk_write copies the rows afterwards.
template <int NTH>
__global__ __launch_bounds__(NTH) void chunk_plan(ChunkArgs a) {
  __shared__ int s_first[kAppendMaxSeq], s_last[kAppendMaxSeq], s_alloc[kAppendMaxSeq], s_need[kAppendMaxSeq];
  __shared__ int s_before[kAppendMaxSeq];
  __shared__ int s_wsum[NTH / 64];
  __shared__ int s_fail;
  const int units = a.B * a.n_kv;
  const int cap = a.max_blocks * a.page;
  if (threadIdx.x == 0) {
    s_fail = 0;
    *a.flag = 0;
  }
  for (int b = threadIdx.x; b < a.B; b += NTH) {
    s_first[b] = -1;
    s_last[b] = -1;
    s_alloc[b] = 0x7fffffff;
  }
  __syncthreads();
  // blocks below the largest n / page of a sequence's heads hold resident slots, so they are allocated; its new
  // slots reach block (largest n + T - 1) / page
  for (int unit = threadIdx.x; unit < units; unit += NTH) {
    const int n = a.n_slots[unit], b = unit / a.n_kv;
    const int tb = chunk_count(a, b);
    if (tb < 0 || n < 0 || n + tb > cap) {
      atomicOr(&s_fail, 1);
      continue;
    }
    if (tb == 0) continue;
    atomicMax(&s_first[b], n / a.page);
    atomicMax(&s_last[b], (n + tb - 1) / a.page);
  }
  __syncthreads();
  // the first unallocated table entry in each sequence's window [first, last] (allocated entries form a
  // prefix), over all (sequence, entry) pairs at once; a window spans at most `span` entries
  const int span = (a.T + a.page - 1) / a.page + 1;
  for (int x = threadIdx.x; x < a.B * span; x += NTH) {
    const int b = x / span, j = s_first[b] + x % span;
    if (s_first[b] < 0 || j > s_last[b]) continue;
    const int cur = a.bt[(int64_t)b * a.max_blocks + j];
    if (cur >= a.num_blocks) atomicOr(&s_fail, 2);
    if (cur < 0) atomicMin(&s_alloc[b], j);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < a.B; b += NTH) {
    const int l = s_last[b], al = s_alloc[b];
    s_need[b] = (l >= 0 && al <= l) ? l - al + 1 : 0;
  }
  __syncthreads();
  const int top0 = *a.free_top;
  if (top0 < 0 || top0 > a.num_blocks) {
    if (threadIdx.x == 0) raise(a.status, SE_DEV_CAPACITY);
    return;
  }
  // exclusive scan of the needs over sequences: sequence b pops free_blocks[top0 - 1 - (s_before[b] + i)]
  int carry = 0;
  for (int base = 0; base < a.B; base += NTH) {
    const int b = base + threadIdx.x;
    const int v = b < a.B ? s_need[b] : 0;
    int total;
    const int before = block_exscan<NTH>(v, s_wsum, total);
    if (b < a.B) s_before[b] = carry + before;
    carry += total;
  }
  if (threadIdx.x == 0 && carry > top0) s_fail |= 1;
  __syncthreads();
  if (s_fail) {
    if (threadIdx.x == 0) raise(a.status, (s_fail & 2) ? SE_DEV_INDEX : SE_DEV_CAPACITY);
    return;  // all or nothing: nothing was written
  }
  for (int b = threadIdx.x; b < a.B; b += NTH)
    for (int i = 0; i < s_need[b]; ++i)
      a.bt[(int64_t)b * a.max_blocks + s_alloc[b] + i] = a.free_blocks[top0 - 1 - (s_before[b] + i)];
  for (int unit = threadIdx.x; unit < units; unit += NTH) {
    const int tb = chunk_count(a, unit / a.n_kv);
    a.n_slots[unit] += tb;
    a.ctx[unit] += tb;
  }
  if (threadIdx.x == 0) {
    *a.free_top = top0 - carry;
    *a.flag = 1;
  }
}

// grid (row tiles, units): copy the chunk's K/V rows of a unit into its new slots n_slots - T + t, set positions
// pos0[b] + t and clear cumulative scores; nothing when chunk_plan did not commit
constexpr int kChunkThreads = 256;
__global__ __launch_bounds__(kChunkThreads) void chunk_write(ChunkArgs a) {
  if (*a.flag != 1) return;
  const int unit = blockIdx.y, b = unit / a.n_kv, g = unit % a.n_kv;
  const int cap = a.max_blocks * a.page;
  const int cpr = a.row_bytes / 16;
  const int rows = kChunkThreads / cpr;  // rows per workgroup
  const int tb = chunk_count(a, b);
  const int base = a.n_slots[unit] - tb;
  const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  const int t = blockIdx.x * rows + threadIdx.x / cpr, ch = threadIdx.x % cpr;
  if (t >= tb) return;
  const int slot = base + t;
  const int blk = bt[slot / a.page];
  const int64_t src = ((int64_t)unit * a.T + t) * a.row_bytes + ch * 16;
  const int64_t dst = (((int64_t)blk * a.n_kv + g) * a.page + slot % a.page) * a.row_bytes + ch * 16;
  const u32x4 kr = ld16_stream(a.k_new + src), vr = ld16_stream(a.v_new + src);
  st16_stream(a.k + dst, kr);
  st16_stream(a.v + dst, vr);
  if (ch == 0) {
    a.pos[(int64_t)unit * cap + slot] = a.pos0[b] + t;
    if (a.cum) a.cum[(int64_t)unit * cap + slot] = 0.f;
  }
}

}  // namespace
}  // namespace se

extern "C" size_t se_compact_evict_workspace_size(const se_cache_t *c, const se_compact_params_t *p) {
  if (se_host::check_cache(c) != SE_OK || !p || p->mode != SE_COMPACT_GATHER) return 0;
  return se_host::align_up((size_t)(2 * c->B + 1) * sizeof(int32_t));
}

extern "C" int32_t se_compact_evict(se_cache_t *c, const int32_t *idx, const int32_t *count,
                                    const se_compact_params_t *p, int32_t *status, void *ws, size_t ws_bytes,
                                    se_stream_t stream) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!idx || !count || !p) return SE_ERR_NULL;
  if (p->idx_stride <= 0 || p->window < 0) return SE_ERR_PARAM;
  hipStream_t st = (hipStream_t)stream;
  const int units = c->B * c->n_kv;
  const int row_bytes = c->d * se::elem_bytes(c->dtype);
  if (row_bytes % 16 != 0 || row_bytes > 512) return SE_ERR_DTYPE;
  if (p->mode == SE_COMPACT_GATHER) {
    if (!c->free_blocks || !c->free_top) return SE_ERR_NULL;
    if (p->idx_stride > 32 * se::kMaxBitmapWords) return SE_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < se_compact_evict_workspace_size(c, p)) return SE_ERR_WORKSPACE;
    se::GatherArgs a;
    a.k = (char *)c->k_pool;
    a.v = (char *)c->v_pool;
    a.bt = c->block_table;
    a.pos = c->pos_map;
    a.cum = c->cum_score;
    a.n_slots = c->n_slots;
    a.idx = idx;
    a.count = count;
    a.status = status;
    a.n_kv = c->n_kv;
    a.page = c->page;
    a.max_blocks = c->max_blocks;
    a.num_blocks = c->num_blocks;
    a.row_bytes = row_bytes;
    a.window = p->window;
    a.idx_stride = p->idx_stride;
    if (p->idx_stride <= se::kSmallRows && row_bytes <= 256) {
      // every unit's move fits one workgroup: all reads, then all writes
      hipLaunchKernelGGL(se::gather_small, dim3(units), dim3(se::kSmallThreads), 0, st, a);
    } else {
      // workgroup 0 moves the hazard set, workgroup x >= 1 tile x - 1; a unit with one tile takes one workgroup
      const int tile_rows = row_bytes <= 256 ? 256 : 128;
      const int nt = (p->idx_stride + tile_rows - 1) / tile_rows;
      a.fold = nt <= 1;
      const dim3 grid(a.fold ? 1 : nt + 1, units);
      if (row_bytes <= 256) hipLaunchKernelGGL(se::gather_move<256>, grid, dim3(se::kMoveThreads), 0, st, a);
      else hipLaunchKernelGGL(se::gather_move<128>, grid, dim3(se::kMoveThreads), 0, st, a);
    }
    se::FinalArgs f;
    f.bt = c->block_table;
    f.n_slots = c->n_slots;
    f.ctx = c->ctx_len;
    f.free_blocks = c->free_blocks;
    f.free_top = c->free_top;
    f.slot_stack = c->slot_stack;
    f.slot_top = c->slot_top;
    f.count = count;
    f.status = status;
    f.B = c->B;
    f.n_kv = c->n_kv;
    f.page = c->page;
    f.max_blocks = c->max_blocks;
    f.num_blocks = c->num_blocks;
    f.slot_cap = (c->slot_stack && c->slot_top) ? c->slot_cap : 0;
    f.window = p->window;
    f.ws = (int32_t *)ws;
    hipLaunchKernelGGL(se::gather_extents, dim3(c->B), dim3(se::kFinalThreads), 0, st, f);
    hipLaunchKernelGGL(se::gather_push, dim3(c->B), dim3(se::kFinalThreads), 0, st, f);
    return se_host::launch_status();
  }
  if (p->mode == SE_COMPACT_EVICT_SLOTS) {
    if (!c->slot_stack || !c->slot_top || c->slot_cap <= 0) return SE_ERR_NULL;
    se::EvictArgs a;
    a.pos = c->pos_map;
    a.ctx = c->ctx_len;
    a.slot_stack = c->slot_stack;
    a.slot_top = c->slot_top;
    a.cum = c->cum_score;
    a.n_slots = c->n_slots;
    a.idx = idx;
    a.count = count;
    a.status = status;
    a.units = units;
    a.max_slots = c->max_blocks * c->page;
    a.slot_cap = c->slot_cap;
    a.idx_stride = p->idx_stride;
    hipLaunchKernelGGL(se::evict_slots_kernel, dim3(units), dim3(se::kEvictThreads), 0, st, a);
    return se_host::launch_status();
  }
  return SE_ERR_PARAM;
}

extern "C" size_t se_cache_append_workspace_size(const se_cache_t *c) {
  if (se_host::check_cache(c) != SE_OK) return 0;
  return se_host::align_up((size_t)c->B * c->n_kv * sizeof(int32_t));
}

extern "C" int32_t se_cache_append(se_cache_t *c, const void *k_new, const void *v_new, const int32_t *pos,
                                   int32_t *status, void *ws, size_t ws_bytes, se_stream_t stream) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!k_new || !v_new || !pos || !c->free_blocks || !c->free_top) return SE_ERR_NULL;
  if (c->slot_cap > 0 && (!c->slot_stack || !c->slot_top)) return SE_ERR_NULL;
  if (c->B * c->n_kv > se::kMaxUnits || c->B > se::kAppendMaxSeq) return SE_ERR_UNSUPPORTED;
  if ((long long)c->num_blocks * c->n_kv * c->page >= (1ll << 31)) return SE_ERR_UNSUPPORTED;  // 32-bit row ids
  const int row_bytes = c->d * se::elem_bytes(c->dtype);
  if (row_bytes % 16 != 0) return SE_ERR_DTYPE;
  if (!ws || ws_bytes < se_cache_append_workspace_size(c)) return SE_ERR_WORKSPACE;
  se::AppendArgs a;
  a.k = (char *)c->k_pool;
  a.v = (char *)c->v_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.ctx = c->ctx_len;
  a.n_slots = c->n_slots;
  a.free_blocks = c->free_blocks;
  a.free_top = c->free_top;
  a.slot_stack = c->slot_stack;
  a.slot_top = c->slot_top;
  a.cum = c->cum_score;
  a.k_new = (const char *)k_new;
  a.v_new = (const char *)v_new;
  a.pos_new = pos;
  a.status = status;
  a.B = c->B;
  a.n_kv = c->n_kv;
  a.page = c->page;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.slot_cap = c->slot_cap;
  a.row_bytes = row_bytes;
  a.dst_row = (int32_t *)ws;
  hipStream_t st = (hipStream_t)stream;
  if (c->B * c->n_kv <= se::kAppendThreadsSmall)
    hipLaunchKernelGGL(se::append_plan<se::kAppendThreadsSmall>, dim3(1), dim3(se::kAppendThreadsSmall), 0, st, a);
  else
    hipLaunchKernelGGL(se::append_plan<se::kAppendThreads>, dim3(1), dim3(se::kAppendThreads), 0, st, a);
  if (c->B * c->n_kv > se::kAppendThreadsSmall) {  // the small plan copies the rows itself
    const int pieces = c->B * c->n_kv * (row_bytes / 16);
    hipLaunchKernelGGL(se::append_copy, dim3((pieces + se::kCopyThreads - 1) / se::kCopyThreads),
                       dim3(se::kCopyThreads), 0, st, a);
  }
  return se_host::launch_status();
}

extern "C" size_t se_cache_append_chunk_workspace_size(const se_cache_t *c, int32_t T) {
  (void)T;
  if (se_host::check_cache(c) != SE_OK) return 0;
  return se_host::align_up(sizeof(int32_t));
}

extern "C" int32_t se_cache_append_chunk(se_cache_t *c, const void *k_new, const void *v_new, const int32_t *pos0,
                                         int32_t T, const int32_t *counts, int32_t *status, void *ws,
                                         size_t ws_bytes, se_stream_t stream) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!k_new || !v_new || !pos0 || !c->free_blocks || !c->free_top) return SE_ERR_NULL;
  if (T < 1 || (long long)T > (long long)c->max_blocks * c->page) return SE_ERR_PARAM;
  if (c->B > se::kAppendMaxSeq) return SE_ERR_UNSUPPORTED;
  const int row_bytes = c->d * se::elem_bytes(c->dtype);
  if (row_bytes % 16 != 0 || row_bytes > 512) return SE_ERR_DTYPE;
  if (!ws || ws_bytes < se_cache_append_chunk_workspace_size(c, T)) return SE_ERR_WORKSPACE;
  se::ChunkArgs a;
  a.k = (char *)c->k_pool;
  a.v = (char *)c->v_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.ctx = c->ctx_len;
  a.n_slots = c->n_slots;
  a.free_blocks = c->free_blocks;
  a.free_top = c->free_top;
  a.cum = c->cum_score;
  a.k_new = (const char *)k_new;
  a.v_new = (const char *)v_new;
  a.pos0 = pos0;
  a.counts = counts;
  a.flag = (int32_t *)ws;
  a.status = status;
  a.B = c->B;
  a.n_kv = c->n_kv;
  a.page = c->page;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.row_bytes = row_bytes;
  a.T = T;
  hipStream_t st = (hipStream_t)stream;
  if (c->B * c->n_kv <= se::kAppendThreadsSmall)
    hipLaunchKernelGGL(se::chunk_plan<se::kAppendThreadsSmall>, dim3(1), dim3(se::kAppendThreadsSmall), 0, st, a);
  else
    hipLaunchKernelGGL(se::chunk_plan<se::kAppendThreads>, dim3(1), dim3(se::kAppendThreads), 0, st, a);
  const int rows = se::kChunkThreads / (row_bytes / 16);
  hipLaunchKernelGGL(se::chunk_write, dim3((T + rows - 1) / rows, c->B * c->n_kv), dim3(se::kChunkThreads), 0, st, a);
  return se_host::launch_status();
}
