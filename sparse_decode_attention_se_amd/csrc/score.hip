// Observation-window attention scores.
//   CAUSAL (SnapKV at the prefill finish_step hook, SparseEngine page "How it works"): the window queries attend
//     causally over all resident keys; softmax weights are summed per key over queries and the GQA group.
//   BIDIR (KARA page, "Method" part 1): every window query scores the compressible region (window minus its
//     protected tail) with no mask; weights are summed the same way.
//
// Per (sequence, KV head) unit the R*Wq query rows of the group form a matrix Q and the keys a matrix K. The row
// softmax needs each row's global normaliser before any weight can be added to a key, so the work is two passes
// over QK^T: pass 1 streams K in chunks and sums exp2(s) per row (with an exact running-max fallback for rows
// whose sums leave a safe range); pass 2 merges the chunks' (reference, sum) pairs, recomputes QK^T and adds
// exp2(s - ref - log2 sum) into per-key column sums. For bf16 (d = 128) QK^T runs on MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate); fp32 inputs use a plain VALU path. A workgroup covers up to 256
// query rows and one key chunk; with several row groups, a last kernel sums their column sums. When one chunk holds
// a unit's whole key range and every wave has at most two steps, a single kernel does both passes.
#include <type_traits>

#include "common.hpp"

namespace se {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// query rows per workgroup of the fp32 VALU path (one thread per row); the MFMA path picks 128 or 256 per call
constexpr int kValuRows = 128;

struct ScoreArgs {
  const char *k;
  const int32_t *bt, *pos, *n_slots;
  const char *q;
  const int32_t *q_pos;
  float *scores;
  float *stats;    // [units][nrg][nkc][256][2] (max, sum) in the log2 domain
  float *colpart;  // [units][nrg][key_span] when nrg > 1
  int32_t *status;
  int32_t mode, n_kv, R, wq, page, max_blocks, num_blocks, window, protect, score_stride;
  int32_t page_shift;  // log2(page) when page is a power of two, else -1
  int32_t nrg, nkc, kc, key_span;
  int32_t rpg;  // query rows per row group (workgroup)
  int32_t accumulate;  // add the scores to what the output holds (H2O cumulative scores)
  float scale_log2;
};

// the one write of a key's score (added to the output's value when accumulating)
SE_DEV void put_score(const ScoreArgs &a, int64_t at, float v) { a.scores[at] = a.accumulate ? a.scores[at] + v : v; }

// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its own L2. The (chunk, row group, unit)
// item of a workgroup is remapped so that every XCD takes a contiguous range of items: the row groups of a unit,
// which stream the same keys, run on one XCD close together in time and share its L2.
SE_DEV void xcd_item(int &chunk, int &rg, int &unit) {
  constexpr int kXcd = 8;
  const int nx = gridDim.x, ny = gridDim.y;
  const int total = nx * ny * gridDim.z;
  const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int per = total / kXcd, rem = total % kXcd;
  const int x = lin % kXcd, i = lin / kXcd;
  const int item = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
  chunk = item % nx;
  rg = (item / nx) % ny;
  unit = item / (nx * ny);
}

// key range of a unit: [k0, k1) slots; scores index = slot - k0
SE_DEV void key_range(const ScoreArgs &a, int unit, int &k0, int &k1, int &n) {
  n = a.n_slots[unit];
  n = min(max(n, 0), a.max_blocks * a.page);
  if (a.mode == SE_SCORE_CAUSAL) {
    k0 = 0;
    k1 = n;
  } else {
    k0 = n - a.window;
    k1 = k0 + (a.window - a.protect);
    if (k0 < 0) {  // a window longer than the unit's slots: an index error, and nothing is scored
      if (threadIdx.x == 0) raise(a.status, SE_DEV_INDEX);
      k0 = k1 = 0;
    }
  }
}

// position limit of query row rho (in the unit's row space); -1 = row does not exist
SE_DEV int row_limit(const ScoreArgs &a, int b, int rho) {
  if (rho >= a.R * a.wq) return -1;
  if (a.mode != SE_SCORE_CAUSAL) return 0x7fffffff;
  return a.q_pos[(int64_t)b * a.wq + rho % a.wq];
}

SE_DEV const char *q_row(const ScoreArgs &a, int b, int g, int rho, int row_bytes) {
  int h = rho / a.wq, t = rho % a.wq;
  return a.q + ((((int64_t)b * a.n_kv + g) * a.R + h) * a.wq + t) * row_bytes;
}

// merge the per-chunk statistics of this workgroup's 256 rows into log2(sum) + max (or +inf for empty rows)
SE_DEV float merge_row(const ScoreArgs &a, int unit, int rg, int r) {
  const float *st = a.stats + (((int64_t)unit * a.nrg + rg) * a.nkc * a.rpg + r) * 2;
  float mm = -1e30f, ll = 0.f;
  int c = 0;
  for (; c + 8 <= a.nkc; c += 8) {  // eight independent loads in flight
    float m8[8], l8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m8[i] = st[(int64_t)(c + i) * a.rpg * 2];
      l8[i] = st[(int64_t)(c + i) * a.rpg * 2 + 1];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float mn = fmaxf(mm, m8[i]);
      ll = ll * __builtin_amdgcn_exp2f(mm - mn) + l8[i] * __builtin_amdgcn_exp2f(m8[i] - mn);
      mm = mn;
    }
  }
  for (; c < a.nkc; ++c) {
    const float m1 = st[(int64_t)c * a.rpg * 2], l1 = st[(int64_t)c * a.rpg * 2 + 1];
    const float mn = fmaxf(mm, m1);
    ll = ll * __builtin_amdgcn_exp2f(mm - mn) + l1 * __builtin_amdgcn_exp2f(m1 - mn);
    mm = mn;
  }
  return ll > 0.f ? mm + __log2f(ll) : INFINITY;
}

SE_DEV void merge_stats(const ScoreArgs &a, int unit, int rg, float *s_mlog) {
  s_mlog[threadIdx.x] = merge_row(a, unit, rg, threadIdx.x);
}


// A wave's step is KB 16-key tiles: KB = 2 where the chunk's keys come from HBM (one row group), 4 where several
// row groups read the same keys and mostly hit the L2.
#ifndef SE_STREAM_NSET
#define SE_STREAM_NSET 2
#endif
constexpr int kNSet = SE_STREAM_NSET;  // register sets of keys per wave (kNSet - 1 steps in flight)
static_assert(kNSet >= 2, "the fused kernel keeps two steps in registers");

// Pass 1 first sums exp2(s c) with no reference subtracted. A row whose chunk sum lies in [2^-80, 2^80] has every
// term finite, and the terms flushed to zero (each below 2^-126, at most 2^15 of them) are under 2^-31 of the sum,
// so the sum is as exact as one taken against the row's maximum. A chunk with a row outside that band (or with a
// non-finite sum) is streamed again with a lazy running max: a row's reference m only moves (and its sum is
// rescaled) when a logit exceeds it by more than kLazy / c in log2 units; until then the terms are exp2 of at most
// kLazy, which fp32 sums hold exactly enough.
constexpr float kLazy = 8.f;
constexpr float kPlainLo = 0x1p-80f, kPlainHi = 0x1p80f;

// max of four values that are finite or -inf: two v_max3_f32, without the NaN-quieting copies fmaxf would add.
// Only for VALU results: inline asm is outside the compiler's hazard checks, and an MFMA result needs wait states
// before a VALU instruction may read it.
SE_DEV float max4(float a, float b, float c, float d) {
  float t, r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(t) : "v"(a), "v"(b), "v"(c));
  asm("v_max3_f32 %0, %1, %2, %2" : "=v"(r) : "v"(t), "v"(d));
  return r;
}

// ---- MFMA path (bf16, d = 128) -------------------------------------------------------------------------------
// S^T = K Q^T per 16x16 tile: A = 16 keys x 32 dims, held in registers, B = 32 dims x 16 query rows, read from LDS.
// Lane l receives query row l%16 and keys 4*(l/16)..+4 of the tile. K-step t covers dims 32t..32t+32 (lane group
// h = l/16 holds dims 32t + 8h..+8), so each key load instruction reads 64 contiguous bytes of 16 rows.
// Each wave streams its own steps of the chunk straight from global memory (the next step's loads in flight while
// the current one is computed): K never passes through LDS and no barrier separates the steps, so the waves of a
// SIMD drift apart and one wave's MFMAs run while another does its softmax work. Where the keys come from HBM,
// steps of 32 keys (two tiles) rather than 64 keep the wave's loads in smaller, more frequent batches, which the
// memory system serves with less queueing, for twice the query-fragment reads from LDS per MFMA.
constexpr int kStreamRows = 256;
constexpr int kStreamQB = kStreamRows / 16;  // 16-row query blocks

// one step of a wave: the K fragments of its 16-key tiles and, per tile, the position of the key this lane loads
// (tile row l%16; -1: outside the chunk or not resident)
template <int KB>
struct KStep {
  bf16x8 f[KB][4];  // [key tile][k-step]
  int pos[KB];
};

// the block-table entries and positions of a step's keys (loaded a step before the keys themselves)
template <int KB>
struct KAddr {
  int blk[KB], pos[KB], page[KB];
};

// every load is issued unconditionally (indices clamped into the chunk), so none waits behind a branch
// the page of a slot: a shift when the page size is a power of two (no integer division in the hot loop)
template <bool POW2>
SE_DEV int page_of(const ScoreArgs &a, int slot) {
  return POW2 ? slot >> a.page_shift : slot / a.page;
}

template <bool POW2, int KB>
SE_DEV void kaddr_load(const ScoreArgs &a, int b, int g, int c0, int c1, int step, KAddr<KB> &ad) {
  const int lane = threadIdx.x & 63;
  const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  const int32_t *pos = a.pos + ((int64_t)b * a.n_kv + g) * a.max_blocks * a.page;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = min(c0 + step * 16 * KB + kb * 16 + (lane & 15), c1 - 1);
    ad.page[kb] = page_of<POW2>(a, key);
    ad.blk[kb] = bt[ad.page[kb]];
    ad.pos[kb] = pos[key];
  }
}

template <bool POW2, int KB>
SE_DEV void kstep_fetch(const ScoreArgs &a, int g, int c0, int c1, int step, const KAddr<KB> &ad, KStep<KB> &ks) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = c0 + step * 16 * KB + kb * 16 + (lane & 15);
    const bool ok = (key < c1) & (ad.pos[kb] >= 0) & ((unsigned)ad.blk[kb] < (unsigned)a.num_blocks);
    const int keep = -(int)ok;  // all ones or zero: arithmetic instead of a select the compiler may branch on
    const int off = POW2 ? (key & (a.page - 1)) : key - ad.page[kb] * a.page;
    const int row = ((ad.blk[kb] * a.n_kv + g) * a.page + off) & keep;
    ks.pos[kb] = (ad.pos[kb] & keep) | ~keep;
    const char *src = a.k + (int64_t)row * 256 + (lane >> 4) * 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) ks.f[kb][t] = __builtin_bit_cast(bf16x8, ld16(src + t * 64));
  }
}

// B fragment (query block qb, k-step t) from the swizzled Q rows in LDS: piece p of row r sits at
// r * 256 + ((p ^ (r % 16)) * 16), so the 16 rows a read touches fall in distinct bank groups
SE_DEV bf16x8 q_frag(const char *s_q, int qb, int t) {
  const int lane = threadIdx.x & 63;
  const int r = qb * 16 + (lane & 15);
  const int piece = t * 4 + (lane >> 4);
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(s_q + r * 256 + ((piece ^ (lane & 15)) << 4)));
}

// PRIO: the MFMAs are issued at raised wave priority, so that the other wave of the SIMD, in its softmax work, takes
// the issue slots between them (pass 1, which holds its row statistics in registers, has no room for the change)
template <bool PRIO = false, int KB>
SE_DEV void stile(const KStep<KB> &ks, const bf16x8 (&qf)[4], floatx4 (&acc)[KB]) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) acc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (PRIO) __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ks.f[kb][t], qf[t], acc[kb], 0, 0, 0);
  if (PRIO) __builtin_amdgcn_s_setprio(0);
}

// max of 16 values that are VALU results (never MFMA results: the asm is outside the compiler's hazard checks,
// and an MFMA result needs wait states before a VALU instruction may read it)
SE_DEV float maxv(const float (&x)[16]) {
  return fmaxf(fmaxf(max4(x[0], x[1], x[2], x[3]), max4(x[4], x[5], x[6], x[7])),
               fmaxf(max4(x[8], x[9], x[10], x[11]), max4(x[12], x[13], x[14], x[15])));
}
SE_DEV float maxv(const float (&x)[8]) { return fmaxf(max4(x[0], x[1], x[2], x[3]), max4(x[4], x[5], x[6], x[7])); }

// keys of the lane's outputs that its query row may not see become -inf (the row's limit and the keys' positions
// come from LDS: s_kp holds the positions of the wave's keys of this step)
template <int KB>
SE_DEV void stream_mask(const int *s_kp, int lim, floatx4 (&acc)[KB]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = s_kp[kb * 16 + (lane >> 4) * 4 + v];
      acc[kb][v] = (p >= 0 && p <= lim) ? acc[kb][v] : -INFINITY;
    }
}

// PASS 1: row statistics of the chunk; PASS 2: column sums with the merged statistics. PASS 3 (a unit's whole key
// range in one chunk of at most two steps per wave): both, in one workgroup, with the keys kept in registers and
// the row statistics merged in LDS.
template <int PASS, int NW, bool POW2, int KB>
__global__ __launch_bounds__(NW * 64, 2) void window_stream(ScoreArgs a) {
  constexpr int NT = NW * 64;
  constexpr int kKB = KB, kSub = 16 * KB;  // tiles and keys per step of a wave
  int chunk, rg, unit;
  xcd_item(chunk, rg, unit);
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ __attribute__((aligned(16))) char s_q[kStreamRows * 256];
  __shared__ int s_lim[kStreamRows];
  __shared__ int s_kp[NW][kSub];
  __shared__ int s_limmin;
  __shared__ float2 s_st3[PASS == 3 ? NW * kStreamRows : 1];  // fused: per-wave row statistics
  __shared__ float s_ml3[PASS == 3 ? kStreamRows : 1];        // fused: merged statistic per row
  __shared__ float s_ml2[PASS == 2 ? kStreamRows : 1];        // pass 2: the chunks' statistics merged per row
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int c0 = k0 + chunk * a.kc, c1 = min(c0 + a.kc, k1);
  if (PASS != 1 && c0 >= c1) return;  // uniform: nothing to score in this chunk
  const int nsub = c1 > c0 ? (c1 - c0 + kSub - 1) / kSub : 0;
  const int rows = min(kStreamRows, a.R * a.wq - rg * kStreamRows);

  // the wave's first step, and the addresses of its second, are in flight while the query rows are staged
  // kNSet register sets of keys (step j in ks[j % kNSet], its addresses in ad[j % kNSet]): the keys of the next
  // kNSet - 1 steps are in flight while a step is computed
  KStep<KB> ks[kNSet];
  KAddr<KB> ad[kNSet];
  int s = __builtin_amdgcn_readfirstlane(wave);
  // ph maps a wave's step order to the step it scores. Each workgroup starts its walk at its own step (rot), so
  // that the concurrent workgroups, whose chunks sit at large power-of-two strides in the pool, read from different
  // memory banks at any moment. Pass 2 walks the same ring backwards from there: the keys pass 1 read last are the
  // likeliest still to be in the last-level cache. The fused kernel (PASS 3) walks in order.
  const int rot = PASS != 3 && nsub > 0 ? (unit * 7 + chunk * 5 + rg * 3) % nsub : 0;
  auto ph = [&](int x) {
    const int y = PASS == 2 ? rot - 1 - x : rot + x;
    return y < 0 ? y + nsub : (y >= nsub ? y - nsub : y);
  };
  auto prime = [&]() __attribute__((always_inline)) {
    if (s < nsub) {
#pragma unroll
      for (int p = 0; p < kNSet - 1; ++p) {
        kaddr_load<POW2>(a, b, g, c0, c1, ph(min(s + p * NW, nsub - 1)), ad[p]);
        kstep_fetch<POW2>(a, g, c0, c1, ph(min(s + p * NW, nsub - 1)), ad[p], ks[p]);
      }
      kaddr_load<POW2>(a, b, g, c0, c1, ph(min(s + (kNSet - 1) * NW, nsub - 1)), ad[kNSet - 1]);
      if (PASS == 3 && kNSet == 2) kstep_fetch<POW2>(a, g, c0, c1, min(s + NW, nsub - 1), ad[1], ks[1]);
    }
  };
  prime();

  if (threadIdx.x == 0) s_limmin = 0x7fffffff;
  const char *qbase = a.q + (((int64_t)b * a.n_kv + g) * a.R * a.wq + (int64_t)rg * kStreamRows) * 256;
  constexpr int kPieces = kStreamRows * 16 / NT;
  u32x4 qv[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {  // rows past the last are read from row 0 and stored as zeros
    const int i = threadIdx.x + j * NT;
    qv[j] = ld16(qbase + (int64_t)((i >> 4) < rows ? i : (i & 15)) * 16);
  }
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int i = threadIdx.x + j * NT, r = i >> 4, p = i & 15;
    const bool in = r < rows;
    const u32x4 v = {in ? qv[j].x : 0u, in ? qv[j].y : 0u, in ? qv[j].z : 0u, in ? qv[j].w : 0u};
    *reinterpret_cast<u32x4 *>(s_q + r * 256 + ((p ^ (r & 15)) << 4)) = v;
  }
  __syncthreads();  // s_limmin initialised
  for (int r = threadIdx.x; r < kStreamRows; r += NT) {
    const int lim = row_limit(a, b, rg * kStreamRows + r);
    s_lim[r] = lim;
    if (lim >= 0) atomicMin(&s_limmin, lim);
    if (PASS == 2) s_ml2[r] = merge_row(a, unit, rg, r);  // max + log2(sum) of every chunk's statistics
  }
  __syncthreads();
  const int limmin = s_limmin;
  const int nqb = (rows + 15) / 16;
  const float c = a.scale_log2;

  // pass 1: per query block, the lane's running sum of exp2(s c - m c) over its keys, and -m c (0 on the first,
  // reference-free stream). On the lazy stream the reference m starts at the first visible logit and afterwards
  // only moves up, when a logit exceeds it by more than kLazy / c.
  float st_l[kStreamQB], st_nmc[kStreamQB];
  // pass 2: per query block, the merged statistic of the lane's row (+inf: no such row)
  float ml[kStreamQB];
  if (PASS != 2) {
#pragma unroll
    for (int qb = 0; qb < kStreamQB; ++qb) st_l[qb] = 0.f, st_nmc[qb] = 0.f;
  } else {
#pragma unroll
    for (int qb = 0; qb < kStreamQB; ++qb) {
      const int r = qb * 16 + (lane & 15);
      ml[qb] = r < rows ? s_ml2[r] : INFINITY;
    }
  }

  auto step = [&](const KStep<KB> &ks, int sidx, auto pass_tag) __attribute__((always_inline)) {
    constexpr int P = decltype(pass_tag)::value;
    int pmin = ks.pos[0], pmax = ks.pos[0];
#pragma unroll
    for (int kb = 1; kb < kKB; ++kb) pmin = min(pmin, ks.pos[kb]), pmax = max(pmax, ks.pos[kb]);
    const bool fast = __builtin_amdgcn_ballot_w64(!(pmin >= 0 && pmax <= limmin)) == 0;
    if (!fast) {
      if (lane < 16) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) s_kp[wave][kb * 16 + lane] = ks.pos[kb];
      }
      // LDS accesses of a wave complete in order; this keeps the compiler from moving the reads above the writes
      asm volatile("" ::: "memory");
    }
    float col[4 * kKB];
#pragma unroll
    for (int i = 0; i < 4 * kKB; ++i) col[i] = 0.f;
    // Outside the (rare) lazy-reference stream, the query fragments of block qb + 1 are read from LDS while block
    // qb's softmax work runs.
    constexpr bool kAhead = P != 1;
    bf16x8 qn[4];
    if (kAhead) {
#pragma unroll
      for (int t = 0; t < 4; ++t) qn[t] = q_frag(s_q, 0, t);
    }
#pragma unroll
    for (int qb = 0; qb < kStreamQB; ++qb) {
      if (qb < nqb) {  // uniform
        floatx4 acc[kKB];
        bf16x8 qf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) qf[t] = kAhead ? qn[t] : q_frag(s_q, qb, t);
        stile<P == 2>(ks, qf, acc);
        if (kAhead && qb + 1 < kStreamQB) {
#pragma unroll
          for (int t = 0; t < 4; ++t) qn[t] = q_frag(s_q, qb + 1, t);
        }
        if (!fast) stream_mask(s_kp[wave], s_lim[qb * 16 + (lane & 15)], acc);
        if constexpr (P == 1) {
          float t[4 * kKB];  // s c - m c against the current reference
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) t[kb * 4 + v] = fmaf(acc[kb][v], c, st_nmc[qb]);
          const float tm = maxv(t);
          const bool first = st_l[qb] == 0.f;  // nothing visible yet: the reference is not set
          const bool mv = (tm > kLazy) | (first & (tm > -INFINITY));
          if (__builtin_amdgcn_ballot_w64(mv)) {
            if (mv) {  // the reference moves to the lane's largest logit of this block
              st_l[qb] = first ? 0.f : st_l[qb] * __builtin_amdgcn_exp2f(-tm);
              st_nmc[qb] -= tm;
#pragma unroll
              for (int i = 0; i < 4 * kKB; ++i) t[i] -= tm;
            }
          }
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < 4 * kKB; ++i) sum += __builtin_amdgcn_exp2f(t[i]);
          st_l[qb] += sum;
        } else if constexpr (P == 4) {  // pass 1, reference-free: masked logits are -inf and add 0
          float sum = 0.f;
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) sum += __builtin_amdgcn_exp2f(acc[kb][v] * c);
          st_l[qb] += sum;
        } else {
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) col[kb * 4 + v] += __builtin_amdgcn_exp2f(fmaf(acc[kb][v], c, -ml[qb]));
        }
      }
    }
    if constexpr (P == 2) {
      // lane j of a row ends with the total of value j % (4 kKB): key tile m / 4, output m % 4 of its lane group
      const float tot = row16_reduce_scatter(col);
      const int j = lane & 15, m = j & (4 * kKB - 1);
      const int key = sidx * kSub + (m >> 2) * 16 + (lane >> 4) * 4 + (m & 3);
      if (j < 4 * kKB && c0 + key < c1) {
        const int idx = c0 + key - k0;
        if (a.nrg == 1) put_score(a, (int64_t)unit * a.score_stride + idx, tot);
        else a.colpart[((int64_t)unit * a.nrg + rg) * a.key_span + idx] = tot;
      }
    }
  };

  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  if constexpr (PASS == 3) {
    // both passes over the wave's (at most two) steps, which stay in registers
    if (s < nsub) step(ks[0], s, P1{});
    if (s + NW < nsub) step(ks[1], s + NW, P1{});
#pragma unroll
    for (int qb = 0; qb < kStreamQB; ++qb) {
      const float mc = st_l[qb] > 0.f ? -st_nmc[qb] : -1e30f;  // this lane's m c (none: no visible key)
      const float mr = cross_row_max(mc);
      const float lr = cross_row_sum(st_l[qb] * __builtin_amdgcn_exp2f(mc - mr));
      if (lane < 16) s_st3[wave * kStreamRows + qb * 16 + lane] = make_float2(mr, lr);
    }
    __syncthreads();
    for (int r = threadIdx.x; r < kStreamRows; r += NT) {
      float mm = -1e30f;
#pragma unroll
      for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_st3[w * kStreamRows + r].x);
      float ll = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) ll += s_st3[w * kStreamRows + r].y * __builtin_amdgcn_exp2f(s_st3[w * kStreamRows + r].x - mm);
      // the row's normaliser max + log2(sum); +inf for rows that do not exist or see no key (they score nothing)
      s_ml3[r] = (r < rows && ll > 0.f) ? mm + __log2f(ll) : INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < kStreamQB; ++qb) ml[qb] = s_ml3[qb * 16 + (lane & 15)];
    if (s < nsub) step(ks[0], s, P2{});
    if (s + NW < nsub) step(ks[1], s + NW, P2{});
    return;
  }
  const int last = nsub - 1;
  // Step j of the wave: first the addresses of step j + kNSet, then the keys of step j + kNSet - 1 (whose addresses
  // came an iteration earlier, ahead of that iteration's keys, so waiting for them leaves the newer keys in flight),
  // then step j itself. The loads are unconditional: past the wave's last step they fetch that step again, unused,
  // so that no path through the loop skips a wait.
  auto stream = [&](auto pass_tag) __attribute__((always_inline)) {
    while (s < nsub) {
#pragma unroll
      for (int p = 0; p < kNSet; ++p) {
        kaddr_load<POW2>(a, b, g, c0, c1, ph(min(s + kNSet * NW, last)), ad[p]);
        kstep_fetch<POW2>(a, g, c0, c1, ph(min(s + (kNSet - 1) * NW, last)), ad[(p + kNSet - 1) % kNSet],
                          ks[(p + kNSet - 1) % kNSet]);
        step(ks[p], ph(s), pass_tag);
        s += NW;
        if (s >= nsub) break;
      }
    }
  };

  if constexpr (PASS == 1) {
    // combine the four lanes of each row, then the waves, and write the chunk's (max, sum) per row (log2 domain)
    float2 *s_st = reinterpret_cast<float2 *>(s_q);  // [NW][kStreamRows], once every wave is done with s_q
    __shared__ int s_redo;
    auto merge_out = [&](bool plain) __attribute__((always_inline)) {
      __syncthreads();  // every wave is done with s_q (and has read s_redo)
      if (threadIdx.x == 0) s_redo = 0;
#pragma unroll
      for (int qb = 0; qb < kStreamQB; ++qb) {
        float mr, lr;
        if (plain) {
          mr = 0.f;
          lr = cross_row_sum(st_l[qb]);
        } else {
          const float mc = st_l[qb] > 0.f ? -st_nmc[qb] : -1e30f;  // this lane's m c (none: no visible key)
          mr = cross_row_max(mc);
          lr = cross_row_sum(st_l[qb] * __builtin_amdgcn_exp2f(mc - mr));
        }
        if (lane < 16) s_st[wave * kStreamRows + qb * 16 + lane] = make_float2(mr, lr);
      }
      __syncthreads();
      float *out = a.stats + ((((int64_t)unit * a.nrg + rg) * a.nkc + chunk) * a.rpg) * 2;
      bool bad = false;
      for (int r = threadIdx.x; r < kStreamRows; r += NT) {
        float mm = -1e30f;
#pragma unroll
        for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_st[w * kStreamRows + r].x);
        float ll = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) ll += s_st[w * kStreamRows + r].y * __builtin_amdgcn_exp2f(s_st[w * kStreamRows + r].x - mm);
        out[r * 2] = mm;
        out[r * 2 + 1] = ll;
        bad |= plain && r < rows && !(ll >= kPlainLo && ll <= kPlainHi);
      }
      if (bad) s_redo = 1;
      __syncthreads();
      return s_redo != 0;
    };
    stream(std::integral_constant<int, 4>{});
    if (merge_out(true)) {  // uniform, rare: a row sum outside the band; the chunk again, exactly
#pragma unroll
      for (int qb = 0; qb < kStreamQB; ++qb) st_l[qb] = 0.f, st_nmc[qb] = 0.f;
      // the queries again (s_q held the statistics), and the wave's first step and the addresses of its second
      __syncthreads();
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));  // the addresses are computed again, not kept alive through the first stream
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        const int i = tid + j * NT, r = i >> 4, p = i & 15;
        const bool in = r < rows;
        const u32x4 v0 = ld16(qbase + (int64_t)(in ? i : (i & 15)) * 16);
        const u32x4 v = {in ? v0.x : 0u, in ? v0.y : 0u, in ? v0.z : 0u, in ? v0.w : 0u};
        *reinterpret_cast<u32x4 *>(s_q + r * 256 + ((p ^ (r & 15)) << 4)) = v;
      }
      s = __builtin_amdgcn_readfirstlane(wave);
      prime();
      __syncthreads();
      stream(std::integral_constant<int, 1>{});
      merge_out(false);
    }
  } else {
    stream(std::integral_constant<int, PASS>{});
  }
}

// ---- bidirectional windows: region keys resident in registers, queries streamed -------------------------------
// A BIDIR unit has at most a few hundred region keys and r * window query rows (C2: 448 keys, 2048 rows), every row
// a softmax over all the keys. The keys are loaded once per workgroup and split over its four waves: wave w holds
// the A fragments of key tiles [w KT, (w + 1) KT) in registers (KT x 4 x 16 B per lane). The query rows stream
// through in 16-row blocks. Per block a wave computes its logits S^T = K Q^T (lane l: query row l % 16, keys
// 4 (l / 16) + i of each tile), the rows' sums of exp2 over its own keys against a reference maximum, and publishes
// (reference, sum) per row in LDS; after one barrier every wave knows each row's overall max M and sum L, and adds
// exp2(s c - m_w c) exp2(m_w c - M) / L of its keys into per-lane column sums. A row's weights are computed once and
// never leave the registers. At the end the 16 lanes of a key (one per query row of the block layout) are summed.
//
// Up to seven key tiles per wave, blocks go in pairs with one barrier per pair: both blocks' MFMAs are issued back
// to back, so the matrix unit works on the second while the vector unit does the first block's softmax. With eight
// tiles the registers hold one pair only at one workgroup per CU; there a software pipeline issues the MFMAs of
// block qb + 1 before the softmax work of block qb instead. The query blocks reach LDS by DMA
// (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at M0 + 16 i, no registers involved) into a ring of
// kQRing slots, several blocks ahead of their use; each wave fetches a quarter of every block and waits for its own
// DMAs before the barrier. The loop is unrolled over the ring, so every LDS address is an immediate offset.
constexpr int kBidirNW = 4;
constexpr int kBidirMaxKT = 8;  // key tiles per wave: regions of up to 4 x 8 x 16 = 512 keys
#ifndef SE_BIDIR_QRING
#define SE_BIDIR_QRING 8
#endif
constexpr int kQRing = SE_BIDIR_QRING;  // LDS slots of 16 query rows (4 KiB each)
// pairs of blocks alternate between two halves of the published statistics, and a pass over the ring must end on
// the second half; the waits keep four blocks (pairs) or five (pipeline) in flight
static_assert(kQRing % 4 == 0 && kQRing >= 8, "ring of a multiple of four slots, at least eight");

// The DMA is inline assembly so that the compiler's wait-count bookkeeping does not track it (it would otherwise
// wait for every DMA in flight before any LDS read); the kernel waits for its DMAs itself in bidir_publish(). It
// has no output register. One wait state separates the M0 write from the DMA that reads it.
SE_DEV void lds_dma16(const char *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// the same from a wave-uniform base address (scalar registers) plus a 32-bit per-lane byte offset
SE_DEV void lds_dma16_s(const char *base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

// Wait until at most N of this wave's DMAs are in flight and its LDS accesses are done, then meet the other waves:
// afterwards every wave's older DMAs have landed. The memory clobber keeps the compiler from moving LDS accesses
// across.
template <int N>
SE_DEV void bidir_publish() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Workgroups per CU the register budget allows: two (256 registers per wave: at seven tiles 112 hold the keys, 124
// the two logit sets, the column sums and the rest) up to seven key tiles per wave; one (512) at eight.
#ifndef SE_BIDIR_PIPE_KT
#define SE_BIDIR_PIPE_KT 8  // key tiles per wave from which the software pipeline is used
#endif
template <int KT>
constexpr bool bidir_pipe() { return KT >= SE_BIDIR_PIPE_KT; }
template <int KT>
constexpr int bidir_wgs_per_cu() { return bidir_pipe<KT>() ? 1 : 2; }

template <int KT, bool POW2>
__global__ __launch_bounds__(kBidirNW * 64, bidir_wgs_per_cu<KT>()) void window_bidir(ScoreArgs a) {
  int chunk, rg, unit;
  xcd_item(chunk, rg, unit);
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ __attribute__((aligned(16))) char s_q[kQRing * 4096];  // query blocks, rows swizzled
  // per parity of the barrier, block of the pair, wave and row: (m c, sum) of the wave's keys
  __shared__ float2 s_ml[2][2][kBidirNW][16];
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int nkeys = k1 - k0;
  if (nkeys <= 0) return;  // uniform: the window is longer than the cache (nothing to score)
  const int total = a.R * a.wq;
  const int row0 = rg * a.rpg;
  const int rows = min(a.rpg, total - row0);
  const int nqb = (rows + 15) / 16;
  const int32_t *bt = a.bt + (int64_t)b * a.max_blocks;
  const int32_t *pos = a.pos + (int64_t)unit * a.max_blocks * a.page;

  // DMA of query block qb (any qb: rows past the unit's last are read from its last row and never scored) into its
  // ring slot. Wave w writes rows 4w..4w+3 of the slot; lane i the 16 bytes at position i % 16 of row 4w + i / 16,
  // which hold piece (i % 16) ^ row of that row (row r's piece p sits at r * 256 + ((p ^ r) * 16), so the 16 rows a
  // fragment read touches fall in distinct banks).
  const char *qunit = a.q + ((int64_t)b * a.n_kv + g) * total * 256;
  const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)s_q + wave * 1024);
  const int dma_r = wave * 4 + (lane >> 4);               // row of the block this lane fetches
  const uint32_t dma_piece = ((lane & 15) ^ dma_r) << 4;  // byte offset of its 16 bytes within the row
  // `slot` is qb % kQRing; callers pass it as a constant so that the LDS address folds into an immediate. The
  // block's first row (clamped to the unit's last) is a scalar base; rows past the unit's last read that row.
  auto dma_block = [&](int qb, int slot) __attribute__((always_inline)) {
    const int first = min(row0 + qb * 16, total - 1);  // wave-uniform
    const uint32_t off = (uint32_t)min(dma_r, total - 1 - first) * 256 + dma_piece;
    lds_dma16_s(qunit + (int64_t)first * 256, off, ring + (uint32_t)slot * 4096);
  };
  // B fragments of a block (k-steps 0..3) from ring slot `slot`: lane l reads row l % 16, piece 4 t + l / 16
  uint32_t frag_off[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = lane & 15;
    frag_off[t] = r * 256 + (((t * 4 + (lane >> 4)) ^ r) << 4);
  }
  auto read_frags = [&](int slot, bf16x8 (&qf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qf[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(s_q + frag_off[t] + slot * 4096));
      // software-pipelined: only the MFMAs read the fragments, so they too live in the accumulation registers
      if constexpr (bidir_pipe<KT>()) asm volatile("" : "+a"(qf[t]));
    }
  };
#pragma unroll
  for (int i = 0; i < kQRing; ++i) dma_block(i, i);  // the first kQRing blocks are in flight during the key loads

  // resident row of region key j (region-relative), or -1
  auto key_row_of = [&](int j) __attribute__((always_inline)) {
    const int key = k0 + min(j, nkeys - 1);
    const int pg = page_of<POW2>(a, key);
    const int blk = bt[pg], p = pos[key];
    const int off = POW2 ? (key & (a.page - 1)) : key - pg * a.page;
    return (j < nkeys && p >= 0 && (unsigned)blk < (unsigned)a.num_blocks) ? (blk * a.n_kv + g) * a.page + off : -1;
  };
  bf16x8 kf[KT][4];
  uint32_t vmask = 0;  // bit 4 kt + i: the key of this lane's output i of tile kt is scored
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int tile = wave * KT + kt;
    const int row = key_row_of(tile * 16 + (lane & 15));
    const char *src = a.k + (int64_t)(row >= 0 ? row : 0) * 256 + (lane >> 4) * 16;
#pragma unroll
    for (int t = 0; t < 4; ++t) kf[kt][t] = __builtin_bit_cast(bf16x8, ld16(src + t * 64));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key_row_of(tile * 16 + 4 * (lane >> 4) + i) >= 0) vmask |= 1u << (kt * 4 + i);
  }
  const bool all_valid = __builtin_amdgcn_ballot_w64(vmask != (KT == 8 ? 0xffffffffu : (1u << (KT * 4)) - 1)) == 0;
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): the keys, their maps and the first blocks have landed
  if constexpr (KT >= 6) {
    // the key fragments, which only the MFMAs read, live in the accumulation registers, so the logits and the
    // vector work keep the ordinary ones
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int t = 0; t < 4; ++t) asm volatile("" : "+a"(kf[kt][t]));
  }
  __syncthreads();

  const float c = a.scale_log2;
  float col[KT * 4];
#pragma unroll
  for (int i = 0; i < KT * 4; ++i) col[i] = 0.f;
  auto mfmas = [&](const bf16x8 (&qf)[4], floatx4 (&acc)[KT]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][t], qf[t], acc[kt], 0, 0, 0);
    if constexpr (KT >= 6) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) asm volatile("" : "+v"(acc[kt]));  // logits in the ordinary registers
    }
  };

  // Softmax work of one block whose logits are in `cur`; returns the lane's row sum l over the wave's keys and sets
  // mc, the reference m c it is taken against. ALLV: every key of the wave is scored (no masking). With ALLV the
  // weights are exp2(s c) with no reference subtracted: a row whose sum of weights over the wave's keys lies in
  // [2^-80, 2^80] has every weight finite and flushes only terms below 2^-126, under 2^-40 of the sum, so its
  // normalised weights are as exact as against its maximum. A block with a row outside that band has its logits
  // computed again from its ring slot (into `qf`, which the MFMAs have consumed) and weighted against each row's
  // exact maximum. Without ALLV the keys that are not scored are masked and the exact maximum is the reference. The
  // weights overwrite the logits.
  auto weights = [&](floatx4 (&cur)[KT], float mc) __attribute__((always_inline)) {
    float l;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cur[kt][i] = __builtin_amdgcn_exp2f(fmaf(cur[kt][i], c, -mc));
        l = kt == 0 && i == 0 ? cur[0][0] : l + cur[kt][i];
      }
    return cross_row_sum(l);
  };
  auto weights_exact = [&](floatx4 (&cur)[KT], float &mc) __attribute__((always_inline)) {
    float x = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) x = fmaxf(x, fmaxf(fmaxf(cur[kt][0], cur[kt][1]), fmaxf(cur[kt][2], cur[kt][3])));
    const float mx = cross_row_max(x);
    mc = mx == -INFINITY ? 0.f : mx * c;  // no scored key: every weight is 0
    return weights(cur, mc);
  };
  auto softmax = [&](floatx4 (&cur)[KT], bf16x8 (&qf)[4], int slot, float &mc, auto allv_tag)
      __attribute__((always_inline)) {
    constexpr bool ALLV = decltype(allv_tag)::value;
    mc = 0.f;
    float l;
    if constexpr (ALLV) {
      l = weights(cur, 0.f);
      if constexpr (bidir_pipe<KT>()) {
        // one MFMA (of the next block), then three vector instructions, 4 KT times: the matrix unit runs under the
        // softmax work
#pragma unroll
        for (int i = 0; i < 4 * KT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      }
      if (__builtin_amdgcn_ballot_w64(!(l >= 0x1p-80f && l <= 0x1p80f))) {  // uniform, rare
        read_frags(slot, qf);
        mfmas(qf, cur);
        l = weights_exact(cur, mc);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[kt][i] = (vmask >> (kt * 4 + i)) & 1u ? cur[kt][i] : -INFINITY;
      l = weights_exact(cur, mc);
    }
    return l;
  };
  // The normalising factor of the lane's row in block qb, from every wave's published (m c, l) in `pub`: the row's
  // total L against the common reference M = max of the waves' references (all 0 in the usual case).
  auto norm = [&](const float2 (&pub)[kBidirNW][16], int qb, float mc, float l, auto allv_tag)
      __attribute__((always_inline)) {
    constexpr bool ALLV = decltype(allv_tag)::value;
    float2 w[kBidirNW];
#pragma unroll
    for (int v = 0; v < kBidirNW; ++v) w[v] = pub[v][lane & 15];
    float f;
    if (__builtin_amdgcn_ballot_w64((__float_as_uint(w[0].x) | __float_as_uint(w[1].x) | __float_as_uint(w[2].x) |
                                     __float_as_uint(w[3].x)) != 0u) == 0 &&
        ALLV && qb * 16 + 16 <= rows) {
      // every reference is 0, so mc = M = 0; with every key scored, l and L are positive (a sum outside
      // [2^-80, 2^80] took the exact path, after which l >= 1); and the whole block holds rows
      f = __builtin_amdgcn_rcpf((w[0].y + w[1].y) + (w[2].y + w[3].y));
    } else {
      float M = -1e30f;
#pragma unroll
      for (int v = 0; v < kBidirNW; ++v) M = w[v].y > 0.f ? fmaxf(M, w[v].x) : M;
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < kBidirNW; ++v) L += w[v].y > 0.f ? w[v].y * __builtin_amdgcn_exp2f(w[v].x - M) : 0.f;
      const bool row_ok = qb * 16 + (lane & 15) < rows && L > 0.f && l > 0.f;
      f = row_ok ? __builtin_amdgcn_exp2f(mc - M) * __builtin_amdgcn_rcpf(L) : 0.f;
    }
    return f;
  };
  auto accumulate = [&](const floatx4 (&cur)[KT], float f) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) col[kt * 4 + i] = fmaf(cur[kt][i], f, col[kt * 4 + i]);
  };
  // the weights are added where they are made: left alone, the compiler sinks each block's additions into the next
  // block's and keeps the weights of every block of the unrolled loop alive at once
  auto pin_col = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KT * 4; ++i) asm volatile("" : "+v"(col[i]));
  };

  floatx4 accA[KT], accB[KT];
  bf16x8 qf[4];

  // Without the pipeline, blocks go in pairs, qb (ring slot `slot`, even) and qb + 1, with one barrier: both blocks'
  // MFMAs are issued back to back (the fragments read just before, visible since the previous barrier), so the
  // second block's run under the first block's softmax work, and the pair's (m c, l) are published together.
  // Afterwards blocks qb + 2 and qb + 3 have landed in LDS for every wave, and the pair's slots are refilled.
  auto pair = [&](int qb, int slot, auto allv_tag) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);  // no overlap of pairs: two logit sets
    read_frags(slot, qf);
    mfmas(qf, accA);
    read_frags(slot + 1, qf);
    mfmas(qf, accB);
    float mcA, mcB;
    const float lA = softmax(accA, qf, slot, mcA, allv_tag);
    const float lB = softmax(accB, qf, slot + 1, mcB, allv_tag);
    const int par = (slot >> 1) & 1;
    if (lane < 16) {
      s_ml[par][0][wave][lane] = make_float2(mcA, lA);
      s_ml[par][1][wave][lane] = make_float2(mcB, lB);
    }
    bidir_publish<kQRing - 4>();
    dma_block(qb + kQRing, slot);  // into the pair's slots, which every wave has read; past the last block: unused
    dma_block(qb + kQRing + 1, slot + 1);
    const float fA = norm(s_ml[par][0], qb, mcA, lA, allv_tag);
    const float fB = norm(s_ml[par][1], qb + 1, mcB, lB, allv_tag);
    accumulate(accA, fA);
    accumulate(accB, fB);
    pin_col();
  };
  // With the pipeline, block qb's logits are in `cur` (MFMAs issued one block earlier); `nxt` receives block
  // qb + 1's, from the fragments in `qf`, which then take block qb + 2's.
  auto single = [&](int qb, int slot, floatx4 (&cur)[KT], floatx4 (&nxt)[KT], auto allv_tag)
      __attribute__((always_inline)) {
    mfmas(qf, nxt);
    float mc;
    const float l = softmax(cur, qf, slot, mc, allv_tag);
    if (lane < 16) s_ml[slot & 1][0][wave][lane] = make_float2(mc, l);
    bidir_publish<kQRing - 3>();  // block qb + 2 complete in LDS for every wave, this block's (m c, l) published
    dma_block(qb + kQRing, slot);
    read_frags((slot + 2) % kQRing, qf);
    accumulate(cur, norm(s_ml[slot & 1][0], qb, mc, l, allv_tag));
    pin_col();
  };

  if constexpr (bidir_pipe<KT>()) {
    read_frags(0, qf);
    mfmas(qf, accA);
    read_frags(1, qf);
  }
  // A multiple of kQRing blocks (a padding block has no rows: its weights are never added), so the loop body holds
  // one iteration per ring slot, with the slot a constant in each, and no exit between them. Past the last block
  // the MFMAs and fragment reads still run (their slots hold finished DMAs of clamped rows) and their results are
  // never used, so the body has no branch between the MFMA issues and the weights.
  const int nqbr = (nqb + kQRing - 1) / kQRing * kQRing;
  auto run = [&](auto allv_tag) __attribute__((always_inline)) {
    for (int qb = 0; qb < nqbr; qb += kQRing) {
#pragma unroll
      for (int j = 0; j < kQRing; j += 2) {
        if constexpr (bidir_pipe<KT>()) {
          single(qb + j, j, accA, accB, allv_tag);
          single(qb + j + 1, j + 1, accB, accA, allv_tag);
        } else {
          pair(qb + j, j, allv_tag);
        }
      }
    }
  };
  if (all_valid) run(std::true_type{});
  else run(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): no DMA outlives the loop

  // sum over the 16 query-row lanes of each key; lane j of a row ends with the total of value j of each group of 16
#pragma unroll
  for (int g0 = 0; g0 < KT * 4; g0 += 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = g0 + i < KT * 4 ? col[g0 + i] : 0.f;
    const float tot = row16_reduce_scatter(v);
    const int j = lane & 15, m = g0 + j;
    if (m < KT * 4) {
      const int key = (wave * KT + m / 4) * 16 + 4 * (lane >> 4) + (m & 3);
      if (key < nkeys) {
        if (a.nrg == 1) put_score(a, (int64_t)unit * a.score_stride + key, tot);
        else a.colpart[((int64_t)unit * a.nrg + rg) * a.key_span + key] = tot;
      }
    }
  }
}

#ifndef SE_STREAM_NW
#define SE_STREAM_NW 4
#endif
#ifndef SE_STREAM_WGS
#define SE_STREAM_WGS 512
#endif
constexpr int kStreamNW = SE_STREAM_NW;
constexpr int kStreamWGs = SE_STREAM_WGS;  // workgroups a launch aims for (two per CU at NW = 4)
constexpr int kFusedKeys = 2 * 64 * kStreamNW;  // key ranges the single-kernel path takes (two 64-key steps per wave)

// ---- VALU path (fp32 inputs, or any d that fits) ---------------------------------------------------------------
template <int DTYPE, int D>
SE_DEV float row_dot(const char *qr, const char *kr) {
  float acc = 0.f;
  if (DTYPE == SE_DTYPE_F32) {
    const float *x = (const float *)qr, *y = (const float *)kr;
#pragma unroll 16
    for (int e = 0; e < D; ++e) acc = fmaf(x[e], y[e], acc);
  } else {
    const uint16_t *x = (const uint16_t *)qr, *y = (const uint16_t *)kr;
#pragma unroll 16
    for (int e = 0; e < D; ++e) acc = fmaf(__uint_as_float((uint32_t)x[e] << 16), __uint_as_float((uint32_t)y[e] << 16), acc);
  }
  return acc;
}

SE_DEV const char *key_row(const ScoreArgs &a, int b, int g, int key, int row_bytes, int &p) {
  const int32_t *pos = a.pos + ((int64_t)b * a.n_kv + g) * a.max_blocks * a.page;
  p = pos[key];
  int blk = a.bt[(int64_t)b * a.max_blocks + key / a.page];
  if (p < 0 || !blk_ok(blk, a.num_blocks)) {
    p = -1;
    return nullptr;
  }
  return a.k + (((int64_t)blk * a.n_kv + g) * a.page + key % a.page) * row_bytes;
}

template <int DTYPE, int D>
__global__ __launch_bounds__(kValuRows) void stats_valu(ScoreArgs a) {
  constexpr int RBY = D * (DTYPE == SE_DTYPE_F32 ? 4 : 2);
  const int unit = blockIdx.z, rg = blockIdx.y, kc = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int rho = rg * kValuRows + threadIdx.x;
  const int lim = row_limit(a, b, rho);
  const char *qr = lim >= 0 ? q_row(a, b, g, rho, RBY) : nullptr;
  float m = -1e30f, l = 0.f;
  const int c0 = k0 + kc * a.kc, c1 = min(c0 + a.kc, k1);
  for (int key = c0; key < c1 && qr; ++key) {
    int p;
    const char *kr = key_row(a, b, g, key, RBY, p);
    if (!kr || p > lim) continue;
    float x = row_dot<DTYPE, D>(qr, kr) * a.scale_log2;
    float mn = fmaxf(m, x);
    l = l * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(x - mn);
    m = mn;
  }
  float *out = a.stats + ((((int64_t)unit * a.nrg + rg) * a.nkc + kc) * kValuRows + threadIdx.x) * 2;
  out[0] = m;
  out[1] = l;
}

template <int DTYPE, int D>
__global__ __launch_bounds__(kValuRows) void colsum_valu(ScoreArgs a) {
  constexpr int RBY = D * (DTYPE == SE_DTYPE_F32 ? 4 : 2);
  const int unit = blockIdx.z, rg = blockIdx.y, kc = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  __shared__ float s_mlog[kValuRows];
  __shared__ int s_lim[kValuRows];
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int c0 = k0 + kc * a.kc, c1 = min(c0 + a.kc, k1);
  if (c0 >= c1) return;
  merge_stats(a, unit, rg, s_mlog);
  s_lim[threadIdx.x] = row_limit(a, b, rg * kValuRows + threadIdx.x);
  __syncthreads();
  const int rows = min(kValuRows, a.R * a.wq - rg * kValuRows);
  for (int key = c0 + threadIdx.x; key < c1; key += kValuRows) {
    int p;
    const char *kr = key_row(a, b, g, key, RBY, p);
    float sum = 0.f;
    for (int r = 0; r < rows && kr; ++r) {
      if (p > s_lim[r]) continue;
      const char *qr = q_row(a, b, g, rg * kValuRows + r, RBY);
      sum += __builtin_amdgcn_exp2f(row_dot<DTYPE, D>(qr, kr) * a.scale_log2 - s_mlog[r]);
    }
    int idx = key - k0;
    if (a.nrg == 1) put_score(a, (int64_t)unit * a.score_stride + idx, sum);
    else a.colpart[((int64_t)unit * a.nrg + rg) * a.key_span + idx] = sum;
  }
}

// sum the row groups' column sums
__global__ void colsum_reduce(ScoreArgs a) {
  const int unit = blockIdx.y;
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < k1 - k0; j += gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int r = 0; r < a.nrg; ++r) s += a.colpart[((int64_t)unit * a.nrg + r) * a.key_span + j];
    put_score(a, (int64_t)unit * a.score_stride + j, s);
  }
}

template <int PASS, int KB>
void launch_stream_kb(const ScoreArgs &a, dim3 grid, hipStream_t st) {
  if (a.page_shift >= 0) hipLaunchKernelGGL((window_stream<PASS, kStreamNW, true, KB>), grid, dim3(kStreamNW * 64), 0, st, a);
  else hipLaunchKernelGGL((window_stream<PASS, kStreamNW, false, KB>), grid, dim3(kStreamNW * 64), 0, st, a);
}
template <int PASS>
void launch_stream(const ScoreArgs &a, dim3 grid, int kb, hipStream_t st) {
  if (kb == 2) launch_stream_kb<PASS, 2>(a, grid, st);
  else launch_stream_kb<PASS, 4>(a, grid, st);
}

template <int KT>
void launch_bidir_kt(const ScoreArgs &a, dim3 grid, hipStream_t st) {
  if (a.page_shift >= 0) hipLaunchKernelGGL((window_bidir<KT, true>), grid, dim3(kBidirNW * 64), 0, st, a);
  else hipLaunchKernelGGL((window_bidir<KT, false>), grid, dim3(kBidirNW * 64), 0, st, a);
}

void launch_bidir(int kt, const ScoreArgs &a, dim3 grid, hipStream_t st) {
  switch (kt) {
    case 1: launch_bidir_kt<1>(a, grid, st); break;
    case 2: launch_bidir_kt<2>(a, grid, st); break;
    case 3: launch_bidir_kt<3>(a, grid, st); break;
    case 4: launch_bidir_kt<4>(a, grid, st); break;
    case 5: launch_bidir_kt<5>(a, grid, st); break;
    case 6: launch_bidir_kt<6>(a, grid, st); break;
    case 7: launch_bidir_kt<7>(a, grid, st); break;
    default: launch_bidir_kt<8>(a, grid, st); break;
  }
}

#ifndef SE_BIDIR_WGS
#define SE_BIDIR_WGS 512
#endif
constexpr int kBidirWGs = SE_BIDIR_WGS;  // workgroups a launch aims for (two per CU)

struct Plan {
  int nrg, nkc, kc, key_span, rpg, nw;  // nw: waves per MFMA workgroup (0: fp32 VALU path, -1: streaming)
  int kb;                               // streaming: 16-key tiles per step of a wave (2 or 4)
  int bidir_kt;                         // > 0: the register-resident bidirectional kernel, key tiles per wave
  size_t stats_bytes, col_bytes;
};

Plan make_plan(const se_cache_t *c, const se_window_params_t *p) {
  Plan pl;
  pl.bidir_kt = 0;
  const int R = c->n_q / c->n_kv;
  const int rows = R * p->n_query;
  const bool mfma = c->dtype == SE_DTYPE_BF16 && c->d == 128;
  const size_t units = (size_t)c->B * c->n_kv;
  if (mfma && p->mode == SE_SCORE_BIDIR && p->window - p->protect <= kBidirNW * kBidirMaxKT * 16) {
    // one workgroup per unit, or row groups of whole 16-row blocks when there are too few units to fill the chip
    pl.key_span = p->window - p->protect;
    const int tiles = (pl.key_span + 15) / 16;
    pl.bidir_kt = (tiles + kBidirNW - 1) / kBidirNW;
    const int blocks = (rows + 15) / 16;
    long long want = (kBidirWGs + (long long)units - 1) / (long long)units;
    if (want > blocks) want = blocks;
    if (want < 1) want = 1;
    const int per = (int)((blocks + want - 1) / want);
    pl.rpg = per * 16;
    pl.nrg = (rows + pl.rpg - 1) / pl.rpg;
    pl.nw = -2;
    pl.nkc = 1;
    pl.kc = pl.key_span;
    pl.stats_bytes = 0;
    pl.col_bytes = pl.nrg > 1 ? se_host::align_up(units * pl.nrg * pl.key_span * sizeof(float)) : 0;
    return pl;
  }
  int maxc;
  if (!mfma) {
    pl.nw = 0, pl.rpg = kValuRows, maxc = 1024;
  } else {
    pl.nw = -1, pl.rpg = kStreamRows, maxc = 0;
  }
  pl.nrg = (rows + pl.rpg - 1) / pl.rpg;
  const int max_slots = c->max_blocks * c->page;
  pl.key_span = p->mode == SE_SCORE_CAUSAL ? max_slots : p->window - p->protect;
  const int span64 = (pl.key_span + 63) / 64 * 64;
  pl.kb = 4;
  if (pl.nw < 0 && pl.key_span <= kFusedKeys) {
    // at most two 64-key steps per wave: one chunk, both passes in one kernel
    pl.kc = (pl.key_span + 64 * kStreamNW - 1) / (64 * kStreamNW) * (64 * kStreamNW);
  } else if (pl.nw < 0) {
    // chunks of whole rounds of steps (one per wave) that give about kStreamWGs workgroups
    pl.kb = pl.nrg == 1 ? 2 : 4;
    const long long groups = (long long)c->B * c->n_kv * pl.nrg;
    const long long per = (kStreamWGs + groups - 1) / groups;
    const int round = 16 * pl.kb * kStreamNW;
    long long kc = (pl.key_span + per - 1) / per;
    kc = (kc + round - 1) / round * round;
    pl.kc = (int)(kc < round ? round : (kc > 16384 ? 16384 : kc));
  } else {
    pl.kc = span64 < maxc ? span64 : maxc;
    if (pl.kc < 64) pl.kc = 64;
  }
  pl.nkc = (pl.key_span + pl.kc - 1) / pl.kc;
  pl.stats_bytes = se_host::align_up(units * pl.nrg * pl.nkc * pl.rpg * 2 * sizeof(float));
  pl.col_bytes = pl.nrg > 1 ? se_host::align_up(units * pl.nrg * pl.key_span * sizeof(float)) : 0;
  return pl;
}


}  // namespace
}  // namespace se

extern "C" size_t se_window_score_workspace_size(const se_cache_t *c, const se_window_params_t *p) {
  if (se_host::check_cache(c) != SE_OK || !p) return 0;
  se::Plan pl = se::make_plan(c, p);
  return pl.stats_bytes + pl.col_bytes;
}

extern "C" int32_t se_window_score(const se_cache_t *c, const void *q_win, const int32_t *q_pos,
                                   const se_window_params_t *p, float *scores, int32_t *status, void *ws,
                                   size_t ws_bytes, se_stream_t stream) {
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!q_win || !p || !scores) return SE_ERR_NULL;
  if (p->n_query <= 0) return SE_ERR_PARAM;
  if (p->mode == SE_SCORE_CAUSAL) {
    if (!q_pos) return SE_ERR_NULL;
    if (p->score_stride < c->max_blocks * c->page) return SE_ERR_SHAPE;
  } else if (p->mode == SE_SCORE_BIDIR) {
    if (p->window <= 0 || p->protect < 0 || p->protect >= p->window) return SE_ERR_PARAM;
    if (p->n_query != p->window) return SE_ERR_PARAM;
    if (p->score_stride < p->window - p->protect) return SE_ERR_SHAPE;
  } else {
    return SE_ERR_PARAM;
  }
  const bool mfma = c->dtype == SE_DTYPE_BF16 && c->d == 128;
  const bool valu = c->dtype == SE_DTYPE_F32 && c->d == 64;
  if (!mfma && !valu) return SE_ERR_DTYPE;
  if ((long long)c->num_blocks * c->n_kv * c->page >= (1ll << 31)) return SE_ERR_UNSUPPORTED;  // 32-bit row ids
  se::Plan pl = se::make_plan(c, p);
  if (pl.stats_bytes + pl.col_bytes > 0 && (!ws || ws_bytes < pl.stats_bytes + pl.col_bytes)) return SE_ERR_WORKSPACE;
  se::ScoreArgs a;
  a.k = (const char *)c->k_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.q = (const char *)q_win;
  a.q_pos = q_pos;
  a.scores = scores;
  a.stats = pl.stats_bytes ? (float *)ws : nullptr;
  a.colpart = pl.col_bytes ? (float *)((char *)ws + pl.stats_bytes) : nullptr;
  a.status = status;
  a.mode = p->mode;
  a.n_kv = c->n_kv;
  a.R = c->n_q / c->n_kv;
  a.wq = p->n_query;
  a.page = c->page;
  a.page_shift = (c->page & (c->page - 1)) == 0 ? __builtin_ctz((unsigned)c->page) : -1;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.window = p->window;
  a.protect = p->protect;
  a.score_stride = p->score_stride;
  a.nrg = pl.nrg;
  a.nkc = pl.nkc;
  a.kc = pl.kc;
  a.key_span = pl.key_span;
  a.rpg = pl.rpg;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  a.accumulate = p->accumulate != 0;
  const int units = c->B * c->n_kv;
  const dim3 grid(pl.nkc, pl.nrg, units);
  hipStream_t st = (hipStream_t)stream;
  if (pl.bidir_kt > 0) {
    se::launch_bidir(pl.bidir_kt, a, grid, st);
  } else if (pl.nw < 0 && pl.key_span <= se::kFusedKeys) {
    se::launch_stream_kb<3, 4>(a, grid, st);
  } else if (pl.nw < 0) {
    se::launch_stream<1>(a, grid, pl.kb, st);
    se::launch_stream<2>(a, grid, pl.kb, st);
  } else {
    hipLaunchKernelGGL((se::stats_valu<SE_DTYPE_F32, 64>), grid, dim3(se::kValuRows), 0, st, a);
    hipLaunchKernelGGL((se::colsum_valu<SE_DTYPE_F32, 64>), grid, dim3(se::kValuRows), 0, st, a);
  }
  if (pl.nrg > 1) {
    const int bx = (pl.key_span + 255) / 256;
    hipLaunchKernelGGL(se::colsum_reduce, dim3(bx, units), dim3(256), 0, st, a);
  }
  return se_host::launch_status();
}
