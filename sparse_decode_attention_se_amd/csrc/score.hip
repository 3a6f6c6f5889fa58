// Observation-window attention scores.
//   CAUSAL (SnapKV at the prefill finish_step hook, SparseEngine page "How it works"): the window queries attend
//     causally over all resident keys; softmax weights are summed per key over queries and the GQA group.
//   BIDIR (KARA page, "Method" part 1): every window query scores the compressible region (window minus its
//     protected tail) with no mask; weights are summed the same way.
//
// Per (sequence, KV head) unit the R*Wq query rows of the group form a matrix Q and the keys a matrix K. The row
// softmax needs each row's global max and sum before any weight can be added to a key, so the work is two passes
// over QK^T: pass 1 streams K in chunks and keeps an online (max, sum) per row; pass 2 merges those, recomputes
// QK^T and adds exp2(s - max - log2 sum) into per-key column sums. For bf16 (d = 128) QK^T runs on MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate); fp32 inputs use a plain VALU path. A workgroup covers 256 query
// rows (4 waves x 64) and one key chunk; with more than 256 rows, a third kernel sums the row groups' column sums.
#include "common.hpp"

namespace se {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowsPerWG = 256;
constexpr int kRowsPerWave = 64;

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
  int32_t nrg, nkc, kc, key_span;
  float scale_log2;
};

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
    if (k0 < 0) k0 = k1 = 0;
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

// ---- MFMA path (bf16, d = 128) -------------------------------------------------------------------------------
// S = Q K^T per 16x16 tile: A = 16 query rows x 32 dims, B = 32 dims x 16 keys; lane l holds A row l%16 and B
// column l%16 with dims 8*(l/16)..+8 of each 32-dim step, and receives S rows 4*(l/16)..+4 of column l%16.
struct KTile {
  bf16x8 f[4];  // 4 k-steps of 32 dims
  int pos;      // position of this lane's key, -1 if it is not a visible key
};

SE_DEV void load_ktile(const ScoreArgs &a, int b, int g, int key, int k1, KTile &kt) {
  const int lane = threadIdx.x & 63;
  const int32_t *pos = a.pos + ((int64_t)b * a.n_kv + g) * a.max_blocks * a.page;
  kt.pos = -1;
  if (key < k1) {
    int p = pos[key];
    int blk = a.bt[(int64_t)b * a.max_blocks + key / a.page];
    if (p >= 0 && blk_ok(blk, a.num_blocks)) {
      kt.pos = p;
      const char *row = a.k + (((int64_t)blk * a.n_kv + g) * a.page + key % a.page) * 256 + (lane >> 4) * 16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kt.f[ks] = __builtin_bit_cast(bf16x8, ld16(row + ks * 64));
      return;
    }
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kt.f[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
}

struct QFrags {
  bf16x8 f[4][4];  // [row block][k-step]
  int lim[4][4];   // [row block][v]: position limit of S row 4*(l/16)+v of the block
};

SE_DEV void load_q(const ScoreArgs &a, int b, int g, int rho_wave, QFrags &qf) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    int rho = rho_wave + rb * 16 + (lane & 15);
    bool ok = rho < a.R * a.wq;
    const char *row = ok ? q_row(a, b, g, rho, 256) + (lane >> 4) * 16 : nullptr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf.f[rb][ks] = __builtin_bit_cast(bf16x8, ok ? ld16(row + ks * 64) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int v = 0; v < 4; ++v) qf.lim[rb][v] = row_limit(a, b, rho_wave + rb * 16 + (lane >> 4) * 4 + v);
  }
}

SE_DEV floatx4 mfma_tile(const QFrags &qf, int rb, const KTile &kt) {
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf.f[rb][ks], kt.f[ks], acc, 0, 0, 0);
  return acc;
}

__global__ __launch_bounds__(kThreads) void stats_mfma(ScoreArgs a) {
  const int unit = blockIdx.z, rg = blockIdx.y, kc = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int rho_wave = rg * kRowsPerWG + wave * kRowsPerWave;
  QFrags qf;
  load_q(a, b, g, rho_wave, qf);
  float m[4][4], l[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      m[rb][v] = -1e30f;
      l[rb][v] = 0.f;
    }
  const int c0 = k0 + kc * a.kc, c1 = min(c0 + a.kc, k1);
  for (int t0 = c0; t0 < c1; t0 += 64) {
    KTile kt[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) load_ktile(a, b, g, t0 + tt * 16 + (lane & 15), c1, kt[tt]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      floatx4 s[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) s[tt] = mfma_tile(qf, rb, kt[tt]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x[4];
        float mn = m[rb][v];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          bool vis = kt[tt].pos >= 0 && kt[tt].pos <= qf.lim[rb][v];
          x[tt] = vis ? s[tt][v] * a.scale_log2 : -INFINITY;
          mn = fmaxf(mn, x[tt]);
        }
        float acc = l[rb][v] * __builtin_amdgcn_exp2f(m[rb][v] - mn);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc += __builtin_amdgcn_exp2f(x[tt] - mn);
        l[rb][v] = acc;
        m[rb][v] = mn;
      }
    }
  }
  // combine the 16 lanes (keys) that share each row, then write the chunk's (max, sum) per row
  float *out = a.stats + ((((int64_t)unit * a.nrg + rg) * a.nkc + kc) * kRowsPerWG) * 2;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mr = row16_max(m[rb][v]);
      float lr = row16_sum(l[rb][v] * __builtin_amdgcn_exp2f(m[rb][v] - mr));
      if ((lane & 15) == 0) {
        int r = wave * kRowsPerWave + rb * 16 + (lane >> 4) * 4 + v;
        out[r * 2] = mr;
        out[r * 2 + 1] = lr;
      }
    }
}

// merge the per-chunk statistics of this workgroup's 256 rows into log2(sum) + max (or +inf for empty rows)
SE_DEV void merge_stats(const ScoreArgs &a, int unit, int rg, float *s_mlog) {
  const int r = threadIdx.x;
  const float *st = a.stats + (((int64_t)unit * a.nrg + rg) * a.nkc * kRowsPerWG) * 2;
  float mm = -1e30f;
  for (int c = 0; c < a.nkc; ++c) mm = fmaxf(mm, st[(c * kRowsPerWG + r) * 2]);
  float ll = 0.f;
  for (int c = 0; c < a.nkc; ++c) {
    const float *p = st + (c * kRowsPerWG + r) * 2;
    ll += p[1] * __builtin_amdgcn_exp2f(p[0] - mm);
  }
  s_mlog[r] = ll > 0.f ? mm + __log2f(ll) : INFINITY;
}

SE_DEV void write_colsums(const ScoreArgs &a, int unit, int rg, int c0, int c1, int k0, const float (*s_col)[1024]) {
  for (int j = threadIdx.x; j < c1 - c0; j += kThreads) {
    float sum = s_col[0][j] + s_col[1][j] + s_col[2][j] + s_col[3][j];
    int idx = c0 + j - k0;
    if (a.nrg == 1) a.scores[(int64_t)unit * a.score_stride + idx] = sum;
    else a.colpart[((int64_t)unit * a.nrg + rg) * a.key_span + idx] = sum;
  }
}

__global__ __launch_bounds__(kThreads) void colsum_mfma(ScoreArgs a) {
  const int unit = blockIdx.z, rg = blockIdx.y, kc = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float s_mlog[kRowsPerWG];
  __shared__ float s_col[4][1024];
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int c0 = k0 + kc * a.kc, c1 = min(c0 + a.kc, k1);
  if (c0 >= c1) return;  // uniform: no keys in this chunk
  merge_stats(a, unit, rg, s_mlog);
  const int rho_wave = rg * kRowsPerWG + wave * kRowsPerWave;
  QFrags qf;
  load_q(a, b, g, rho_wave, qf);
  __syncthreads();
  float ml[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) ml[rb][v] = s_mlog[wave * kRowsPerWave + rb * 16 + (lane >> 4) * 4 + v];
  for (int t0 = c0; t0 < c1; t0 += 64) {
    KTile kt[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) load_ktile(a, b, g, t0 + tt * 16 + (lane & 15), c1, kt[tt]);
    float col[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        floatx4 s = mfma_tile(qf, rb, kt[tt]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          bool vis = kt[tt].pos >= 0 && kt[tt].pos <= qf.lim[rb][v];
          float p = __builtin_amdgcn_exp2f(s[v] * a.scale_log2 - ml[rb][v]);
          col[tt] += vis ? p : 0.f;
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float cs = cross_row_sum(col[tt]);
      int j = t0 + tt * 16 + lane - c0;
      if (lane < 16 && t0 + tt * 16 + lane < c1) s_col[wave][j] = cs;
    }
  }
  __syncthreads();
  write_colsums(a, unit, rg, c0, c1, k0, s_col);
}

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
__global__ __launch_bounds__(kThreads) void stats_valu(ScoreArgs a) {
  constexpr int RBY = D * (DTYPE == SE_DTYPE_F32 ? 4 : 2);
  const int unit = blockIdx.z, rg = blockIdx.y, kc = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int rho = rg * kRowsPerWG + threadIdx.x;
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
  float *out = a.stats + ((((int64_t)unit * a.nrg + rg) * a.nkc + kc) * kRowsPerWG + threadIdx.x) * 2;
  out[0] = m;
  out[1] = l;
}

template <int DTYPE, int D>
__global__ __launch_bounds__(kThreads) void colsum_valu(ScoreArgs a) {
  constexpr int RBY = D * (DTYPE == SE_DTYPE_F32 ? 4 : 2);
  const int unit = blockIdx.z, rg = blockIdx.y, kc = blockIdx.x;
  const int b = unit / a.n_kv, g = unit % a.n_kv;
  __shared__ float s_mlog[kRowsPerWG];
  __shared__ int s_lim[kRowsPerWG];
  int k0, k1, n;
  key_range(a, unit, k0, k1, n);
  const int c0 = k0 + kc * a.kc, c1 = min(c0 + a.kc, k1);
  if (c0 >= c1) return;
  merge_stats(a, unit, rg, s_mlog);
  s_lim[threadIdx.x] = row_limit(a, b, rg * kRowsPerWG + threadIdx.x);
  __syncthreads();
  const int rows = min(kRowsPerWG, a.R * a.wq - rg * kRowsPerWG);
  for (int key = c0 + threadIdx.x; key < c1; key += kThreads) {
    int p;
    const char *kr = key_row(a, b, g, key, RBY, p);
    float sum = 0.f;
    for (int r = 0; r < rows && kr; ++r) {
      if (p > s_lim[r]) continue;
      const char *qr = q_row(a, b, g, rg * kRowsPerWG + r, RBY);
      sum += __builtin_amdgcn_exp2f(row_dot<DTYPE, D>(qr, kr) * a.scale_log2 - s_mlog[r]);
    }
    int idx = key - k0;
    if (a.nrg == 1) a.scores[(int64_t)unit * a.score_stride + idx] = sum;
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
    a.scores[(int64_t)unit * a.score_stride + j] = s;
  }
}

struct Plan {
  int nrg, nkc, kc, key_span;
  size_t stats_bytes, col_bytes;
};

Plan make_plan(const se_cache_t *c, const se_window_params_t *p) {
  Plan pl;
  const int R = c->n_q / c->n_kv;
  const int rows = R * p->n_query;
  pl.nrg = (rows + kRowsPerWG - 1) / kRowsPerWG;
  const int max_slots = c->max_blocks * c->page;
  pl.key_span = p->mode == SE_SCORE_CAUSAL ? max_slots : p->window - p->protect;
  const int span64 = (pl.key_span + 63) / 64 * 64;
  pl.kc = span64 < 1024 ? span64 : 1024;
  if (pl.kc < 64) pl.kc = 64;
  pl.nkc = (pl.key_span + pl.kc - 1) / pl.kc;
  const size_t units = (size_t)c->B * c->n_kv;
  pl.stats_bytes = se_host::align_up(units * pl.nrg * pl.nkc * kRowsPerWG * 2 * sizeof(float));
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
  se::Plan pl = se::make_plan(c, p);
  if (!ws || ws_bytes < pl.stats_bytes + pl.col_bytes) return SE_ERR_WORKSPACE;
  se::ScoreArgs a;
  a.k = (const char *)c->k_pool;
  a.bt = c->block_table;
  a.pos = c->pos_map;
  a.n_slots = c->n_slots;
  a.q = (const char *)q_win;
  a.q_pos = q_pos;
  a.scores = scores;
  a.stats = (float *)ws;
  a.colpart = pl.col_bytes ? (float *)((char *)ws + pl.stats_bytes) : nullptr;
  a.status = status;
  a.mode = p->mode;
  a.n_kv = c->n_kv;
  a.R = c->n_q / c->n_kv;
  a.wq = p->n_query;
  a.page = c->page;
  a.max_blocks = c->max_blocks;
  a.num_blocks = c->num_blocks;
  a.window = p->window;
  a.protect = p->protect;
  a.score_stride = p->score_stride;
  a.nrg = pl.nrg;
  a.nkc = pl.nkc;
  a.kc = pl.kc;
  a.key_span = pl.key_span;
  a.scale_log2 = p->scale * 1.4426950408889634f;
  const int units = c->B * c->n_kv;
  const dim3 grid(pl.nkc, pl.nrg, units);
  hipStream_t st = (hipStream_t)stream;
  if (mfma) {
    hipLaunchKernelGGL(se::stats_mfma, grid, dim3(se::kThreads), 0, st, a);
    hipLaunchKernelGGL(se::colsum_mfma, grid, dim3(se::kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((se::stats_valu<SE_DTYPE_F32, 64>), grid, dim3(se::kThreads), 0, st, a);
    hipLaunchKernelGGL((se::colsum_valu<SE_DTYPE_F32, 64>), grid, dim3(se::kThreads), 0, st, a);
  }
  if (pl.nrg > 1) {
    const int bx = (pl.key_span + 255) / 256;
    hipLaunchKernelGGL(se::colsum_reduce, dim3(bx, units), dim3(256), 0, st, a);
  }
  return se_host::launch_status();
}
