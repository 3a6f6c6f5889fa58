// Token2Chunk span expansion (KARA page, "Method" part 2): consecutive candidates in index order are the
// endpoints of possible chunks; a gap of 1..max_gap slots between them is rated by the IEEE fp32 quotient
// (s_a + s_b) / (b - a) of its endpoints' scores over its span, gaps are filled whole in rating order (ties:
// lower a) while the count of candidates plus fills stays within the budget, and the output is the ascending
// union followed by the protected tail.
//
// One workgroup per (sequence, KV head), with LDS sized to the input list. Ranks come from an all-pairs comparison
// of the gap priorities (one broadcast LDS read per comparison; the lists are a few hundred long), the greedy pass
// over the ranked gaps is inherently sequential and runs on one lane over the gap sizes stored in rank order, and
// a workgroup scan writes the expanded list in order.
#include "common.hpp"

namespace se {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxList = 4096;
constexpr int kMaxGap = 32767;  // gap sizes are kept as 16-bit values

struct T2CArgs {
  const int32_t *idx, *count, *n_slots;
  const float *scores;
  int32_t *idx_out, *count_out, *status;
  int32_t max_gap, budget, window, protect, score_stride, in_stride, out_stride, max_slots;
};

// LDS per workgroup for lists of L entries: candidates, gap priorities, gap index by rank (int32 each), gap size by
// rank (int16) and fill flags (byte)
inline size_t t2c_lds_bytes(int in_stride) {
  const size_t L = (size_t)((in_stride + 3) & ~3);
  return L * (4 + 4 + 4 + 2 + 1);
}

__global__ __launch_bounds__(kThreads) void t2c_kernel(T2CArgs a) {
  extern __shared__ __attribute__((aligned(16))) char s_dyn[];
  const int L = (a.in_stride + 3) & ~3;
  int *s_c = reinterpret_cast<int *>(s_dyn);
  float *s_prio = reinterpret_cast<float *>(s_c + L);  // NaN: the gap does not qualify
  int *s_gap_of = reinterpret_cast<int *>(s_prio + L);  // gap index of rank r
  short *s_size_of = reinterpret_cast<short *>(s_gap_of + L);  // its size
  unsigned char *s_fill = reinterpret_cast<unsigned char *>(s_size_of + L);
  __shared__ int s_wsum[kThreads / 64];
  __shared__ int s_m, s_bad, s_nq;
  const int unit = blockIdx.x, t = threadIdx.x;
  const int n = a.n_slots[unit];
  const int cnt = min(max(a.count[unit], 0), a.in_stride);
  const int base = n - a.window, thr = n - a.protect;
  const int32_t *in = a.idx + (int64_t)unit * a.in_stride;
  const float *sc = a.scores + (int64_t)unit * a.score_stride;
  if (t == 0) {
    s_m = 0;
    s_nq = 0;
    s_bad = (a.count[unit] < 0 || a.count[unit] > a.in_stride || base < 0 || n > a.max_slots) ? 1 : 0;
  }
  __syncthreads();
  for (int i = t; i < cnt; i += kThreads) {
    int s = in[i];
    if (s < base || s >= n || (i > 0 && in[i - 1] >= s)) atomicOr(&s_bad, 1);
    if (s < thr && (i + 1 == cnt || in[i + 1] >= thr)) s_m = i + 1;  // candidates are the prefix below thr
    s_c[i] = s;
  }
  __syncthreads();
  if (s_bad) {
    if (t == 0) {
      raise(a.status, SE_DEV_INDEX);
      a.count_out[unit] = 0;
    }
    return;
  }
  const int m = s_m;
  const int gaps = m > 0 ? m - 1 : 0;
  // gap priorities; a gap that does not qualify gets a quiet NaN, which no comparison below counts
  int nq = 0;
  for (int i = t; i < gaps; i += kThreads) {
    const int x = s_c[i], y = s_c[i + 1], g = y - x - 1;
    const bool q = g >= 1 && g <= a.max_gap;
    s_prio[i] = q ? __fdiv_rn(sc[x - base] + sc[y - base], (float)(y - x)) : __int_as_float(0x7fc00000);
    s_fill[i] = 0;
    nq += q;
  }
  if (nq) atomicAdd(&s_nq, nq);
  __syncthreads();
  // rank of each qualifying gap: priority descending, then lower left endpoint
  for (int i = t; i < gaps; i += kThreads) {
    const float pi = s_prio[i];
    if (pi != pi) continue;  // does not qualify
    int r = 0;
    for (int j = 0; j < gaps; ++j) {
      const float pj = s_prio[j];
      r += (pj > pi) | ((pj == pi) & (j < i));
    }
    s_gap_of[r] = i;
    s_size_of[r] = (short)(s_c[i + 1] - s_c[i] - 1);
  }
  __syncthreads();
  if (t == 0) {  // first fit in rank order until the budget is met
    int total = m;
    const int q = s_nq;
#pragma unroll 8
    for (int r = 0; r < q; ++r) {
      const int g = s_size_of[r];
      if (total >= a.budget) break;
      if (total + g <= a.budget) {
        s_fill[s_gap_of[r]] = 1;
        total += g;
      }
    }
  }
  __syncthreads();
  // emit candidates with their filled gaps in order, then the tail
  const int per = (m + kThreads - 1) / kThreads;
  int mine = 0;
  for (int i = t * per; i < min(m, (t + 1) * per); ++i) mine += 1 + ((i < gaps && s_fill[i]) ? s_c[i + 1] - s_c[i] - 1 : 0);
  int expanded;
  const int before = block_exscan<kThreads>(mine, s_wsum, expanded);
  const int total = expanded + (cnt - m);
  if (total > a.out_stride) {
    if (t == 0) {
      raise(a.status, SE_DEV_CAPACITY);
      a.count_out[unit] = 0;
    }
    return;
  }
  int32_t *out = a.idx_out + (int64_t)unit * a.out_stride;
  int o = before;
  for (int i = t * per; i < min(m, (t + 1) * per); ++i) {
    out[o++] = s_c[i];
    if (i < gaps && s_fill[i])
      for (int s = s_c[i] + 1; s < s_c[i + 1]; ++s) out[o++] = s;
  }
  for (int i = m + t; i < cnt; i += kThreads) out[expanded + (i - m)] = in[i];
  if (t == 0) a.count_out[unit] = total;
}

}  // namespace
}  // namespace se

extern "C" int32_t se_token2chunk(const se_cache_t *c, const int32_t *idx, const int32_t *count, const float *scores,
                                  const se_t2c_params_t *p, int32_t *idx_out, int32_t *count_out, int32_t *status,
                                  void *ws, size_t ws_bytes, se_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int32_t rc = se_host::check_cache(c);
  if (rc != SE_OK) return rc;
  if (!idx || !count || !scores || !p || !idx_out || !count_out) return SE_ERR_NULL;
  if (p->max_gap < 0 || p->budget < 0 || p->window <= 0 || p->protect < 0 || p->protect > p->window)
    return SE_ERR_PARAM;
  if (p->max_gap > se::kMaxGap) return SE_ERR_UNSUPPORTED;
  if (p->in_stride <= 0 || p->in_stride > se::kMaxList) return SE_ERR_UNSUPPORTED;
  if (p->score_stride < p->window - p->protect) return SE_ERR_SHAPE;
  if (p->out_stride < p->in_stride && p->out_stride < p->budget + p->protect) return SE_ERR_SHAPE;
  if (idx == idx_out || count == count_out) return SE_ERR_PARAM;  // out of place only
  se::T2CArgs a;
  a.idx = idx;
  a.count = count;
  a.n_slots = c->n_slots;
  a.scores = scores;
  a.idx_out = idx_out;
  a.count_out = count_out;
  a.status = status;
  a.max_gap = p->max_gap;
  a.budget = p->budget;
  a.window = p->window;
  a.protect = p->protect;
  a.score_stride = p->score_stride;
  a.in_stride = p->in_stride;
  a.out_stride = p->out_stride;
  a.max_slots = c->max_blocks * c->page;
  hipLaunchKernelGGL(se::t2c_kernel, dim3(c->B * c->n_kv), dim3(se::kThreads), se::t2c_lds_bytes(p->in_stride),
                     (hipStream_t)stream, a);
  return se_host::launch_status();
}
