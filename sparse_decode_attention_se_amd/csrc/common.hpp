// Shared device and host helpers of libse (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/se.h"

#define SE_DEV __device__ __forceinline__

namespace se {

constexpr int kWave = 64;

// ---- element types --------------------------------------------------------------------------------------------
// bf16 is carried as its 16-bit pattern; widening to fp32 is a shift.
SE_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
SE_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
SE_DEV uint16_t f32_to_bf16_exact(float x) { return (uint16_t)(__float_as_uint(x) >> 16); }  // x already bf16

// 16-byte vector load / store (global, through the vector memory path)
struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};
SE_DEV u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// A 16-byte load marked non-temporal, for data read once. A streaming read of 8 GiB reaches 7.09 TB/s with it
// against 6.29 with plain loads, but it does not find what the last-level cache holds: data that a kernel of the
// same step has just written or read (a compaction's moved rows, the scorer's region keys) is read with plain
// loads (measured per call on each workload).
typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));
SE_DEV u32x4 ld16_stream(const void *p) {
  return __builtin_bit_cast(u32x4, __builtin_nontemporal_load(reinterpret_cast<const u32v4 *>(p)));
}
// a 16-byte store marked non-temporal, for K and V rows written into the pools: they go to memory without being
// kept in the caches, where the next kernel's streaming reads would otherwise meet them
SE_DEV void st16_stream(void *p, const u32x4 &v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32v4, v), reinterpret_cast<u32v4 *>(p));
}
SE_DEV void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// ---- wave reductions ------------------------------------------------------------------------------------------
// DPP row_ror:n rotates within a row of 16 lanes; four steps leave the row total in every lane of the row.
template <int CTRL>
SE_DEV float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

SE_DEV float row16_sum(float x) {
  x += dpp_f<kRowRor8>(x);
  x += dpp_f<kRowRor4>(x);
  x += dpp_f<kRowRor2>(x);
  x += dpp_f<kRowRor1>(x);
  return x;
}
SE_DEV float row16_max(float x) {
  x = fmaxf(x, dpp_f<kRowRor8>(x));
  x = fmaxf(x, dpp_f<kRowRor4>(x));
  x = fmaxf(x, dpp_f<kRowRor2>(x));
  x = fmaxf(x, dpp_f<kRowRor1>(x));
  return x;
}
// sum over lanes with the same (lane % 16): the four rows of the wave. v_permlane16_swap with both operands x
// returns (x of the even row of each row pair, x of the odd row) in every lane of the pair; v_permlane32_swap does
// the same for the two halves of the wave. Both stay on the VALU (no LDS crossbar).
SE_DEV float cross_row_sum(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
SE_DEV float cross_row_max(float x) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
// sums of 16 values over the 16 lanes of a row, scattered: lane j of the row receives the total of value j.
// Four exchange rounds (partners 15 - j, 7 - j within each half, j ^ 2, j ^ 1); each halves the values a lane
// carries: 15 DPP additions instead of 16 full row sums.
template <int N, int CTRL, int M>
SE_DEV void rs_round(float (&v)[M], bool hi) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = hi ? v[N / 2 + i] : v[i];
    const float send = hi ? v[i] : v[N / 2 + i];
    v[i] = keep + dpp_f<CTRL>(send);
  }
}
SE_DEV float row16_reduce_scatter(float (&v)[16]) {
  const int j = threadIdx.x & 15;
  rs_round<16, 0x140>(v, j & 8);  // row_mirror: j <-> 15 - j
  rs_round<8, 0x141>(v, j & 4);   // row_half_mirror: j <-> 7 - j
  rs_round<4, 0x4e>(v, j & 2);    // quad_perm [2,3,0,1]
  rs_round<2, 0xb1>(v, j & 1);    // quad_perm [1,0,3,2]
  return v[0];
}
// the same for 8 values: three rounds within each half-row leave lanes j and j ^ 8 with the sums over their halves
// of value j % 8, and one rotation by 8 adds the halves
SE_DEV float row16_reduce_scatter(float (&v)[8]) {
  const int j = threadIdx.x & 15;
  rs_round<8, 0x141>(v, j & 4);
  rs_round<4, 0x4e>(v, j & 2);
  rs_round<2, 0xb1>(v, j & 1);
  return v[0] + dpp_f<kRowRor8>(v[0]);
}
// lane N of each row of 16 lanes, in every lane of the row (DPP row_newbcast)
template <int N>
SE_DEV float row16_bcast(float x) {
  return dpp_f<0x150 + N>(x);
}

SE_DEV float wave_sum(float x) { return cross_row_sum(row16_sum(x)); }
SE_DEV float wave_max(float x) { return cross_row_max(row16_max(x)); }

SE_DEV int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Exclusive prefix sum of v over the workgroup's NTH threads in thread order, and the total: a scan within each
// wave by lane shifts, then the waves' totals through LDS (s_wsum: NTH / 64 ints). Two barriers; every thread of
// the workgroup must call it, and s_wsum may be reused right after (the first barrier guards it).
template <int NTH>
SE_DEV int block_exscan(int v, int *s_wsum, int &total) {
  constexpr int kWaves = NTH / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __syncthreads();
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int x = s_wsum[w];
    before += w < wave ? x : 0;
    total += x;
  }
  return before + incl - v;
}

SE_DEV bool blk_ok(int32_t blk, int32_t num_blocks) { return blk >= 0 && blk < num_blocks; }

// fp32 -> u32 with the same order (unsigned comparison), -0 taken as +0: the selection keys of top-K
SE_DEV uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- status ---------------------------------------------------------------------------------------------------
SE_DEV void raise(int32_t *status, int32_t bit) {
  if (status) atomicOr(status, bit);
}

// ---- cache addressing -----------------------------------------------------------------------------------------
struct CacheView {
  const char *k, *v;
  const int32_t *bt, *pos;
  int32_t n_kv, d, page, max_blocks, row_bytes;
  SE_DEV int64_t max_slots() const { return (int64_t)max_blocks * page; }
  // byte offset of slot s of (b, g) in a pool, given the physical block
  SE_DEV int64_t row_off(int32_t blk, int32_t g, int32_t s) const {
    return (((int64_t)blk * n_kv + g) * page + (s % page)) * row_bytes;
  }
};

inline int elem_bytes(int dtype) { return dtype == SE_DTYPE_BF16 ? 2 : 4; }

}  // namespace se

// ---- host-side validation shared by the entry points ---------------------------------------------------------
namespace se_host {

inline int32_t check_cache(const se_cache_t *c) {
  if (!c) return SE_ERR_NULL;
  if (!c->k_pool || !c->v_pool || !c->block_table || !c->pos_map || !c->ctx_len || !c->n_slots) return SE_ERR_NULL;
  if (c->dtype != SE_DTYPE_F32 && c->dtype != SE_DTYPE_BF16) return SE_ERR_DTYPE;
  if (c->B <= 0 || c->n_kv <= 0 || c->n_q <= 0 || c->d <= 0 || c->page <= 0 || c->num_blocks <= 0 ||
      c->max_blocks <= 0 || c->slot_cap < 0)
    return SE_ERR_SHAPE;
  if (c->n_q % c->n_kv != 0) return SE_ERR_SHAPE;
  if ((long long)c->max_blocks * c->page > (1ll << 30)) return SE_ERR_SHAPE;
  return SE_OK;
}

inline int32_t launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SE_OK : SE_ERR_HIP;
}

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

}  // namespace se_host
