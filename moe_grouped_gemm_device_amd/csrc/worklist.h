// Device-side group table: the argument builder that every grouped-GEMM
// kernel runs in its prologue, and that the standalone builder kernel writes
// out for inspection.
//
// From the device-resident group sizes one 256-thread workgroup computes in
// LDS, with no host involvement (grouped_gemm PR "Support GPU-resident batch
// sizes": a single-block scan of the batch sizes fills the kernel arguments):
//   off[g]     exclusive prefix sum of the clamped sizes,
//   eff[g]     the clamped size (negative -> 0, nothing past total_M),
//   tstart[g]  first fixed-M tile of group g (tiles of bm rows; only
//              non-empty groups own tiles -- FBGEMM PR "F8I4 Grouped Gemm
//              Optimization for Sparse M": min(total_M, groups) problems),
//   order[i]   the dynamic-K order: groups by size descending, ties by index
//              (same PR as above, review thread: kDynamicK sorts by k).
// A fixed-M table needs tstart and a dynamic-K table needs order, never
// both, so the two share one array (less LDS beside the GEMM's K stages).
#pragma once

#include "common.h"

namespace mg {

constexpr int kTableThreads = 256;

// LDS bytes a table for E groups needs (off, eff, tstart or order, and the
// scan scratch).
__host__ __device__ inline int table_lds_bytes(int E) { return 4 * (3 * (E + 1)) + 2 * 8 * 8; }

struct GroupTable {
  int32_t* off;     // [E+1]
  int32_t* eff;     // [E]
  int32_t* tstart;  // [E+1]  (fixed-M tables)
  int32_t* order;   // [E]    (dynamic-K tables; same storage as tstart)
  int64_t* scratch; // [16]
};

__device__ inline GroupTable carve_table(void* lds, int E) {
  int32_t* p = reinterpret_cast<int32_t*>(lds);
  GroupTable t;
  t.scratch = reinterpret_cast<int64_t*>(p);
  p += 32;
  t.off = p;
  t.eff = p + (E + 1);
  t.tstart = p + 2 * (E + 1);
  t.order = t.tstart;
  return t;
}

__device__ inline int64_t wave_incl_scan64(int64_t x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t t = __shfl_up(x, d, kWave);
    if (lane >= d) x += t;
  }
  return x;
}

// Inclusive scan over the threads of the workgroup (at most 8 waves).
__device__ inline int64_t block_incl_scan64(int64_t x, int64_t* s_wave) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  x = wave_incl_scan64(x);
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  __syncthreads();
  return x + before;
}

// Builds the table.  Must be called by all threads of the workgroup
// (256 or 512; groups are owned by the first 256).  Returns (in every
// thread) an error code: 0, 1 (a negative size) or 2 (sizes sum past
// total_M).  want_order builds the dynamic-K ordering (O(E^2/256) work)
// instead of the fixed-M tile starts.
// Up to 64 * P groups, P consecutive groups per lane of wave 0: no
// workgroup-wide scans, one barrier.  The running sum of the sizes saturates
// at total_M + 1 (every partial sum then fits 32 bits, and min(sum, total_M)
// and "sum > total_M" are unchanged; a saturating sum of non-negative terms
// does not depend on how the terms are grouped), so the results equal the
// general path's.
template <int P>
__device__ inline int build_group_table_wave(const int32_t* __restrict__ sizes, int E, int64_t total_M, int bm,
                                             bool want_order, GroupTable t) {
  const int lane = threadIdx.x & (kWave - 1);
  if (threadIdx.x < kWave) {
    const int g0 = lane * P;
    const uint32_t cap = (uint32_t)(total_M + 1);   // total_M < 2^31
    const uint32_t tm = (uint32_t)total_M;
    int32_t raw[P];
#pragma unroll
    for (int i = 0; i < P; ++i) raw[i] = g0 + i < E ? sizes[g0 + i] : 0;
    // the lane's own groups: saturating inclusive sums
    uint32_t pre[P];
    uint32_t run = 0;
    bool neg = false;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      neg = neg || raw[i] < 0;
      const uint32_t v = raw[i] > 0 ? ((uint32_t)raw[i] < cap ? (uint32_t)raw[i] : cap) : 0u;
      const uint64_t sum = (uint64_t)run + v;
      run = sum < cap ? (uint32_t)sum : cap;
      pre[i] = run;
    }
    // lane totals across the wave
    uint32_t incl = run;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)incl, d, kWave);
      if (lane >= d) {
        const uint64_t sum = (uint64_t)incl + o;
        incl = sum < cap ? (uint32_t)sum : cap;
      }
    }
    const uint32_t up = (uint32_t)__shfl_up((int)incl, 1, kWave);
    const uint32_t excl = lane == 0 ? 0u : up;
    int32_t off[P], eff[P];
    int32_t tiles = 0;
    uint32_t a = excl < tm ? excl : tm;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint64_t sum = (uint64_t)excl + pre[i];
      const uint32_t end = sum < cap ? (uint32_t)sum : cap;
      const uint32_t b = end < tm ? end : tm;
      off[i] = (int32_t)a;
      eff[i] = (int32_t)(b - a);   // 0 past E: those groups add nothing
      tiles += (int32_t)(((uint32_t)eff[i] + (uint32_t)bm - 1u) / (uint32_t)bm);
      a = b;
    }
    int32_t tincl = tiles;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int32_t o = __shfl_up(tincl, d, kWave);
      if (lane >= d) tincl += o;
    }
    int32_t tr = tincl - tiles;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (g0 + i < E) {
        t.off[g0 + i] = off[i];
        t.eff[g0 + i] = eff[i];
        if (!want_order) t.tstart[g0 + i] = tr;
      }
      tr += (int32_t)(((uint32_t)eff[i] + (uint32_t)bm - 1u) / (uint32_t)bm);
    }
    // the last lane's inclusive sums are the totals (lanes past E add 0)
    const uint32_t total = (uint32_t)__shfl((int)incl, kWave - 1, kWave);
    const int32_t ttotal = __shfl(tincl, kWave - 1, kWave);
    if (lane == 0) {
      t.off[E] = (int32_t)(total < tm ? total : tm);
      if (!want_order) t.tstart[E] = ttotal;
    }
    const bool any_neg = __ballot(neg) != 0;
    const bool any_over = total > tm;
    if (want_order) {   // every lane of the wave takes part in the shuffles
      // rank of group g: groups with a larger size, or the same size and a
      // smaller index (a slot past E holds size 0 and a larger index than
      // any group, so it never counts)
      int rank[P];
#pragma unroll
      for (int i = 0; i < P; ++i) rank[i] = 0;
      const int lanes = (E + P - 1) / P;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        for (int hl = 0; hl < lanes; ++hl) {
          const int32_t e = __shfl(eff[j], hl, kWave);
          const int h = hl * P + j;
#pragma unroll
          for (int i = 0; i < P; ++i) rank[i] += (e > eff[i]) || (e == eff[i] && h < g0 + i);
        }
      }
#pragma unroll
      for (int i = 0; i < P; ++i)
        if (g0 + i < E) t.order[rank[i]] = g0 + i;
    }
    if (lane == 0) t.scratch[15] = any_neg ? 1 : any_over ? 2 : 0;
  }
  __syncthreads();
  return (int)t.scratch[15];
}

__device__ inline int build_group_table(const int32_t* __restrict__ sizes, int E, int64_t total_M, int bm,
                                        bool want_order, GroupTable t) {
  if (E <= kWave) return build_group_table_wave<1>(sizes, E, total_M, bm, want_order, t);
  if (E <= 4 * kWave) return build_group_table_wave<4>(sizes, E, total_M, bm, want_order, t);
  const int tid = threadIdx.x;
  const int per = (E + kTableThreads - 1) / kTableThreads;   // groups per thread (<= 4)
  const int g0 = tid * per;
  int64_t local = 0;
  int neg = 0;
  int32_t raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    raw[i] = 0;
    if (i < per && g0 + i < E) {
      const int32_t s = sizes[g0 + i];
      if (s < 0) neg = 1;
      raw[i] = s > 0 ? s : 0;
      local += raw[i];
    }
  }
  const int64_t incl = block_incl_scan64(local, t.scratch);
  int64_t run = incl - local;
  int32_t tiles_local = 0;
  int32_t eff_l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    eff_l[i] = 0;
    if (i < per && g0 + i < E) {
      const int64_t a = run < total_M ? run : total_M;
      const int64_t b0 = run + raw[i];
      const int64_t b = b0 < total_M ? b0 : total_M;
      t.off[g0 + i] = (int32_t)a;
      eff_l[i] = (int32_t)(b - a);
      t.eff[g0 + i] = eff_l[i];
      tiles_local += (eff_l[i] + bm - 1) / bm;
      run = b0;
    }
  }
  // grand total and error flags (last thread holding groups knows the sum)
  const int64_t tincl = block_incl_scan64(tiles_local, t.scratch + 8);
  int32_t tr = (int32_t)(tincl - tiles_local);
  if (!want_order) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < per && g0 + i < E) {
        t.tstart[g0 + i] = tr;
        tr += (eff_l[i] + bm - 1) / bm;
      }
    }
  }
  const int last = (E - 1) / per;   // thread owning group E-1
  int over = 0;
  if (tid == last) {
    t.off[E] = (int32_t)(incl < total_M ? incl : total_M);
    if (!want_order) t.tstart[E] = (int32_t)tincl;
    over = incl > total_M;
  }
  // predicate reductions (each returns non-zero if any thread's is)
  const int any_neg = __syncthreads_or(neg);
  const int any_over = __syncthreads_or(over);
  if (want_order) {
    for (int g = tid; g < E; g += blockDim.x) {
      const int32_t eg = t.eff[g];
      int rank = 0;
      for (int h = 0; h < E; ++h) {
        const int32_t e = t.eff[h];
        rank += (e > eg) || (e == eg && h < g);
      }
      t.order[rank] = g;
    }
    __syncthreads();
  }
  return any_neg ? 1 : any_over ? 2 : 0;
}

// Fixed-M tile index -> {group, first row, rows}.
__device__ inline int4 fixed_m_entry(const GroupTable& t, int E, int bm, int32_t tile) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {   // last group whose first tile is <= tile
    const int mid = (lo + hi + 1) >> 1;
    if (t.tstart[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int32_t i = tile - t.tstart[lo];
  const int32_t r0 = i * bm;
  const int32_t rows = t.eff[lo] - r0 < bm ? t.eff[lo] - r0 : bm;
  return make_int4(lo, t.off[lo] + r0, rows, 0);
}

}  // namespace mg
