// Device-side argument builder (K1).
//
// One workgroup turns the device-resident group sizes into
//   * exclusive offsets offs[E+1],
//   * a fixed-M tile work list that covers only non-empty groups (FBGEMM PR
//     "F8I4 Grouped Gemm Optimization for Sparse M", summary: the grouped GEMM
//     runs over min(total_M, groups) problems), and
//   * the dynamic-K order: groups by size descending (grouped_gemm PR
//     "Support GPU-resident batch sizes", review thread: kDynamicK problems
//     are sorted by k in descending order), ties by group index.
// The host never reads the sizes, so nothing synchronizes and the launch is
// graph-capturable.  At most 1024 groups: one thread per group, as in the
// single-threadblock design of the same PR's description.
#include "kernels.h"

namespace mg {

__device__ inline int64_t wave_incl_scan(int64_t x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int64_t t = __shfl_up(x, d, kWave);
    if (lane >= d) x += t;
  }
  return x;
}

// Inclusive block scan of one int64 per thread (blockDim.x <= 1024).
__device__ inline int64_t block_incl_scan(int64_t x, int64_t* s_wave) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  x = wave_incl_scan(x);
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int64_t w = lane < nwaves ? s_wave[lane] : 0;
    w = wave_incl_scan(w);
    if (lane < nwaves) s_wave[lane] = w;
  }
  __syncthreads();
  if (wave > 0) x += s_wave[wave - 1];
  __syncthreads();
  return x;
}

__global__ void __launch_bounds__(1024) build_worklist_kernel(BuildArgs a) {
  __shared__ int64_t s_wave[16];
  __shared__ int32_t s_tile_start[kMaxExperts + 1];
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_eff[kMaxExperts];
  __shared__ int s_flags;

  const int tid = threadIdx.x;
  const int E = a.E;
  if (tid == 0) s_flags = 0;
  __syncthreads();

  int64_t sz = 0;
  if (tid < E) {
    int32_t raw = a.sizes[tid];
    if (raw < 0) atomicOr(&s_flags, 1);
    sz = raw > 0 ? raw : 0;
  }
  const int64_t incl = block_incl_scan(sz, s_wave);
  const int64_t excl = incl - sz;
  const int64_t total = a.total_M;
  const int64_t off = excl < total ? excl : total;
  const int64_t end = incl < total ? incl : total;
  const int32_t eff = (int32_t)(end - off);
  if (tid == E - 1 && incl > total) atomicOr(&s_flags, 2);

  const int32_t tiles = (int32_t)((eff + a.bm - 1) / a.bm);
  const int64_t tincl = block_incl_scan(tiles, s_wave);
  if (tid < E) {
    s_off[tid] = (int32_t)off;
    s_eff[tid] = eff;
    s_tile_start[tid] = (int32_t)(tincl - tiles);
    a.offs[tid] = (int32_t)off;
    if (tid == E - 1) {
      a.offs[E] = (int32_t)end;
      s_tile_start[E] = (int32_t)tincl;
      if (a.want_fixed) *a.count = (int32_t)tincl;
    }
  }
  __syncthreads();

  if (a.want_fixed) {
    const int32_t n = s_tile_start[E];
    for (int32_t t = tid; t < n; t += blockDim.x) {
      // last group whose first tile is <= t (empty groups share their
      // successor's start, so the match is the non-empty owner of tile t)
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_tile_start[mid] <= t) lo = mid; else hi = mid - 1;
      }
      const int g = lo;
      const int32_t i = t - s_tile_start[g];
      const int32_t r0 = i * a.bm;
      const int32_t rows = s_eff[g] - r0 < a.bm ? s_eff[g] - r0 : a.bm;
      int4 ent = make_int4(g, s_off[g] + r0, rows, 0);
      reinterpret_cast<int4*>(a.entries)[t] = ent;
    }
  }
  if (a.want_dynamic && tid < E) {
    int rank = 0;
    for (int h = 0; h < E; ++h) {
      const int32_t e = s_eff[h];
      rank += (e > eff) || (e == eff && h < tid);
    }
    reinterpret_cast<int4*>(a.dk_entries)[rank] = make_int4(tid, (int32_t)off, eff, 0);
  }
  if (tid == 0 && s_flags != 0 && a.err != nullptr) {
    *a.err = (s_flags & 1) ? 1 : 2;
  }
}

hipError_t launch_build_worklist(const BuildArgs& a, hipStream_t stream) {
  int threads = (int)align_up(a.E, kWave);
  if (threads < kWave) threads = kWave;
  hipLaunchKernelGGL(build_worklist_kernel, dim3(1), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mg
