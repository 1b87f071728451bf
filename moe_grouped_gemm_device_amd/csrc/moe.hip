// Token permutation for the token-sorted fused MoE path (K5), SiLU-and-mul
// (K6) and the top-k weighted combine (K7), for gfx950.
//
// applied-ai issue "Column-major fused MoE": moe_align_block_size sorts the
// flattened (token, slot) pairs by expert and pads every expert's run to a
// multiple of block_m with the sentinel T*k (docstring and worked example);
// fused_moe_kernel reads A row sorted_id // top_k and masks the sentinel;
// fused_moe applies silu_and_mul between the two GEMMs and sums the top-k
// expert outputs of every token.
//
// The alignment is a stable counting sort with no device-to-host traffic.
// Up to 1024 pairs it runs in one workgroup (perm_small_kernel); beyond, in
// three small kernels:
//   1. per chunk of pairs: stable rank of every pair among the chunk's pairs
//      with the same expert, and the chunk's per-expert counts;
//   2. one workgroup: per-expert totals, padded run starts, per-chunk bases,
//      block -> expert table, padded sizes, padded length, and the sentinel
//      in every slot no pair will take (each run's padding and the tail up
//      to the capacity);
//   3. scatter: position = base[chunk][expert] + rank; inverse positions.
// The gather of X rows runs last.
#include "kernels.h"

namespace mg {

constexpr int PT = 256;                 // threads per permutation workgroup

struct PermWs {
  int32_t* chunk_counts;   // [nchunks][E], becomes chunk bases after pass 2
  int32_t* rank;           // [P]
};

// Stable within-chunk ranks.  A chunk is processed in sub-chunks of 256
// pairs; inside a wave, lanes with equal experts are matched with ballots;
// waves take turns (in order) to advance the per-expert cursors in LDS.
__global__ void __launch_bounds__(PT) perm_rank_kernel(const int32_t* __restrict__ ids, int64_t P, int32_t E,
                                                      int64_t chunk, int32_t* __restrict__ chunk_counts,
                                                      int32_t* __restrict__ rank) {
  extern __shared__ int32_t cursor[];   // [E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += PT) cursor[e] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk < P ? c0 + chunk : P;
  for (int64_t sub = c0; sub < c1; sub += PT) {
    const int64_t f = sub + tid;
    int e = -1;
    if (f < c1) {
      e = ids[f];
      if (e < 0 || e >= E) e = -1;
    }
    uint64_t active = __ballot(e >= 0);
    int my_rank = 0, my_cnt = 0, my_leader = 0;
    while (active) {
      const int leader = __ffsll((unsigned long long)active) - 1;
      const int el = __shfl(e, leader, kWave);
      const uint64_t m = __ballot(e == el) & active;
      if ((m >> lane) & 1) {
        my_rank = __popcll(m & ((1ull << lane) - 1));
        my_cnt = __popcll(m);
        my_leader = leader;
      }
      active &= ~m;
    }
    int base = 0;
    for (int w = 0; w < PT / kWave; ++w) {
      if (wave == w && e >= 0 && lane == my_leader) {
        base = cursor[e];
        cursor[e] = base + my_cnt;
      }
      __syncthreads();
    }
    const int b = __shfl(base, my_leader, kWave);
    if (e >= 0) rank[f] = b + my_rank;
  }
  for (int e = tid; e < E; e += PT) chunk_counts[(int64_t)blockIdx.x * E + e] = cursor[e];
}

// One workgroup (>= E threads, <= 1024): thread e owns expert e.
__global__ void __launch_bounds__(1024) perm_plan_kernel(int32_t E, int32_t block_m, int64_t nchunks,
                                                        int32_t* __restrict__ chunk_counts,
                                                        int32_t* __restrict__ expert_ids, int64_t nblk,
                                                        int32_t* __restrict__ ntpp,
                                                        int32_t* __restrict__ padded,
                                                        int32_t* __restrict__ sorted_ids, int64_t cap,
                                                        int32_t sentinel) {
  __shared__ int32_t s_start[kMaxExperts + 1];
  __shared__ int32_t s_blk[kMaxExperts + 1];
  const int e = threadIdx.x;
  // the per-chunk counts are read eight at a time, so that one memory
  // latency covers eight chunks instead of one
  constexpr int PB = 8;
  int64_t total = 0;
  if (e < E) {
    int64_t c = 0;
    for (; c + PB <= nchunks; c += PB) {
      int32_t v[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) v[u] = chunk_counts[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < PB; ++u) total += v[u];
    }
    for (; c < nchunks; ++c) total += chunk_counts[c * E + e];
  }
  const int32_t pad = (int32_t)((total + block_m - 1) / block_m * block_m);
  if (e < E) padded[e] = pad;
  // exclusive scan of padded sizes across experts (E <= 1024; serial in LDS
  // by thread 0 keeps this obviously right and costs ~E adds)
  if (e < E) s_start[e] = pad;
  __syncthreads();
  if (e == 0) {
    int32_t run = 0, blk = 0;
    for (int h = 0; h < E; ++h) {
      const int32_t p = s_start[h];
      s_start[h] = run;
      s_blk[h] = blk;
      run += p;
      blk += p / block_m;
    }
    s_start[E] = run;
    s_blk[E] = blk;
    *ntpp = run;
  }
  __syncthreads();
  if (e < E) {
    int32_t base = s_start[e];
    int64_t c = 0;
    for (; c + PB <= nchunks; c += PB) {
      int32_t v[PB];
#pragma unroll
      for (int u = 0; u < PB; ++u) v[u] = chunk_counts[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        chunk_counts[(c + u) * E + e] = base;
        base += v[u];
      }
    }
    for (; c < nchunks; ++c) {
      const int32_t cnt = chunk_counts[c * E + e];
      chunk_counts[c * E + e] = base;
      base += cnt;
    }
    for (int32_t b = s_blk[e]; b < s_blk[e + 1] && b < nblk; ++b) expert_ids[b] = e;
    // this run's padding (after its base + total pairs) takes the sentinel
    for (int32_t i = base; i < s_start[e + 1] && i < cap; ++i) sorted_ids[i] = sentinel;
  }
  for (int64_t i = (int64_t)s_start[E] + threadIdx.x; i < cap; i += blockDim.x) sorted_ids[i] = sentinel;
}

__global__ void __launch_bounds__(256) perm_scatter_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                          int32_t E, int64_t chunk,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ rank,
                                                          int32_t* __restrict__ sorted_ids,
                                                          int32_t* __restrict__ inv) {
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= P) return;
  const int e = ids[f];
  if (e < 0 || e >= E) {
    inv[f] = -1;
    return;
  }
  const int64_t c = f / chunk;
  const int32_t pos = chunk_base[c * E + e] + rank[f];
  sorted_ids[pos] = (int32_t)f;
  inv[f] = pos;
}

// x_sorted[i] = x[sorted[i] / k] (16 bytes per thread), zeros for the sentinel.
__global__ void __launch_bounds__(256) gather_rows_kernel(const uint16_t* __restrict__ x, int64_t P, int32_t k,
                                                         int32_t hidden, const int32_t* __restrict__ sorted_ids,
                                                         int64_t rows, uint16_t* __restrict__ out) {
  const int cpr = hidden >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / cpr;
  const int ch = (int)(idx - row * cpr);
  if (row >= rows) return;
  const int32_t f = sorted_ids[row];
  uint4 v = make_uint4(0, 0, 0, 0);
  if (f >= 0 && f < P) v = *reinterpret_cast<const uint4*>(x + (int64_t)(f / k) * hidden + ch * 8);
  *reinterpret_cast<uint4*>(out + row * hidden + ch * 8) = v;
}

// Small routings (at most 1024 pairs, decode-sized) in one workgroup and one
// launch: the stable ranks of perm_rank (ballot matching inside a wave,
// waves advancing the per-expert cursors in order), the plan of
// perm_plan and the scatter, with the ranks kept in registers.
constexpr int kPermSmall = 1024;

__global__ void __launch_bounds__(kPermSmall) perm_small_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                               int32_t E, int32_t block_m,
                                                               int32_t* __restrict__ expert_ids, int64_t nblk,
                                                               int32_t* __restrict__ ntpp,
                                                               int32_t* __restrict__ padded,
                                                               int32_t* __restrict__ sorted_ids, int64_t cap,
                                                               int32_t* __restrict__ inv, int32_t sentinel) {
  __shared__ int32_t cursor[kMaxExperts];
  __shared__ int32_t s_start[kMaxExperts + 1];
  __shared__ int32_t s_blk[kMaxExperts + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kPermSmall) cursor[e] = 0;
  __syncthreads();
  // stable rank of pair tid among the earlier pairs of its expert
  const int f = tid;
  int e = -1;
  if (f < P) {
    e = ids[f];
    if (e < 0 || e >= E) e = -1;
  }
  uint64_t active = __ballot(e >= 0);
  int my_rank = 0, my_cnt = 0, my_leader = 0;
  while (active) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const int el = __shfl(e, leader, kWave);
    const uint64_t m = __ballot(e == el) & active;
    if ((m >> lane) & 1) {
      my_rank = __popcll(m & ((1ull << lane) - 1));
      my_cnt = __popcll(m);
      my_leader = leader;
    }
    active &= ~m;
  }
  int base = 0;
  for (int w = 0; w < kPermSmall / kWave; ++w) {
    if (wave == w && e >= 0 && lane == my_leader) {
      base = cursor[e];
      cursor[e] = base + my_cnt;
    }
    __syncthreads();
  }
  const int rank = __shfl(base, my_leader, kWave) + my_rank;
  // plan: padded run sizes, their starts (serial scan by thread 0, E adds),
  // the block -> expert table, the sentinel in every slot no pair takes
  int32_t pad = 0;
  if (tid < E) {
    pad = (cursor[tid] + block_m - 1) / block_m * block_m;
    padded[tid] = pad;
    s_start[tid] = pad;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0, blk = 0;
    for (int h = 0; h < E; ++h) {
      const int32_t p = s_start[h];
      s_start[h] = run;
      s_blk[h] = blk;
      run += p;
      blk += p / block_m;
    }
    s_start[E] = run;
    s_blk[E] = blk;
    *ntpp = run;
  }
  __syncthreads();
  if (tid < E) {
    for (int32_t b = s_blk[tid]; b < s_blk[tid + 1] && b < nblk; ++b) expert_ids[b] = tid;
    for (int32_t i = s_start[tid] + cursor[tid]; i < s_start[tid + 1] && i < cap; ++i) sorted_ids[i] = sentinel;
  }
  for (int64_t i = (int64_t)s_start[E] + tid; i < cap; i += kPermSmall) sorted_ids[i] = sentinel;
  // scatter
  if (f < P) {
    if (e >= 0) {
      const int32_t pos = s_start[e] + rank;
      sorted_ids[pos] = (int32_t)f;
      inv[f] = pos;
    } else {
      inv[f] = -1;
    }
  }
}

static int64_t perm_chunk(int64_t P, int32_t E) {
  // keep nchunks * E <= 2^20 so the count table stays small
  int64_t chunk = 1024;
  while (cdiv(P, chunk) * E > (1 << 20)) chunk *= 2;
  return chunk;
}

int64_t perm_workspace_bytes(int64_t P, int32_t E) {
  const int64_t chunk = perm_chunk(P, E);
  const int64_t nchunks = cdiv(P > 0 ? P : 1, chunk);
  return align_up(nchunks * E * 4, 256) + align_up((P > 0 ? P : 1) * 4, 256);
}

hipError_t launch_moe_permute_ws(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t block_m,
                                 const uint16_t* x, int32_t hidden, int32_t* sorted_ids, int32_t* expert_ids,
                                 int32_t* ntpp, int32_t* inv, int32_t* padded, uint16_t* x_sorted,
                                 int64_t cap, int64_t nblk, void* ws, hipStream_t stream) {
  const int64_t P = T * k;
  const int64_t chunk = perm_chunk(P, E);
  const int64_t nchunks = cdiv(P > 0 ? P : 1, chunk);
  int32_t* counts = reinterpret_cast<int32_t*>(ws);
  int32_t* rank = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(ws) + align_up(nchunks * E * 4, 256));

  if (P <= kPermSmall) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(kPermSmall), 0, stream, ids, P, E, block_m, expert_ids,
                       nblk, ntpp, padded, sorted_ids, cap, inv, (int32_t)P);
  } else {
    hipLaunchKernelGGL(perm_rank_kernel, dim3((unsigned)nchunks), dim3(PT), (size_t)E * 4, stream, ids, P, E,
                       chunk, counts, rank);
    int plan_threads = (int)align_up(E, kWave);
    hipLaunchKernelGGL(perm_plan_kernel, dim3(1), dim3(plan_threads), 0, stream, E, block_m, nchunks, counts,
                       expert_ids, nblk, ntpp, padded, sorted_ids, cap, (int32_t)P);
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)cdiv(P, 256)), dim3(256), 0, stream, ids, P, E,
                       chunk, counts, rank, sorted_ids, inv);
  }
  if (x != nullptr && x_sorted != nullptr && cap > 0) {
    const int64_t n = cap * (hidden / 8);
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, x, P, k,
                       hidden, sorted_ids, cap, x_sorted);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K7: out[t, :] = bf16(sum_j w[t,j] * y[inv[t*k+j], :]), fp32, j ascending.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) unpermute_kernel(const uint16_t* __restrict__ y,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w, int64_t T, int32_t k,
                                                       int32_t hidden, uint16_t* __restrict__ out) {
  const int ch = blockIdx.x * 256 + threadIdx.x;
  if (ch * 8 >= hidden) return;
  for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {   // grid rows stride over the tokens
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const int32_t pos = inv[t * k + j];
      if (pos < 0) continue;
      const float wt = w ? w[t * k + j] : 1.f;
      const uint4 v = *reinterpret_cast<const uint4*>(y + (int64_t)pos * hidden + ch * 8);
      const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wt * bf16_to_f32(ww[i] & 0xFFFFu);
        acc[2 * i + 1] += wt * bf16_to_f32(ww[i] >> 16);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(out + t * hidden + ch * 8) = o;
  }
}

hipError_t launch_moe_unpermute(const uint16_t* y, const int32_t* inv, const float* w, int64_t T, int32_t k,
                                int32_t hidden, uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(hidden / 8, 256), (unsigned)(T < 65535 ? T : 65535));   // grid y is at most 65535
  hipLaunchKernelGGL(unpermute_kernel, grid, dim3(256), 0, stream, y, inv, w, T, k, hidden, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K6: act = bf16(silu(gate) * up), gate = first half of the row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) silu_mul_kernel(const uint16_t* __restrict__ h, int64_t rows,
                                                      int32_t inter, uint16_t* __restrict__ act) {
  const int cpr = inter >> 3;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / cpr;
  const int ch = (int)(idx - row * cpr);
  if (row >= rows) return;
  const uint16_t* hr = h + row * (2 * (int64_t)inter);
  const uint4 g = *reinterpret_cast<const uint4*>(hr + ch * 8);
  const uint4 u = *reinterpret_cast<const uint4*>(hr + inter + ch * 8);
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
  const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float g0 = bf16_to_f32(gw[i] & 0xFFFFu), g1 = bf16_to_f32(gw[i] >> 16);
    const float u0 = bf16_to_f32(uw[i] & 0xFFFFu), u1 = bf16_to_f32(uw[i] >> 16);
    const float a0 = g0 / (1.f + expf(-g0)) * u0;
    const float a1 = g1 / (1.f + expf(-g1)) * u1;
    o[i] = pack_bf16x2(a0, a1);
  }
  *reinterpret_cast<uint4*>(act + row * inter + ch * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_silu_mul(const uint16_t* h, int64_t rows, int32_t inter, uint16_t* act, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = rows * (inter / 8);
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, stream, h, rows, inter, act);
  return hipGetLastError();
}

}  // namespace mg

namespace mg {

// ---------------------------------------------------------------------------
// K0: router.  Per token: softmax of its E logits in fp32, its top_k experts
// in descending order and their probabilities, optionally divided by their
// sum (applied-ai issue "Column-major fused MoE", fused_moe: fp32 softmax of
// the gating output, topk, renormalize).  One wave per token, VPL logits per
// lane.  The experts are chosen on the logits (softmax is increasing, so the
// order is that of the probabilities), ties to the lower expert index.  The
// max and sum are butterfly reductions, identical in every lane.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int64_t T, int32_t E,
                                                          int32_t k, int32_t renorm, int32_t* __restrict__ ids,
                                                          float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += stride) {
    const float* z = logits + t * E;
    float v[VPL], ex[VPL];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      v[i] = e < E ? z[e] : -INFINITY;
      mx = fmaxf(mx, v[i]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      ex[i] = (lane + 64 * i < E) ? expf(v[i] - mx) : 0.f;
      s += ex[i];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    uint32_t taken = 0;       // bit i: this lane's logit i is chosen
    float chosen = 0.f;       // sum of the chosen probabilities, j ascending
    int my_id = 0;            // lane j keeps the j-th choice
    float my_w = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;    // no candidate
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || v[i] > bv)) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        const bool better = oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
        if (better) {
          bv = ov;
          bi = oi;
        }
      }
      // bi is the same in every lane; its owner marks it and supplies exp
      const int owner = bi & 63, slot = bi >> 6;
      float mine = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i == slot) mine = ex[i];
      if (lane == owner) taken |= 1u << slot;
      const float p = __shfl(mine, owner, 64) / s;
      if (lane == j) {
        my_id = bi;
        my_w = p;
      }
      chosen += p;
    }
    if (renorm) my_w = my_w / chosen;
    if (lane < k) {
      ids[t * k + lane] = my_id;
      wts[t * k + lane] = my_w;
    }
  }
}

hipError_t launch_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renorm, int32_t* ids,
                             float* wts, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int64_t want = (T + 3) / 4;
  const int blocks = (int)(want < 16384 ? want : 16384);
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) hipLaunchKernelGGL(route_topk_kernel<1>, dim3(blocks), dim3(256), 0, stream, logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 2) hipLaunchKernelGGL(route_topk_kernel<2>, dim3(blocks), dim3(256), 0, stream, logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 4) hipLaunchKernelGGL(route_topk_kernel<4>, dim3(blocks), dim3(256), 0, stream, logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 8) hipLaunchKernelGGL(route_topk_kernel<8>, dim3(blocks), dim3(256), 0, stream, logits, T, E, k, renorm, ids, wts);
  else if (vpl <= 16) hipLaunchKernelGGL(route_topk_kernel<16>, dim3(blocks), dim3(256), 0, stream, logits, T, E, k, renorm, ids, wts);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mg
