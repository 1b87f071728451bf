// FP8 quantizers (K3 rowwise, K4 per-group colwise single/dual) and the int4
// weight quantizer, for gfx950.
//
// Scale recipe (torchao commit "Optimize FP8 MoE backward pass: fused colwise
// kernel + AMD tuning": the three-step rowwise definition in the commit
// message, and the colwise kernel in bench_colwise_block_configs.py):
//   amax = max |x| over the scaled block (exact in bf16),
//   t    = fp32(448 / max(amax, 1e-12)), the division done in fp64,
//   s    = 2^floor(log2 t), taken exactly by clearing t's mantissa bits,
//   code = e4m3(clamp(x * s, -448, 448)) with round-to-nearest-even.
// The format is OCP e4m3fn (largest finite 448): gfx950's fp8 convert and
// MFMA instructions use it, where the page's MI300X runs used e4m3fnuz.
//
// All three kernels are HBM-bound: each element is read twice (amax pass,
// cast pass; the second read mostly hits cache) and written once as a byte.
#include "kernels.h"
#include "worklist.h"

namespace mg {

__device__ inline float fp8_scale_from_amax(float amax) {
  const double clamped = (double)amax > 1e-12 ? (double)amax : 1e-12;
  const float t = (float)(448.0 / clamped);
  return __uint_as_float(__float_as_uint(t) & 0xFF800000u);
}

__device__ inline float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Four fp32 values (already within +-448) -> four e4m3 codes, RNE, packed
// little-endian into one word (v_cvt_pk_fp8_f32).
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return w;
}

// 8 bf16 (one 16-byte chunk) times s -> 8 e4m3 codes (two words).
__device__ inline uint2 quant_chunk(const uint4& x, float s) {
  const float f0 = clamp448(bf16_to_f32(x.x & 0xFFFFu) * s), f1 = clamp448(bf16_to_f32(x.x >> 16) * s);
  const float f2 = clamp448(bf16_to_f32(x.y & 0xFFFFu) * s), f3 = clamp448(bf16_to_f32(x.y >> 16) * s);
  const float f4 = clamp448(bf16_to_f32(x.z & 0xFFFFu) * s), f5 = clamp448(bf16_to_f32(x.z >> 16) * s);
  const float f6 = clamp448(bf16_to_f32(x.w & 0xFFFFu) * s), f7 = clamp448(bf16_to_f32(x.w >> 16) * s);
  return make_uint2(e4m3x4(f0, f1, f2, f3), e4m3x4(f4, f5, f6, f7));
}

// |bf16| max of a chunk, as fp32 bits compared as integers (non-negative
// finite floats order like their bit patterns).
__device__ inline uint32_t chunk_absmax_bits(const uint4& x) {
  uint32_t m = 0;
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (w[i] & 0x7FFFu) << 16;
    const uint32_t hi = (w[i] >> 16 & 0x7FFFu) << 16;
    m = max(m, max(lo, hi));
  }
  return m;
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// K3: rowwise.  One wave per row; a row of up to 64*8*RCH elements stays in
// registers between the two passes (HBM read once); longer rows take a
// second read for the cast pass.
// ---------------------------------------------------------------------------
constexpr int RCH = 8;   // chunks per lane held in registers

// Source row of output row `row`: the row itself, or, with a row list
// (token rows in sorted order), x[src[row] / top_k], where an entry past the
// n_pairs (token, slot) pairs -- the padding sentinel -- stands for a row of
// zeros (nch = 0: nothing is read, amax 0).
__device__ inline const uint16_t* rowwise_source(const uint16_t* x, int64_t row, int64_t ld,
                                                 const int32_t* src, int32_t top_k, int64_t n_pairs,
                                                 int& nch) {
  if (src == nullptr) return x + row * ld;
  const int32_t id = src[row];
  if (id < 0 || id >= n_pairs) {
    nch = 0;
    return x;
  }
  return x + (int64_t)(id / top_k) * ld;
}

__global__ void __launch_bounds__(256) quant_rowwise_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                           int32_t cols, int64_t ld,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scales,
                                                           const int32_t* __restrict__ src, int32_t top_k,
                                                           int64_t n_pairs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  uint8_t* qr = q + row * (int64_t)cols;
  const int ncols = cols >> 3;   // 16-byte chunks in the row
  int nch = ncols;               // of them read from x
  const uint16_t* xr = rowwise_source(x, row, ld, src, top_k, n_pairs, nch);
  uint4 held[RCH];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < RCH; ++i) {
    const int ch = lane + i * kWave;
    held[i] = make_uint4(0, 0, 0, 0);
    if (ch < nch) {
      held[i] = *reinterpret_cast<const uint4*>(xr + ch * 8);
      m = max(m, chunk_absmax_bits(held[i]));
    }
  }
  for (int ch = lane + RCH * kWave; ch < nch; ch += kWave)
    m = max(m, chunk_absmax_bits(*reinterpret_cast<const uint4*>(xr + ch * 8)));
  m = wave_max_u32(m);
  const float s = fp8_scale_from_amax(__uint_as_float(m));
  if (lane == 0) scales[row] = s;
#pragma unroll
  for (int i = 0; i < RCH; ++i) {
    const int ch = lane + i * kWave;
    if (ch < ncols) *reinterpret_cast<uint2*>(qr + ch * 8) = quant_chunk(held[i], s);
  }
  for (int ch = lane + RCH * kWave; ch < ncols; ch += kWave)
    *reinterpret_cast<uint2*>(qr + ch * 8) =
        quant_chunk(ch < nch ? *reinterpret_cast<const uint4*>(xr + ch * 8) : make_uint4(0, 0, 0, 0), s);
}

// Few long rows (the sorted activations of a decode step: about a hundred
// rows of 4096-14336): a wave per row would leave most compute units idle
// and stream each row through one wave, so here a workgroup takes a row,
// held in the registers of its 256 threads.  The amax is a max, so scale
// and codes are the same bits as the wave-per-row kernel's.
constexpr int RCH_WG = 8;              // chunks per thread held in registers
constexpr int64_t kRowwiseWgRows = 1024;
constexpr int32_t kRowwiseWgCols = 2048;

__global__ void __launch_bounds__(256) quant_rowwise_wg_kernel(const uint16_t* __restrict__ x, int32_t cols,
                                                              int64_t ld, uint8_t* __restrict__ q,
                                                              float* __restrict__ scales,
                                                              const int32_t* __restrict__ src, int32_t top_k,
                                                              int64_t n_pairs) {
  __shared__ uint32_t wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  uint8_t* qr = q + row * (int64_t)cols;
  const int ncols = cols >> 3;
  int nch = ncols;
  const uint16_t* xr = rowwise_source(x, row, ld, src, top_k, n_pairs, nch);
  uint4 held[RCH_WG];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < RCH_WG; ++i) {
    const int ch = tid + i * 256;
    held[i] = make_uint4(0, 0, 0, 0);
    if (ch < nch) {
      held[i] = *reinterpret_cast<const uint4*>(xr + ch * 8);
      m = max(m, chunk_absmax_bits(held[i]));
    }
  }
  for (int ch = tid + RCH_WG * 256; ch < nch; ch += 256)
    m = max(m, chunk_absmax_bits(*reinterpret_cast<const uint4*>(xr + ch * 8)));
  m = wave_max_u32(m);
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = fp8_scale_from_amax(__uint_as_float(m));
  if (tid == 0) scales[row] = s;
#pragma unroll
  for (int i = 0; i < RCH_WG; ++i) {
    const int ch = tid + i * 256;
    if (ch < ncols) *reinterpret_cast<uint2*>(qr + ch * 8) = quant_chunk(held[i], s);
  }
  for (int ch = tid + RCH_WG * 256; ch < ncols; ch += 256)
    *reinterpret_cast<uint2*>(qr + ch * 8) =
        quant_chunk(ch < nch ? *reinterpret_cast<const uint4*>(xr + ch * 8) : make_uint4(0, 0, 0, 0), s);
}

hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int32_t cols, int64_t ld, uint8_t* q,
                                float* s, hipStream_t stream, const int32_t* src, int32_t top_k,
                                int64_t n_pairs) {
  if (rows <= 0) return hipSuccess;
  if (rows <= kRowwiseWgRows && cols >= kRowwiseWgCols)
    hipLaunchKernelGGL(quant_rowwise_wg_kernel, dim3((unsigned)rows), dim3(256), 0, stream, x, cols, ld, q, s,
                       src, top_k, n_pairs);
  else
    hipLaunchKernelGGL(quant_rowwise_kernel, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, stream, x, rows,
                       cols, ld, q, s, src, top_k, n_pairs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SiLU*mul followed by rowwise e4m3, in one pass: the second FFN GEMM's e4m3
// operand straight from the first GEMM's [rows, 2I] output (applied-ai issue
// "Column-major fused MoE", fused_moe: act = silu(gate) * up; torchao commit
// "Optimize FP8 MoE backward pass": the rowwise scale+cast as one kernel).
// act is formed exactly as silu_mul_kernel forms it (fp32 from the bf16
// halves, rounded to bf16), and its codes and scale exactly as the rowwise
// quantizer forms them from those bf16 values, so the result is the same
// bits as silu_mul followed by quantize_rowwise_fp8, without the bf16 act
// making a round trip through HBM.  One workgroup per row; a row of up to
// 256 * 8 * SQ_HELD values stays in registers between the amax and the
// cast, longer rows recompute act from h for the cast.  act is written too
// when the caller passes a buffer for it.
// ---------------------------------------------------------------------------
constexpr int SQ_HELD = 8;   // act chunks (8 values each) per thread held in registers

// act chunk ch of row hr (gate at hr, up at hr + inter): 8 bf16 values
__device__ inline uint4 silu_mul_chunk(const uint16_t* hr, int32_t inter, int ch) {
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
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ void __launch_bounds__(256) silu_mul_quant_kernel(const uint16_t* __restrict__ h, int32_t inter,
                                                            uint16_t* __restrict__ act, uint8_t* __restrict__ q,
                                                            float* __restrict__ scales) {
  __shared__ uint32_t wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const uint16_t* hr = h + row * (2 * (int64_t)inter);
  uint8_t* qr = q + row * (int64_t)inter;
  uint16_t* ar = act != nullptr ? act + row * (int64_t)inter : nullptr;
  const int ncols = inter >> 3;
  uint4 held[SQ_HELD];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < SQ_HELD; ++i) {
    const int ch = tid + i * 256;
    held[i] = make_uint4(0, 0, 0, 0);
    if (ch < ncols) {
      held[i] = silu_mul_chunk(hr, inter, ch);
      m = max(m, chunk_absmax_bits(held[i]));
      if (ar != nullptr) *reinterpret_cast<uint4*>(ar + ch * 8) = held[i];
    }
  }
  for (int ch = tid + SQ_HELD * 256; ch < ncols; ch += 256) {
    const uint4 v = silu_mul_chunk(hr, inter, ch);
    m = max(m, chunk_absmax_bits(v));
    if (ar != nullptr) *reinterpret_cast<uint4*>(ar + ch * 8) = v;
  }
  m = wave_max_u32(m);
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = fp8_scale_from_amax(__uint_as_float(m));
  if (tid == 0) scales[row] = s;
#pragma unroll
  for (int i = 0; i < SQ_HELD; ++i) {
    const int ch = tid + i * 256;
    if (ch < ncols) *reinterpret_cast<uint2*>(qr + ch * 8) = quant_chunk(held[i], s);
  }
  for (int ch = tid + SQ_HELD * 256; ch < ncols; ch += 256)
    *reinterpret_cast<uint2*>(qr + ch * 8) = quant_chunk(silu_mul_chunk(hr, inter, ch), s);
}

hipError_t launch_silu_mul_quant(const uint16_t* h, int64_t rows, int32_t inter, uint16_t* act, uint8_t* q,
                                 float* scales, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_quant_kernel, dim3((unsigned)rows), dim3(256), 0, stream, h, inter, act, q, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K4: per-group colwise, single or dual.  The unit of work is a tile of 64
// columns x 256 rows of one group: the device group table cuts every group's
// rows into 256-row chunks, so a large group spreads over many workgroups
// (with Zipf-skewed loads one group can hold a sixth of the rows).  Four
// launches on the stream:
//   1. zero the scale arrays, which hold column amax bits until step 4;
//   2. per tile: column |x| max, folded in with an integer atomic max on the
//      fp32 bits (non-negative floats order like their bit patterns);
//   3. per tile, walked in reverse order so that the second read meets the
//      most recently read rows still in cache: the scale from the finished
//      amax, the cast, a transpose through LDS and column-major 16-byte
//      stores (byte stores only where a run starts or ends inside a 16-byte
//      piece shared with a neighbouring group);
//   4. amax -> scale.
// Codes of rows past the groups are not written.
// ---------------------------------------------------------------------------
constexpr int QC_COLS = 64;    // columns per tile
constexpr int QC_ROWS = 256;   // rows per tile (chunk of a group)

struct ColwiseArgs {
  const uint16_t* x[2];
  int32_t cols[2];
  uint8_t* q[2];
  uint32_t* s[2];    // scale arrays [G][cols], amax bits until the last launch
  const int32_t* sizes;
  int32_t G;
  int32_t ntensors;
  int64_t rows;
};

// Chunks of a group are its intersections with the global 256-row blocks,
// so interior chunk edges fall on 256-row boundaries (16-byte aligned in the
// column-major output when the row count is a multiple of 16) and only a
// group's own first and last rows can share a 16-byte piece with another
// group.  Rewrites tab.tstart with these chunk counts (build_group_table must
// have filled off/eff); called by all threads.
__device__ inline void colwise_chunk_table(GroupTable& tab, int32_t G) {
  const int tid = threadIdx.x;
  const int per = (G + kTableThreads - 1) / kTableThreads;
  const int g0 = tid * per;
  int32_t cnt[4];
  int64_t local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cnt[i] = 0;
    if (i < per && g0 + i < G) {
      const int32_t off = tab.off[g0 + i], eff = tab.eff[g0 + i];
      if (eff > 0) cnt[i] = (int32_t)(((int64_t)off + eff - 1) / QC_ROWS - off / QC_ROWS + 1);
      local += cnt[i];
    }
  }
  const int64_t incl = block_incl_scan64(local, tab.scratch);
  int32_t run = (int32_t)(incl - local);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < per && g0 + i < G) {
      tab.tstart[g0 + i] = run;
      run += cnt[i];
    }
  }
  if (tid == (G - 1) / per) tab.tstart[G] = (int32_t)incl;
  __syncthreads();
}

// Chunk -> {group, first row, rows}.
__device__ inline int4 colwise_chunk(const GroupTable& tab, int32_t G, int32_t chunk) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {   // last group whose first chunk is <= chunk
    const int mid = (lo + hi + 1) >> 1;
    if (tab.tstart[mid] <= chunk) lo = mid; else hi = mid - 1;
  }
  const int64_t off = tab.off[lo], end = off + tab.eff[lo];
  const int64_t b0 = (off / QC_ROWS + (chunk - tab.tstart[lo])) * (int64_t)QC_ROWS;
  const int64_t r0 = b0 > off ? b0 : off;
  const int64_t r1 = b0 + QC_ROWS < end ? b0 + QC_ROWS : end;
  return make_int4(lo, (int)r0, (int)(r1 - r0), 0);
}

// Tile index -> (tensor, chunk, block of W columns); consecutive tiles share
// rows.
template <int W>
__device__ inline void colwise_tile(const ColwiseArgs& a, int64_t nch, int64_t item, int& t, int32_t& chunk,
                                    int& cb) {
  const int64_t cba = cdiv(a.cols[0], W);
  t = 0;
  if (item >= nch * cba) {
    item -= nch * cba;
    t = 1;
  }
  const int64_t cbs = cdiv(a.cols[t], W);
  chunk = (int32_t)(item / cbs);
  cb = (int)(item - (int64_t)chunk * cbs);
}

template <int W>
__device__ inline int64_t colwise_tiles(const ColwiseArgs& a, int64_t nch) {
  int64_t n = nch * cdiv(a.cols[0], W);
  if (a.ntensors > 1) n += nch * cdiv(a.cols[1], W);
  return n;
}

// Workgroups that take part in a persistent loop over n equal items: with
// r = ceil(n / grid) rounds, ceil(n / r) workgroups suffice, and every round
// but the last keeps all of them busy.
__device__ inline int64_t balanced_active(int64_t n) {
  const int64_t G = gridDim.x;
  if (n <= 0) return 0;
  const int64_t rounds = (n + G - 1) / G;
  return (n + rounds - 1) / rounds;
}

constexpr int QA_COLS = 256;   // columns per amax tile: a wave reads two 512-byte row runs per load

__global__ void __launch_bounds__(256) colwise_zero_kernel(ColwiseArgs a) {
  for (int t = 0; t < a.ntensors; ++t) {
    const int64_t n = (int64_t)a.G * a.cols[t];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) a.s[t][i] = 0u;
  }
}

__global__ void __launch_bounds__(256) colwise_amax_kernel(ColwiseArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  __shared__ uint32_t red[4][QA_COLS];
  const GroupTable tab = carve_table(table_lds, a.G);
  GroupTable tabw = tab;
  build_group_table(a.sizes, a.G, a.rows, QC_ROWS, false, tabw);
  colwise_chunk_table(tabw, a.G);
  const int64_t nch = tab.tstart[a.G];
  const int64_t n = colwise_tiles<QA_COLS>(a, nch);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid & 31, rg = tid >> 5;   // 8-column chunk of the tile, row group (rows rg + 8 j)
  // balanced rounds: the fewest workgroups that take the tiles in as many
  // rounds as the grid needs, so no round runs with most of the grid idle
  const int64_t active = balanced_active(n);
  if ((int64_t)blockIdx.x >= active) return;
  for (int64_t item = blockIdx.x; item < n; item += active) {
    int t, cb;
    int32_t chunk;
    colwise_tile<QA_COLS>(a, nch, item, t, chunk, cb);
    const int4 e = colwise_chunk(tab, a.G, chunk);
    const int cols = a.cols[t];
    const int c = cb * QA_COLS + cc * 8;
    const uint16_t* x = a.x[t] + (int64_t)e.y * cols + c;
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < cols) {
      // 32 rows per thread, 8 loads in flight at a time; rows past the chunk
      // re-read its first row
#pragma unroll
      for (int jb = 0; jb < QC_ROWS / 8; jb += 8) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = rg + 8 * (jb + j);
          v[j] = *reinterpret_cast<const uint4*>(x + (int64_t)(r < e.z ? r : 0) * cols);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            m[2 * i] = max(m[2 * i], (w[i] & 0x7FFFu) << 16);
            m[2 * i + 1] = max(m[2 * i + 1], (w[i] >> 16 & 0x7FFFu) << 16);
          }
        }
      }
    }
    // reduce over the 8 row groups: the two of a wave by a shuffle, then the
    // 4 waves through LDS
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = max(m[i], (uint32_t)__shfl_xor((int)m[i], 32, kWave));
    if (lane < 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = m[i];
    }
    __syncthreads();
    {
      const uint32_t v = max(max(red[0][tid], red[1][tid]), max(red[2][tid], red[3][tid]));
      const int col = cb * QA_COLS + tid;
      if (col < cols && v != 0u) atomicMax(a.s[t] + (int64_t)e.x * cols + col, v);
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) colwise_cast_kernel(ColwiseArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  // tile[c][r]: code of row r of column c.  Rows of 276 bytes: the dword
  // writes below (4 rows of one column per lane) hit 64 distinct banks.
  constexpr int TROW = QC_ROWS + 20;
  __shared__ __attribute__((aligned(16))) uint8_t tile[QC_COLS][TROW];
  __shared__ float sc[QC_COLS];
  __shared__ int sh[QC_COLS];
  const GroupTable tab = carve_table(table_lds, a.G);
  GroupTable tabw = tab;
  build_group_table(a.sizes, a.G, a.rows, QC_ROWS, false, tabw);
  colwise_chunk_table(tabw, a.G);
  const int64_t nch = tab.tstart[a.G];
  const int64_t n = colwise_tiles<QC_COLS>(a, nch);
  const int tid = threadIdx.x;
  const int cc = tid & 7, rq = tid >> 3;   // 8-column chunk, row quad within 128 rows
  const int64_t active = balanced_active(n);   // as in the amax pass
  if ((int64_t)blockIdx.x >= active) return;
  for (int64_t item = n - 1 - blockIdx.x; item >= 0; item -= active) {
    int t, cb;
    int32_t chunk;
    colwise_tile<QC_COLS>(a, nch, item, t, chunk, cb);
    const int4 e = colwise_chunk(tab, a.G, chunk);
    const int cols = a.cols[t];
    const int64_t M = a.rows;
    if (tid < QC_COLS) {
      const int col = cb * QC_COLS + tid;
      float v = 0.f;
      if (col < cols) v = fp8_scale_from_amax(__uint_as_float(a.s[t][(int64_t)e.x * cols + col]));
      sc[tid] = v;
      // byte offset of the column's first row within its 16-byte piece
      sh[tid] = (int)((reinterpret_cast<uintptr_t>(a.q[t]) + (uint64_t)((int64_t)col * M + e.y)) & 15u);
    }
    __syncthreads();
    const int c = cb * QC_COLS + cc * 8;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = sc[cc * 8 + i];
    const uint16_t* x = a.x[t] + (int64_t)e.y * cols + c;
    // the whole tile's loads first (rows past the chunk re-read its first row)
    constexpr int HALVES = QC_ROWS / 128;
    uint4 vv[HALVES][4];
#pragma unroll
    for (int h = 0; h < HALVES; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 128 * h + 4 * rq + k;
        vv[h][k] = make_uint4(0, 0, 0, 0);
        if (c < cols) vv[h][k] = *reinterpret_cast<const uint4*>(x + (int64_t)(r < e.z ? r : 0) * cols);
      }
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
      const int r0 = 128 * h + 4 * rq;
      // codes of 4 rows x 8 columns; column i's 4 codes form one dword
      uint32_t col4[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w[4] = {vv[h][k].x, vv[h][k].y, vv[h][k].z, vv[h][k].w};
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float f0 = clamp448(bf16_to_f32(w[i / 2] & 0xFFFFu) * sv[i]);
          const float f1 = clamp448(bf16_to_f32(w[i / 2] >> 16) * sv[i + 1]);
          const uint32_t codes = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0u, false);
          col4[i] |= (codes & 0xFFu) << (8 * k);
          col4[i + 1] |= (codes >> 8 & 0xFFu) << (8 * k);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(&tile[cc * 8 + i][r0]) = col4[i];
    }
    __syncthreads();
    // Column-major stores.  Column cl's rows [0, e.z) start at global byte
    // address A = col * M + row0 (plus the base), which sits s0 bytes into a
    // 16-byte piece; piece p covers rows [16 p - s0, 16 p - s0 + 16).  Its
    // bytes come from the tile by a byte funnel shift of aligned dwords.
    constexpr int PIECES = QC_ROWS / 16 + 1;
    for (int qi = tid; qi < QC_COLS * PIECES; qi += 256) {
      const int cl = qi / PIECES, p = qi - cl * PIECES;
      const int col = cb * QC_COLS + cl;
      if (col >= cols) continue;
      const int s0 = sh[cl];
      const int lo = p * 16 - s0, hi = lo + 16;   // rows of this piece
      if (hi <= 0 || lo >= e.z) continue;
      uint8_t* dst = a.q[t] + (int64_t)col * M + e.y + lo;   // 16-byte aligned
      if (lo >= 0 && hi <= e.z) {
        const int d0 = lo >> 2, sb = lo & 3;   // first dword, byte shift
        const uint32_t* trow = reinterpret_cast<const uint32_t*>(&tile[cl][0]);
        uint32_t w[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) w[j] = trow[d0 + j < TROW / 4 ? d0 + j : TROW / 4 - 1];
        uint4 out;
        out.x = __builtin_amdgcn_alignbyte(w[1], w[0], sb);
        out.y = __builtin_amdgcn_alignbyte(w[2], w[1], sb);
        out.z = __builtin_amdgcn_alignbyte(w[3], w[2], sb);
        out.w = __builtin_amdgcn_alignbyte(w[4], w[3], sb);
        *reinterpret_cast<uint4*>(dst) = out;
      } else {
        for (int b = 0; b < 16; ++b) {
          const int r = lo + b;
          if (r >= 0 && r < e.z) dst[b] = tile[cl][r];
        }
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) colwise_finalize_kernel(ColwiseArgs a) {
  for (int t = 0; t < a.ntensors; ++t) {
    const int64_t n = (int64_t)a.G * a.cols[t];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
      a.s[t][i] = __float_as_uint(fp8_scale_from_amax(__uint_as_float(a.s[t][i])));
  }
}

hipError_t launch_quant_colwise(const uint16_t* a, int32_t cols_a, const uint16_t* b, int32_t cols_b,
                                const int32_t* sizes, int32_t G, int64_t rows, uint8_t* qa, float* sa,
                                uint8_t* qb, float* sb, hipStream_t stream) {
  ColwiseArgs x;
  x.x[0] = a;
  x.cols[0] = cols_a;
  x.q[0] = qa;
  x.s[0] = reinterpret_cast<uint32_t*>(sa);
  x.ntensors = b != nullptr ? 2 : 1;
  x.x[1] = b;
  x.cols[1] = b != nullptr ? cols_b : 0;
  x.q[1] = qb;
  x.s[1] = reinterpret_cast<uint32_t*>(sb);
  x.sizes = sizes;
  x.G = G;
  x.rows = rows;
  const int64_t scale_words = (int64_t)G * (cols_a + x.cols[1]);
  const int small = (int)(cdiv(scale_words, 256) < 1024 ? cdiv(scale_words, 256) : 1024);
  const int grid = device_cu_count() * 8;
  const size_t dyn = (size_t)table_lds_bytes(G);
  hipLaunchKernelGGL(colwise_zero_kernel, dim3(small), dim3(256), 0, stream, x);
  if (rows > 0) {
    hipLaunchKernelGGL(colwise_amax_kernel, dim3(grid), dim3(256), dyn, stream, x);
    hipLaunchKernelGGL(colwise_cast_kernel, dim3(grid), dim3(256), dyn, stream, x);
  }
  hipLaunchKernelGGL(colwise_finalize_kernel, dim3(small), dim3(256), 0, stream, x);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// int4 weight quantizer (FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse
// M": int4 weights).  Symmetric, one bf16 scale per (expert, column,
// 128-long K chunk): s = bf16_rne(amax / 7) from the fp64 quotient,
// q = clamp(rint(w / s), -8, 7) in fp64.  One thread per column n of a
// (expert, chunk) pair.
// ---------------------------------------------------------------------------

// Round a non-negative double to the nearest bf16 (ties to even), directly
// from the double's bits.
__device__ inline uint16_t bf16_rne_from_double(double d) {
  if (!(d > 0.0)) return 0;
  uint64_t u = (uint64_t)__double_as_longlong(d);
  const int e = (int)((u >> 52) & 0x7FF) - 1023;
  if (e < -126) {
    // bf16 subnormal range: quantize to multiples of 2^-133
    const double m = d * 0x1p133;          // exact scaling by a power of two
    const double r = __builtin_rint(m);    // ties to even
    const uint32_t bits = (uint32_t)r;     // <= 128
    return (uint16_t)bits;                 // 2^-133 * bits; 128 -> smallest normal
  }
  // keep 7 fraction bits of 52: round at bit 45
  const uint64_t lsb = (u >> 45) & 1u;
  u += (1ull << 44) - 1 + lsb;
  const int e2 = (int)((u >> 52) & 0x7FF) - 1023;   // may have carried
  const uint32_t frac = (uint32_t)((u >> 45) & 0x7F);
  const uint32_t be = (uint32_t)(e2 + 127);
  return (uint16_t)((be << 7) | frac);
}

__global__ void __launch_bounds__(256) quant_int4_kernel(const uint16_t* __restrict__ w, int32_t K,
                                                        int32_t N, uint8_t* __restrict__ w4,
                                                        uint16_t* __restrict__ sw) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int j = blockIdx.y;       // K chunk
  const int e = blockIdx.z;       // expert
  if (n >= N) return;
  const uint16_t* col = w + ((int64_t)e * K + (int64_t)j * 128) * N + n;
  float amax = 0.f;
  for (int k = 0; k < 128; ++k) amax = fmaxf(amax, fabsf(bf16_to_f32(col[(int64_t)k * N])));
  const uint16_t sb = bf16_rne_from_double((double)amax / 7.0);
  sw[((int64_t)e * (K / 128) + j) * N + n] = sb;
  const double s = (double)bf16_to_f32(sb);
  uint8_t* dst = w4 + ((int64_t)e * N + n) * (K / 2) + (int64_t)j * 64;
  for (int i = 0; i < 64; i += 16) {
    uint32_t words[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t word = 0;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int k = 2 * (i + 4 * wd) + bb;   // 8 nibbles per word
        int qv = 0;
        if (s != 0.0) {
          double t = __builtin_rint((double)bf16_to_f32(col[(int64_t)k * N]) / s);
          t = t > 7.0 ? 7.0 : (t < -8.0 ? -8.0 : t);
          qv = (int)t;
        }
        word |= ((uint32_t)qv & 0xFu) << (4 * bb);
      }
      words[wd] = word;
    }
    *reinterpret_cast<uint4*>(dst + i) = make_uint4(words[0], words[1], words[2], words[3]);
  }
}

hipError_t launch_quant_int4(const uint16_t* w, int32_t E, int32_t K, int32_t N, uint8_t* w4, uint16_t* sw,
                             hipStream_t stream) {
  dim3 grid((unsigned)cdiv(N, 256), (unsigned)(K / 128), (unsigned)E);
  hipLaunchKernelGGL(quant_int4_kernel, grid, dim3(256), 0, stream, w, K, N, w4, sw);
  return hipGetLastError();
}

}  // namespace mg
