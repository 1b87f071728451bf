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
// All of them are HBM-bound.  The rowwise kernels hold a row in registers
// and the colwise kernel a 1024-row chunk of 64 columns, so each element is
// read from HBM once and written once as a byte.
#include "gemm_dev.h"

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
// K4: per-group colwise, single or dual, in two launches.
//
// Sets and chunks.  A set is (tensor, group, block of 64 columns).  A group
// of at most CW_CHUNK rows is one chunk; a longer group's chunks are its
// intersections with the global CW_CHUNK-row blocks, so that interior chunk
// edges fall on block boundaries (16-byte aligned in the column-major
// output when the row count is a multiple of 16) and only the group's own
// first and last rows can share a 16-byte piece of a column with another
// group.  A group touching more than CW_MAX_CHUNKS blocks gives each chunk
// several consecutive blocks ("runs").  An empty group has one chunk of no
// rows, which writes the scales of amax 0.
//
// Pass 1 walks every chunk.  A workgroup reads the chunk's first run (up to
// 256 rows x 64 columns) into registers, 8 consecutive rows x 8 columns per
// thread (waves whose rows all lie past the run skip their share), and
// folds the column |x| maxima.  A set of one chunk is finished there and
// then: scales from the maxima, cast, transpose through LDS, column-major
// stores in aligned 16-byte pieces, and the bytes of pieces shared with a
// neighbouring group one per lane -- its input is read from HBM once.  A chunk
// of a larger set stores its 64 partial maxima in the workspace instead.
// Pass 2 walks the chunks of the larger sets, most recently read first so
// that the second read meets them in cache: maximum of the set's partials,
// scales (the set's first chunk writes them), cast and stores as above.
// Neither pass waits on another workgroup, and the workspace holds no
// counters.
// ---------------------------------------------------------------------------
constexpr int CW_COLS = 64;                    // columns per set
constexpr int CW_RPT = 8;                      // rows per thread held in registers
constexpr int CW_CHUNK = (256 / 8) * CW_RPT;   // rows per chunk run (256)
constexpr int CW_UNITS = CW_CHUNK / 16;        // 16-byte units per column row of the LDS tile
constexpr int CW_PIECES = CW_UNITS + 1;        // aligned 16-byte pieces a column's run can touch
constexpr int CW_MAX_CHUNKS = 128;             // chunks per set at most

struct ColwiseArgs {
  const uint16_t* x[2];
  int32_t cols[2];
  int32_t ncb[2];     // 64-column blocks per tensor
  uint8_t* q[2];
  float* s[2];
  const int32_t* sizes;
  int32_t G;
  int32_t ntensors;
  int64_t rows;
  int64_t ld;         // bytes from one code row (input column) to the next, >= rows
  int32_t* err;       // sticky error word (invalid group sizes)
  uint32_t* part;     // partial maxima: 64 words per (chunk slot, column block)
  int64_t part_t1;    // word offset of tensor 1's partials
};

ColwiseLayout colwise_layout(int32_t G, int64_t rows, int32_t cols_a, int32_t cols_b) {
  ColwiseLayout L;
  const int64_t ncb = cdiv(cols_a, CW_COLS) + (cols_b > 0 ? cdiv(cols_b, CW_COLS) : 0);
  // chunk slots per column block: a chunk lies in one of the row blocks,
  // consecutive groups share at most one block, and an empty group adds one
  L.slots = cdiv(rows, CW_CHUNK) + 2 * (int64_t)G;
  L.part_off = 256;
  L.total = L.part_off + 4 * L.slots * ncb * CW_COLS;
  L.items = L.slots * ncb;
  return L;
}

// Blocks a group touches, the blocks per chunk (1 unless the group touches
// more than CW_MAX_CHUNKS), and the group's chunk count (1 for a group of
// at most CW_CHUNK rows, wherever it starts).
__device__ inline int32_t cw_blocks_of(int32_t off, int32_t eff) {
  return (off + eff - 1) / CW_CHUNK - off / CW_CHUNK + 1;
}
__device__ inline int32_t cw_runs_per_chunk(int32_t nblk) { return (nblk + CW_MAX_CHUNKS - 1) / CW_MAX_CHUNKS; }
__device__ inline int32_t cw_chunks_of(int32_t off, int32_t eff) {
  if (eff <= CW_CHUNK) return 1;
  const int32_t nblk = cw_blocks_of(off, eff);
  const int32_t f = cw_runs_per_chunk(nblk);
  return (nblk + f - 1) / f;
}

// Chunk tables, from off/eff (build_group_table): tab.tstart[g] = chunks of
// groups before g (every group), big[g] = chunks of the groups before g
// that have more than one; called by all threads.
__device__ inline void cw_chunk_tables(GroupTable& tab, int32_t* big, int32_t G) {
  const int tid = threadIdx.x;
  const int per = (G + kTableThreads - 1) / kTableThreads;
  const int g0 = tid * per;
  int32_t cnt[4];
  int64_t local = 0, local_big = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cnt[i] = 0;
    if (i < per && g0 + i < G) {
      cnt[i] = cw_chunks_of(tab.off[g0 + i], tab.eff[g0 + i]);
      local += cnt[i];
      local_big += cnt[i] > 1 ? cnt[i] : 0;
    }
  }
  const int64_t incl = block_incl_scan64(local, tab.scratch);
  const int64_t incl_big = block_incl_scan64(local_big, tab.scratch + 8);
  int32_t run = (int32_t)(incl - local), run_big = (int32_t)(incl_big - local_big);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < per && g0 + i < G) {
      tab.tstart[g0 + i] = run;
      big[g0 + i] = run_big;
      run += cnt[i];
      run_big += cnt[i] > 1 ? cnt[i] : 0;
    }
  }
  if (tid == (G - 1) / per) {
    tab.tstart[G] = (int32_t)incl;
    big[G] = (int32_t)incl_big;
  }
  __syncthreads();
}

// The last group g with start[g] <= key (start non-decreasing from 0): two
// ballots of one wave, G <= 64 * 64.  Uniform across the wave.
__device__ inline int cw_find_group(const int32_t* start, int G, int32_t key) {
  const int lane = threadIdx.x & (kWave - 1);
  const int S = (G + kWave - 1) / kWave;
  const int g1 = lane * S;
  const uint64_t b1 = __ballot(g1 < G && start[g1] <= key);
  const int base = (63 - __builtin_clzll(b1)) * S;
  const int g2 = base + lane;
  const uint64_t b2 = __ballot(lane < S && g2 < G && start[g2] <= key);
  return base + 63 - __builtin_clzll(b2);
}

// Element k (0..7, compile-time) of a 16-byte chunk of bf16, as fp32.
template <int K>
__device__ inline float bf16_elem(const uint4& v) {
  const uint32_t w = K / 2 == 0 ? v.x : (K / 2 == 1 ? v.y : (K / 2 == 2 ? v.z : v.w));
  return bf16_to_f32(K % 2 == 0 ? (w & 0xFFFFu) : (w >> 16));
}

// Column maxima of 8 columns over a thread's rows (fp32 bits of |x|).
__device__ inline void cw_fold_max(uint32_t (&m)[8], const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[2 * i] = max(m[2 * i], (w[i] & 0x7FFFu) << 16);
    m[2 * i + 1] = max(m[2 * i + 1], (w[i] >> 16 & 0x7FFFu) << 16);
  }
}

// LDS tile of codes: column c's row r at byte c * CW_CHUNK + (((r / 16) ^
// (c / 8 % 8)) * 16) + r % 16.  The unit index is XORed with the column's
// 8-column group, so that the 8 lanes writing one row group's unit of 8
// columns reach 8 different bank groups.
__device__ inline int cw_tile_unit(int cl, int unit) { return cl * CW_CHUNK + ((unit ^ ((cl >> 3) & 7)) << 4); }

// Codes of column K for a thread's 8 rows, four rows per word, as one half
// of a 16-byte unit of the tile.
template <int K>
__device__ inline void cw_cast_col(uint8_t* tile, const uint4 (&v)[CW_RPT], float s, int cc, int rg) {
  static_assert(CW_RPT == 8, "half a 16-byte unit per thread and column");
  uint32_t d[2];
#pragma unroll
  for (int qd = 0; qd < 2; ++qd) {
    const int i = 4 * qd;
    d[qd] = e4m3x4(clamp448(bf16_elem<K>(v[i]) * s), clamp448(bf16_elem<K>(v[i + 1]) * s),
                   clamp448(bf16_elem<K>(v[i + 2]) * s), clamp448(bf16_elem<K>(v[i + 3]) * s));
  }
  *reinterpret_cast<uint2*>(tile + cw_tile_unit(cc * 8 + K, rg >> 1) + (rg & 1) * 8) = make_uint2(d[0], d[1]);
}

// LDS of either pass besides the group tables: the code tile and the
// per-column maxima, scales and piece shifts.
struct CwShared {
  uint8_t tile[CW_COLS * CW_CHUNK];
  uint32_t red[4][CW_COLS];
  float sc[CW_COLS];
  int sh[CW_COLS];
};

// One chunk of one set.  Its run sb covers rows [max(lo, (B0 + sb) *
// CW_CHUNK), min(end, (B0 + sb + 1) * CW_CHUNK)) for a chunk on the block
// grid, and [lo, end) for a one-chunk group (B0 = -1).
struct CwChunk {
  int t, g, cb, j, nch, nsb;
  int32_t slot0;        // chunk slot of the set's first chunk
  int64_t B0, lo, end;  // first block (or -1), the group's first row and end
};

// Work item -> chunk.  key counts the items of tensor t: groups in order,
// then column blocks, then chunks; start[g] counts the chunks of the groups
// before g that the pass walks (all, or those of sets of several chunks).
__device__ inline CwChunk cw_decode(const ColwiseArgs& a, const GroupTable& tab, const int32_t* start, int t,
                                    int64_t key) {
  CwChunk c;
  const int ncb = a.ncb[t];
  c.t = t;
  c.g = cw_find_group(start, a.G, (int32_t)(key / ncb));
  const int32_t c0 = start[c.g];
  c.nch = start[c.g + 1] - c0;
  const int64_t rem = key - (int64_t)c0 * ncb;
  c.cb = (int)(rem / c.nch);
  c.j = (int)(rem - (int64_t)c.cb * c.nch);
  c.slot0 = tab.tstart[c.g];
  const int32_t eff = tab.eff[c.g], off = tab.off[c.g];
  c.lo = off;
  c.end = (int64_t)off + eff;
  c.nsb = 1;
  c.B0 = -1;
  if (eff > CW_CHUNK) {
    const int32_t nblk = cw_blocks_of(off, eff);
    const int32_t f = cw_runs_per_chunk(nblk);
    c.B0 = (int64_t)(off / CW_CHUNK) + (int64_t)c.j * f;
    const int64_t left = (c.end - 1) / CW_CHUNK - c.B0 + 1;
    c.nsb = (int)(f < left ? f : left);
  }
  return c;
}

// The work of both passes on one chunk.  PASS 1: read run 0 and fold the
// maxima; a chunk of a larger set stores its partial maxima and is done.
// PASS 2: the set's maximum from the partials.  Then (a one-chunk set in
// pass 1, every chunk in pass 2): scales, cast and stores of every run.
template <int PASS>
__device__ inline void cw_chunk(const ColwiseArgs& a, const CwChunk& c, CwShared& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid & 7, rg = tid >> 3;   // 8-column group, row group (rows 8 rg .. 8 rg + 7)
  const int t = c.t, cb = c.cb;
  const int ncb = a.ncb[t], cols = a.cols[t];
  const int64_t LD = a.ld;
  const int64_t row_bytes = 2 * (int64_t)cols;
  const uint32_t vo0 = (uint32_t)(rg * CW_RPT * row_bytes) + (uint32_t)(cc * 16);
  constexpr int WAVE_ROWS = CW_CHUNK / 4;   // rows of wave w: [WAVE_ROWS w, WAVE_ROWS (w + 1))
  auto run_first = [&](int sb) -> int64_t {
    if (c.B0 < 0) return c.lo;
    const int64_t b = (c.B0 + sb) * CW_CHUNK;
    return b > c.lo ? b : c.lo;
  };
  auto run_rows = [&](int sb) -> int {
    const int64_t s0 = run_first(sb);
    const int64_t lim = c.B0 < 0 ? c.end : (c.B0 + sb + 1) * CW_CHUNK;
    const int64_t e1 = lim < c.end ? lim : c.end;
    return e1 > s0 ? (int)(e1 - s0) : 0;
  };
  // buffer over a run's rows from the set's first column: rows past the run
  // and columns past the tensor's last read as zeros
  auto run_rsrc = [&](int sb, int nr) {
    return make_rsrc(a.x[t] + run_first(sb) * cols + cb * CW_COLS,
                     (int64_t)nr * row_bytes - 2 * (int64_t)cb * CW_COLS);
  };
  // a run into v (a wave with no rows in the run reads nothing); kept in
  // cache when pass 2 reads it again, streamed otherwise
  uint4 v[CW_RPT];
  auto load_run = [&](int sb, int nr, bool keep) {
    if (WAVE_ROWS * wave >= nr) return;
    const auto r = run_rsrc(sb, nr);
#pragma unroll
    for (int i = 0; i < CW_RPT; ++i) {
      const int vo = (int)(vo0 + (uint32_t)(i * row_bytes));
      const i32x4 w = keep ? __builtin_amdgcn_raw_buffer_load_b128(r, vo, 0, kPolicyCached)
                           : __builtin_amdgcn_raw_buffer_load_b128(r, vo, 0, kPolicyStream);
      v[i] = make_uint4((uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]);
    }
  };
  // the set's partial maxima: chunk jj's 64 words at pbase + jj * ncb * 64
  uint32_t* pbase = a.part + (t ? a.part_t1 : 0) + ((int64_t)c.slot0 * ncb + cb) * CW_COLS;
  const int64_t pstride = (int64_t)ncb * CW_COLS;
  uint32_t cmax = 0;
  int nr = run_rows(0);
  if constexpr (PASS == 1) {
#pragma unroll
    for (int i = 0; i < CW_RPT; ++i) v[i] = make_uint4(0, 0, 0, 0);
    // every run of the chunk through v (only a one-chunk set, which has one
    // run, keeps it for the cast; a wave with no rows in a later run folds
    // the earlier run's rows of the same set again, which leaves the maxima
    // unchanged)
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int sb = 0; sb < c.nsb; ++sb) {
      load_run(sb, sb == 0 ? nr : run_rows(sb), c.nch > 1);
#pragma unroll
      for (int i = 0; i < CW_RPT; ++i) cw_fold_max(m, v[i]);
    }
    // column maxima over the 32 row groups: 8 per wave by shuffles, then the
    // 4 waves through LDS
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m[k] = max(m[k], (uint32_t)__shfl_xor((int)m[k], 8, kWave));
      m[k] = max(m[k], (uint32_t)__shfl_xor((int)m[k], 16, kWave));
      m[k] = max(m[k], (uint32_t)__shfl_xor((int)m[k], 32, kWave));
    }
    if (lane < 8) {
#pragma unroll
      for (int k = 0; k < 8; ++k) L.red[wave][lane * 8 + k] = m[k];
    }
    __syncthreads();
    if (tid < CW_COLS) cmax = max(max(L.red[0][tid], L.red[1][tid]), max(L.red[2][tid], L.red[3][tid]));
    if (c.nch > 1) {
      if (tid < CW_COLS) pbase[c.j * pstride + tid] = cmax;
      return;
    }
  } else {
    // the set's maximum over its chunks' partials: wave w folds chunks w,
    // w + 4, ..., eight loads in flight per lane, then the 4 waves through
    // LDS
    uint32_t pm = 0;
    for (int jb = wave; jb < c.nch; jb += 32) {
      uint32_t pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jj = jb + 4 * u;
        pv[u] = jj < c.nch ? pbase[jj * pstride + lane] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) pm = max(pm, pv[u]);
    }
    L.red[wave][lane] = pm;
    __syncthreads();
    if (tid < CW_COLS) cmax = max(max(L.red[0][tid], L.red[1][tid]), max(L.red[2][tid], L.red[3][tid]));
  }
  if (tid < CW_COLS) {
    const float s = fp8_scale_from_amax(__uint_as_float(cmax));
    L.sc[tid] = s;
    const int col = cb * CW_COLS + tid;
    if (c.j == 0 && col < cols) a.s[t][(int64_t)c.g * cols + col] = s;
  }
  // ---- cast and store, run by run
  for (int sb = 0; sb < c.nsb; ++sb) {
    const int64_t s0 = run_first(sb);
    if (PASS == 2 || sb > 0) {
      nr = run_rows(sb);
      load_run(sb, nr, false);
    }
    if (tid < CW_COLS) {
      // byte offset of the column's first row of this run within its 16-byte
      // piece
      const int64_t col = cb * CW_COLS + tid;
      L.sh[tid] = (int)((reinterpret_cast<uintptr_t>(a.q[t]) + (uint64_t)(col * LD + s0)) & 15u);
    }
    __syncthreads();   // sc and sh visible; the tile's previous contents consumed
    if (WAVE_ROWS * wave < nr) {
      float sv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) sv[k] = L.sc[cc * 8 + k];
      cw_cast_col<0>(L.tile, v, sv[0], cc, rg);
      cw_cast_col<1>(L.tile, v, sv[1], cc, rg);
      cw_cast_col<2>(L.tile, v, sv[2], cc, rg);
      cw_cast_col<3>(L.tile, v, sv[3], cc, rg);
      cw_cast_col<4>(L.tile, v, sv[4], cc, rg);
      cw_cast_col<5>(L.tile, v, sv[5], cc, rg);
      cw_cast_col<6>(L.tile, v, sv[6], cc, rg);
      cw_cast_col<7>(L.tile, v, sv[7], cc, rg);
    }
    __syncthreads();
    // Column-major stores.  Column cl's rows [0, nr) start at global byte
    // address A = col * LD + s0 (plus the base), which sits sh bytes into a
    // 16-byte piece; piece p covers rows [16 p - sh, 16 p - sh + 16).  Its
    // bytes come from the tile by a byte funnel shift of aligned words.
    // Pieces the run fills are stored whole here; the others (shared with a
    // neighbouring group, or the run's only piece) byte by byte below.
    bool edges = false;
    for (int qi = tid; qi < CW_COLS * CW_PIECES; qi += 256) {
      const int cl = qi / CW_PIECES, p = qi - cl * CW_PIECES;
      const int col = cb * CW_COLS + cl;
      if (col >= cols) continue;
      const int lo = p * 16 - L.sh[cl], hi = lo + 16;   // rows of this piece
      if (hi <= 0 || lo >= nr) continue;
      if (lo < 0 || hi > nr) {
        edges = true;
        continue;
      }
      uint8_t* dst = a.q[t] + (int64_t)col * LD + s0 + lo;   // 16-byte aligned
      const int d0 = lo >> 2, bs = lo & 3;                   // first word, byte shift
      uint32_t w[5];
#pragma unroll
      for (int jw = 0; jw < 5; ++jw) {
        const int d = d0 + jw < 4 * CW_UNITS ? d0 + jw : 4 * CW_UNITS - 1;
        w[jw] = *reinterpret_cast<const uint32_t*>(L.tile + cw_tile_unit(cl, d >> 2) + (d & 3) * 4);
      }
      uint4 o;
      o.x = __builtin_amdgcn_alignbyte(w[1], w[0], bs);
      o.y = __builtin_amdgcn_alignbyte(w[2], w[1], bs);
      o.z = __builtin_amdgcn_alignbyte(w[3], w[2], bs);
      o.w = __builtin_amdgcn_alignbyte(w[4], w[3], bs);
      *reinterpret_cast<uint4*>(dst) = o;
    }
    // Bytes of the pieces not stored whole, one per lane: a column's run
    // has at most 15 such bytes before its first whole piece (or all nr if
    // it has none) and 15 after its last.
    if (__syncthreads_or(edges)) {
      for (int qi = tid; qi < CW_COLS * 32; qi += 256) {
        const int cl = qi >> 5, e = qi & 31;
        const int col = cb * CW_COLS + cl;
        if (col >= cols) continue;
        const int sh = L.sh[cl];
        const int head = sh == 0 ? 0 : (16 - sh < nr ? 16 - sh : nr);   // rows before the first whole piece
        const int whole = (nr - head) / 16;                              // whole pieces after them
        const int tail = nr - head - 16 * whole;                         // rows after those
        int r;
        if (e < 16) {
          if (e >= head) continue;
          r = e;
        } else {
          if (e - 16 >= tail) continue;
          r = head + 16 * whole + (e - 16);
        }
        a.q[t][(int64_t)col * LD + s0 + r] = L.tile[cw_tile_unit(cl, r >> 4) + (r & 15)];
      }
    }
    __syncthreads();   // the tile and sh are free again
  }
}

__host__ __device__ inline int64_t cw_bytes_dyn(int G) { return table_lds_bytes(G) + 4 * (G + 1); }

// Both passes: group tables, then a grid-stride walk over the pass's
// chunks (pass 2 from the last).
template <int PASS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5, 5))) colwise_kernel(ColwiseArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  __shared__ __attribute__((aligned(16))) CwShared L;
  const GroupTable tab = carve_table(table_lds, a.G);
  int32_t* big = reinterpret_cast<int32_t*>(table_lds + table_lds_bytes(a.G));
  GroupTable tabw = tab;
  const int err = build_group_table(a.sizes, a.G, a.rows, CW_CHUNK, false, tabw);
  if (PASS == 1 && err != 0 && blockIdx.x == 0 && threadIdx.x == 0) *a.err = err;
  cw_chunk_tables(tabw, big, a.G);
  const int32_t* start = PASS == 1 ? tab.tstart : big;
  const int64_t nchk = start[a.G];
  const int64_t n0 = nchk * a.ncb[0];
  const int64_t n = n0 + (a.ntensors > 1 ? nchk * a.ncb[1] : 0);
  for (int64_t k = blockIdx.x; k < n; k += gridDim.x) {
    const int64_t it = PASS == 1 ? k : n - 1 - k;
    const int t = it >= n0 ? 1 : 0;
    const CwChunk c = cw_decode(a, tab, start, t, t ? it - n0 : it);
    cw_chunk<PASS>(a, c, L);
    __syncthreads();   // LDS free for the next chunk
  }
}

hipError_t launch_quant_colwise(const uint16_t* a, int32_t cols_a, const uint16_t* b, int32_t cols_b,
                                const int32_t* sizes, int32_t G, int64_t rows, int64_t ld, uint8_t* qa, float* sa,
                                uint8_t* qb, float* sb, void* ws, hipStream_t stream) {
  const ColwiseLayout L = colwise_layout(G, rows, cols_a, b != nullptr ? cols_b : 0);
  ColwiseArgs x;
  x.x[0] = a;
  x.cols[0] = cols_a;
  x.ncb[0] = (int32_t)cdiv(cols_a, CW_COLS);
  x.q[0] = qa;
  x.s[0] = sa;
  x.ntensors = b != nullptr ? 2 : 1;
  x.x[1] = b;
  x.cols[1] = b != nullptr ? cols_b : 0;
  x.ncb[1] = b != nullptr ? (int32_t)cdiv(cols_b, CW_COLS) : 0;
  x.q[1] = qb;
  x.s[1] = sb;
  x.sizes = sizes;
  x.G = G;
  x.rows = rows;
  x.ld = ld;
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  x.err = reinterpret_cast<int32_t*>(w);
  x.part = reinterpret_cast<uint32_t*>(w + L.part_off);
  x.part_t1 = L.slots * x.ncb[0] * CW_COLS;
  const size_t dyn = (size_t)cw_bytes_dyn(G);
  // resident workgroups per CU at this group table's size (cached per G)
  static int occ_of[kMaxExperts + 1];
  int occ = occ_of[G];
  if (occ == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, colwise_kernel<1>, 256, dyn) != hipSuccess || occ < 1)
      occ = 1;
    occ_of[G] = occ;
  }
  const int64_t resident = (int64_t)device_cu_count() * occ;
  const int grid = (int)(L.items < resident ? L.items : resident);
  hipLaunchKernelGGL(colwise_kernel<1>, dim3(grid), dim3(256), dyn, stream, x);
  hipLaunchKernelGGL(colwise_kernel<2>, dim3(grid), dim3(256), dyn, stream, x);
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
