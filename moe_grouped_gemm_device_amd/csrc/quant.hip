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

__global__ void __launch_bounds__(256) quant_rowwise_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                           int32_t cols, int64_t ld,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = x + row * ld;
  uint8_t* qr = q + row * (int64_t)cols;
  const int nch = cols >> 3;   // 16-byte chunks in the row
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
    if (ch < nch) *reinterpret_cast<uint2*>(qr + ch * 8) = quant_chunk(held[i], s);
  }
  for (int ch = lane + RCH * kWave; ch < nch; ch += kWave)
    *reinterpret_cast<uint2*>(qr + ch * 8) = quant_chunk(*reinterpret_cast<const uint4*>(xr + ch * 8), s);
}

hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int32_t cols, int64_t ld, uint8_t* q,
                                float* s, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rowwise_kernel, dim3((unsigned)cdiv(rows, 4)), dim3(256), 0, stream, x, rows,
                     cols, ld, q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K4: per-group colwise, single or dual.  Grid (column blocks of 64, groups);
// a workgroup owns 64 columns of one group (of tensor a, then of tensor b in
// the same launch).  Rows are walked in 64-row slabs aligned to 64; each
// thread covers 8 columns x 2 rows of a slab.  Pass 1 reduces the column
// amax; pass 2 scales, converts, transposes the 64x64 byte slab in LDS and
// writes each column's 64 rows as 16-byte pieces (byte stores where a piece
// straddles the group's first or last row, since neighbouring groups are
// written by other workgroups).
// ---------------------------------------------------------------------------
constexpr int CW = 64;   // columns per workgroup
constexpr int RS = 64;   // rows per slab

__device__ void colwise_one(const uint16_t* __restrict__ x, int32_t cols, int64_t rows, int64_t r0,
                            int64_t r1, int g, int cb, uint8_t* __restrict__ q, float* __restrict__ sc,
                            uint8_t (*tile)[RS + 16], uint32_t* s_red, float* s_scale) {
  const int tid = threadIdx.x;
  const int cchunk = tid & 7;          // which 8-column chunk
  const int rsub = tid >> 3;           // 0..31: row within half-slab
  const int c0 = cb * CW;
  const int col = c0 + cchunk * 8;
  const bool col_ok = col < cols;
  const int64_t start = r0 & ~(int64_t)(RS - 1);

  // pass 1: column amax over the group's rows
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t base = start; base < r1; base += RS) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t r = base + rsub + 32 * h;
      if (col_ok && r >= r0 && r < r1) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + r * cols + col);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          m[2 * i] = max(m[2 * i], (w[i] & 0x7FFFu) << 16);
          m[2 * i + 1] = max(m[2 * i + 1], (w[i] >> 16 & 0x7FFFu) << 16);
        }
      }
    }
  }
  // reduce over the 32 threads sharing a column chunk: lanes differing in
  // bits 3..5 within a wave by shuffles, then across the 4 waves in LDS
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t v = m[i];
    v = max(v, (uint32_t)__shfl_xor((int)v, 8, kWave));
    v = max(v, (uint32_t)__shfl_xor((int)v, 16, kWave));
    v = max(v, (uint32_t)__shfl_xor((int)v, 32, kWave));
    m[i] = v;
  }
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s_red[wave * CW + lane * 8 + i] = m[i];
  }
  __syncthreads();
  if (tid < CW) {
    const uint32_t a = max(max(s_red[tid], s_red[CW + tid]), max(s_red[2 * CW + tid], s_red[3 * CW + tid]));
    const float s = fp8_scale_from_amax(__uint_as_float(a));
    s_scale[tid] = s;
    if (c0 + tid < cols) sc[(int64_t)g * cols + c0 + tid] = s;
  }
  __syncthreads();
  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = s_scale[cchunk * 8 + i];

  // pass 2: cast, transpose through LDS, column-major store
  for (int64_t base = start; base < r1; base += RS) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = rsub + 32 * h;
      const int64_t r = base + rr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col_ok && r >= r0 && r < r1) v = *reinterpret_cast<const uint4*>(x + r * cols + col);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = clamp448(bf16_to_f32(w[i] & 0xFFFFu) * sv[2 * i]);
        const float hi = clamp448(bf16_to_f32(w[i] >> 16) * sv[2 * i + 1]);
        const uint32_t codes = __builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, 0u, false);
        tile[cchunk * 8 + 2 * i][rr] = (uint8_t)(codes & 0xFF);
        tile[cchunk * 8 + 2 * i + 1][rr] = (uint8_t)(codes >> 8 & 0xFF);
      }
    }
    __syncthreads();
    {
      // 64 columns x 4 pieces of 16 rows
      const int c = tid >> 2, piece = tid & 3;
      const int64_t rp = base + piece * 16;
      if (c0 + c < cols && rp < r1 && rp + 16 > r0) {
        uint8_t* dst = q + (int64_t)(c0 + c) * rows + rp;
        const uint8_t* src = &tile[c][piece * 16];
        const bool whole = rp >= r0 && rp + 16 <= r1 && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0);
        if (whole) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          for (int b = 0; b < 16; ++b) {
            const int64_t r = rp + b;
            if (r >= r0 && r < r1) dst[b] = src[b];
          }
        }
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) quant_colwise_kernel(const uint16_t* __restrict__ a, int32_t cols_a,
                                                           const uint16_t* __restrict__ b, int32_t cols_b,
                                                           const int32_t* __restrict__ sizes, int32_t G,
                                                           int64_t rows, uint8_t* __restrict__ qa,
                                                           float* __restrict__ sa, uint8_t* __restrict__ qb,
                                                           float* __restrict__ sb) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[CW][RS + 16];
  __shared__ uint32_t s_red[4 * CW];
  __shared__ float s_scale[CW];
  __shared__ int64_t s_r[2];
  const int g = blockIdx.y;
  const int cb = blockIdx.x;
  if (threadIdx.x == 0) {
    // group bounds: exclusive prefix of the (clamped) sizes
    int64_t off = 0;
    for (int h = 0; h < g; ++h) off += sizes[h] > 0 ? sizes[h] : 0;
    int64_t end = off + (sizes[g] > 0 ? sizes[g] : 0);
    s_r[0] = off < rows ? off : rows;
    s_r[1] = end < rows ? end : rows;
  }
  __syncthreads();
  const int64_t r0 = s_r[0], r1 = s_r[1];
  if (cb * CW < cols_a)
    colwise_one(a, cols_a, rows, r0, r1, g, cb, qa, sa, tile, s_red, s_scale);
  if (b != nullptr && cb * CW < cols_b) {
    __syncthreads();
    colwise_one(b, cols_b, rows, r0, r1, g, cb, qb, sb, tile, s_red, s_scale);
  }
}

hipError_t launch_quant_colwise(const uint16_t* a, int32_t cols_a, const uint16_t* b, int32_t cols_b,
                                const int32_t* sizes, int32_t G, int64_t rows, uint8_t* qa, float* sa,
                                uint8_t* qb, float* sb, hipStream_t stream) {
  const int32_t cmax = (b != nullptr && cols_b > cols_a) ? cols_b : cols_a;
  dim3 grid((unsigned)cdiv(cmax, CW), (unsigned)G);
  hipLaunchKernelGGL(quant_colwise_kernel, grid, dim3(256), 0, stream, a, cols_a, b, cols_b, sizes, G, rows,
                     qa, sa, qb, sb);
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
