// F8I4 grouped GEMM for sparse M (K2, int4 variant), gfx950.
//
// FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse M": fp8 activations
// times int4 weights, launched only over the problems that have rows
// (min(total_M, groups)), so a single routed token among 128 experts costs
// about what one expert costs.  Here the fixed-M work list from the device
// builder (32-row tiles) times 32-column slices of N forms the work items;
// empty experts never appear in it.
//
// The work is bound by streaming the int4 weights, so the kernel reads them
// straight into registers in the layout of v_mfma_scale_f32_32x32x64_f8f6f4
// (lane l: output column l % 32, a run of 32 consecutive k), turns each
// nibble into the e4m3 code of the same integer (exact: -8..7 are e4m3
// values) with two byte permutes, and runs the fp8 MFMA per 128-long K chunk
// into a fresh accumulator that is then scaled by that chunk's bf16 weight
// scale (keeping the dequantization exact) and added to the running sum.
// The four waves of a workgroup split K; their partial tiles are summed in
// LDS, divided by the row scale of the activations and rounded to bf16.
#include "kernels.h"
#include "worklist.h"

namespace mg {

// e4m3 codes of the integers 0..7 and of -8..-1 (by nibble & 7).
constexpr uint32_t kPosLo = 0x44403800u;   // 0, 1, 2, 3  -> 00 38 40 44
constexpr uint32_t kPosHi = 0x4E4C4A48u;   // 4, 5, 6, 7  -> 48 4A 4C 4E
constexpr uint32_t kNegLo = 0xCACCCED0u;   // -8,-7,-6,-5 -> D0 CE CC CA
constexpr uint32_t kNegHi = 0xB8C0C4C8u;   // -4,-3,-2,-1 -> C8 C4 C0 B8

// Four nibbles (in the low 16 bits of v) -> four e4m3 codes.
__device__ inline uint32_t nib4_to_e4m3(uint32_t v) {
  // spread nibbles into bytes: byte i = nibble i
  const uint32_t sel = (v & 0xFu) | ((v >> 4 & 0xFu) << 8) | ((v >> 8 & 0xFu) << 16) | ((v >> 12 & 0xFu) << 24);
  const uint32_t idx = sel & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(kPosHi, kPosLo, idx);
  const uint32_t neg = __builtin_amdgcn_perm(kNegHi, kNegLo, idx);
  const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xFFu;
  return (pos & ~m) | (neg & m);
}

// 16 bytes = 32 nibbles (k ascending, low nibble first) -> 32 e4m3 codes.
__device__ inline i32x8 i4x32_to_e4m3(const uint4& w) {
  i32x8 r;
  r[0] = (int)nib4_to_e4m3(w.x & 0xFFFFu);
  r[1] = (int)nib4_to_e4m3(w.x >> 16);
  r[2] = (int)nib4_to_e4m3(w.y & 0xFFFFu);
  r[3] = (int)nib4_to_e4m3(w.y >> 16);
  r[4] = (int)nib4_to_e4m3(w.z & 0xFFFFu);
  r[5] = (int)nib4_to_e4m3(w.z >> 16);
  r[6] = (int)nib4_to_e4m3(w.w & 0xFFFFu);
  r[7] = (int)nib4_to_e4m3(w.w >> 16);
  return r;
}

constexpr int F_BM = kF8I4RowTile;
constexpr int F_BN = 32;
constexpr int F_UNROLL = 4;   // K chunks whose weights are requested together

__global__ void __launch_bounds__(256) f8i4_kernel(GemmArgs a) {
  __shared__ float red[4][F_BM * F_BN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.Kc;
  const int N = a.Nout;
  const int nchunk = K / 128;
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  const GroupTable tab = carve_table(table_lds, a.E);
  const int err = build_group_table(a.sizes, a.E, a.total_rows, F_BM, false, tab);
  if (err != 0 && blockIdx.x == 0 && tid == 0 && a.err != nullptr) *a.err = err;
  const int n_tiles = (int)cdiv(N, F_BN);
  const int64_t items = (int64_t)tab.tstart[a.E] * n_tiles;
  const uint8_t* xq = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* w4 = reinterpret_cast<const uint8_t*>(a.B);

  // chunk range of this wave
  const int per = (nchunk + 3) / 4;
  const int j0 = wave * per;
  const int j1 = j0 + per < nchunk ? j0 + per : nchunk;

  int64_t first = blockIdx.x;
  if ((gridDim.x & 7) == 0) first = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);

  for (int64_t w = first; w < items; w += gridDim.x) {
    const int64_t mt = w / n_tiles;
    const int nt = (int)(w - mt * n_tiles);
    const int4 e = fixed_m_entry(tab, a.E, F_BM, (int32_t)mt);
    const int g = e.x;
    const int64_t row0 = e.y;
    const int m_valid = e.z;
    const int n0 = nt * F_BN;
    const int col = lane & 31;
    const int half = lane >> 5;
    const bool col_ok = n0 + col < N;
    const bool row_ok = col < m_valid;   // A fragment row = lane % 32
    const uint8_t* wrow = w4 + ((int64_t)g * N + (col_ok ? n0 + col : 0)) * (K / 2);
    const uint8_t* xrow = xq + (row0 + (row_ok ? col : 0)) * (int64_t)K;
    const uint16_t* srow = a.s4 + (int64_t)g * nchunk * N + (col_ok ? n0 + col : 0);

    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;

    for (int jb = j0; jb < j1; jb += F_UNROLL) {
      uint4 wv[F_UNROLL][2];
      float sc[F_UNROLL];
#pragma unroll
      for (int u = 0; u < F_UNROLL; ++u) {
        const int j = jb + u;
        wv[u][0] = wv[u][1] = make_uint4(0, 0, 0, 0);
        sc[u] = 0.f;
        if (j < j1 && col_ok) {
          // k = 128 j + 64 s + 32 half .. +32  ->  bytes (128 j + 64 s + 32 half) / 2
          // weights are read once: non-temporal loads
          const i32x4 w0 = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wrow + j * 64 + half * 16));
          const i32x4 w1 = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(wrow + j * 64 + 32 + half * 16));
          wv[u][0] = make_uint4((uint32_t)w0[0], (uint32_t)w0[1], (uint32_t)w0[2], (uint32_t)w0[3]);
          wv[u][1] = make_uint4((uint32_t)w1[0], (uint32_t)w1[1], (uint32_t)w1[2], (uint32_t)w1[3]);
          sc[u] = bf16_to_f32(srow[(int64_t)j * N]);
        }
      }
#pragma unroll
      for (int u = 0; u < F_UNROLL; ++u) {
        const int j = jb + u;
        if (j < j1) {
          f32x16 part;
#pragma unroll
          for (int v = 0; v < 16; ++v) part[v] = 0.f;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int kk = j * 128 + s * 64 + half * 32;
            i32x8 af;
            if (row_ok) {
              const i32x4 lo = *reinterpret_cast<const i32x4*>(xrow + kk);
              const i32x4 hi = *reinterpret_cast<const i32x4*>(xrow + kk + 16);
              af = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q) af[q] = 0;
            }
            const i32x8 bf = i4x32_to_e4m3(wv[u][s]);
            part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, part, 0, 0, 0, 127, 0, 127);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] += part[v] * sc[u];
        }
      }
    }

    // cross-wave reduction of the four K slices
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * half + (v & 3);
      red[wave][r * F_BN + col] = acc[v];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < (F_BM * F_BN) / 256; ++i) {
      const int idx = tid + i * 256;
      const int r = idx / F_BN, c = idx % F_BN;
      if (r < m_valid && n0 + c < N) {
        const float sum = (red[0][idx] + red[1][idx]) + (red[2][idx] + red[3][idx]);
        const float y = sum * (1.f / a.sa[row0 + r]);
        reinterpret_cast<uint16_t*>(a.C)[(row0 + r) * a.c_ld + n0 + c] = (uint16_t)f32_to_bf16_rne(y);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_f8i4(const GemmArgs& a, int64_t cap_entries, hipStream_t stream) {
  const int64_t max_items = cap_entries * cdiv(a.Nout, F_BN);
  if (max_items <= 0) return hipSuccess;
  const int64_t slots = (int64_t)device_cu_count() * 4;
  const int grid = (int)(max_items < slots ? max_items : slots);
  hipLaunchKernelGGL(f8i4_kernel, dim3(grid), dim3(256), (size_t)table_lds_bytes(a.E), stream, a);
  return hipGetLastError();
}

}  // namespace mg
