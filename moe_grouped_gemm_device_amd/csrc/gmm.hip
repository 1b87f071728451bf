// Persistent MFMA grouped GEMM for gfx950 (K2): bf16 and fp8-e4m3 operands.
//
// One kernel template covers the three products of the grouped GEMM and its
// backward (grouped_gemm PR "Support GPU-resident batch sizes": gmm forward,
// and the gradient of out.sum() -- dX through W transposed, dW as a
// "dynamic-k" problem whose contraction runs over each group's own rows):
//   FIXED_M   : C[r, :] = A[r, :] . B_g        (forward, dX)
//   DYNAMIC_K : C_g    = A_g^T . B_g           (dW; empty group -> zeros)
// The work list comes from the device builder, so only non-empty groups are
// visited (FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse M").
//
// Design (CDNA4): 256 threads = 4 waves in a 2x2 arrangement, each wave owns
// a (BM/2) x (BN/2) sub-tile built from 32x32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4 with unit
// block scales for e4m3).  K tiles are 128 bytes per row (64 bf16 or 128 fp8),
// staged global -> registers -> LDS with double buffering: the next tile's
// global loads are in flight while the current LDS tile feeds the MFMAs.
// Operands whose contraction index is strided (W in [K, N] layout, X^T and
// dY in dW) are transposed in registers (4 x 8 bf16 blocks) on their way to
// LDS so every MFMA fragment is one 16-byte LDS read.  The epilogue applies
// the fp8 scales, rounds to bf16 and goes through LDS so each lane writes
// 16 contiguous bytes.  The grid is persistent (about two workgroups per CU)
// and consecutive work items are placed on the same XCD.
#include "kernels.h"
#include "worklist.h"

namespace mg {

constexpr int kThreads = 256;

template <int ELEM> struct ElemTraits;
template <> struct ElemTraits<EL_BF16> {
  static constexpr int EPC = 8;    // elements per 16-byte chunk
  static constexpr int ESZ = 2;    // bytes per element
  static constexpr int BK = 64;    // contraction elements per tile row (128 B)
  static constexpr int KSUB = 4;   // MFMA k-steps per tile
};
template <> struct ElemTraits<EL_FP8> {
  static constexpr int EPC = 16;
  static constexpr int ESZ = 1;
  static constexpr int BK = 128;
  static constexpr int KSUB = 2;
};

// Zero the bytes of a 16-byte fp8 chunk whose contraction index c + b lies
// outside [lo, hi).
__device__ inline uint4 mask_fp8_chunk(uint4 x, int64_t c, int64_t lo, int64_t hi) {
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t keep = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t cc = c + d * 4 + b;
      if (cc >= lo && cc < hi) keep |= 0xFFu << (8 * b);
    }
    w[d] &= keep;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Tile of R rows x BK contraction elements from an operand whose
// contraction index is contiguous: element (i, c) at base + i * ld + c.
template <int R, int ELEM>
struct KcTile {
  using T = ElemTraits<ELEM>;
  static constexpr int N = R * 8 / kThreads;
  static_assert(N >= 1, "tile too small");
  uint4 v[N];

  __device__ inline void load(const uint8_t* base, int64_t ld, int rows_valid, int64_t c0,
                              int64_t c_lo, int64_t c_hi) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      const int64_t c = c0 + ch * T::EPC;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < rows_valid && c + T::EPC > c_lo && c < c_hi) {
        x = *reinterpret_cast<const uint4*>(base + (row * ld + c) * T::ESZ);
        if (ELEM == EL_FP8 && (c < c_lo || c + T::EPC > c_hi)) x = mask_fp8_chunk(x, c, c_lo, c_hi);
      }
      v[i] = x;
    }
  }
  __device__ inline void store(uint8_t* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<uint4*>(lds + lds_off(row, ch)) = v[i];
    }
  }
};

// bf16 element j (0..7) of a 16-byte chunk.
template <int J>
__device__ inline uint32_t half_of(const uint4& u) {
  const uint32_t d = (J < 2) ? u.x : (J < 4) ? u.y : (J < 6) ? u.z : u.w;
  return (J & 1) ? (d >> 16) : (d & 0xFFFFu);
}

// Tile of R rows x 64 contraction elements (bf16) from an operand whose
// row index is contiguous: element (i, c) at base + c * ld + i.  Each thread
// loads a 4 (contraction) x 8 (rows) block and writes it transposed.
template <int R>
struct McTile {
  static constexpr int RB = R / 8;          // row blocks
  static constexpr int NB = 16 * RB;        // 16 contraction blocks of 4
  static constexpr int PER = (NB + kThreads - 1) / kThreads;
  uint4 v[PER][4];

  __device__ inline void load(const uint16_t* base, int64_t ld, int rows_valid, int64_t c0,
                              int64_t c_lo, int64_t c_hi) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = threadIdx.x + p * kThreads;
      const int rb = q % RB, cb = q / RB;
      const bool rok = (q < NB) && (rb * 8 < rows_valid);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int64_t c = c0 + cb * 4 + ii;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (rok && c >= c_lo && c < c_hi) x = *reinterpret_cast<const uint4*>(base + c * ld + rb * 8);
        v[p][ii] = x;
      }
    }
  }

  template <int J>
  __device__ inline void store_row(uint8_t* lds, int p, int rb, int cb) const {
    const int row = rb * 8 + J;
    const uint32_t d0 = half_of<J>(v[p][0]) | (half_of<J>(v[p][1]) << 16);
    const uint32_t d1 = half_of<J>(v[p][2]) | (half_of<J>(v[p][3]) << 16);
    *reinterpret_cast<uint2*>(lds + lds_off(row, cb >> 1) + (cb & 1) * 8) = make_uint2(d0, d1);
  }

  __device__ inline void store(uint8_t* lds) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = threadIdx.x + p * kThreads;
      if (q < NB) {
        const int rb = q % RB, cb = q / RB;
        store_row<0>(lds, p, rb, cb);
        store_row<1>(lds, p, rb, cb);
        store_row<2>(lds, p, rb, cb);
        store_row<3>(lds, p, rb, cb);
        store_row<4>(lds, p, rb, cb);
        store_row<5>(lds, p, rb, cb);
        store_row<6>(lds, p, rb, cb);
        store_row<7>(lds, p, rb, cb);
      }
    }
  }
};

template <int R, int ELEM, bool KC> struct TileSel;
template <int R, int ELEM> struct TileSel<R, ELEM, true> { using type = KcTile<R, ELEM>; };
template <int R> struct TileSel<R, EL_BF16, false> { using type = McTile<R>; };

template <int BM, int BN, bool A_KC, bool B_KC, int KIND, int ELEM, int EPI>
__global__ void __launch_bounds__(kThreads) gmm_kernel(GemmArgs a) {
  using T = ElemTraits<ELEM>;
  constexpr int BK = T::BK;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int SROW = BN + 8;   // bf16 elements per staged output row
  static_assert(BM * SROW * 2 <= 2 * STAGE, "staging does not fit");
  static_assert(TI >= 1 && TJ >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  using ATile = typename TileSel<BM, ELEM, A_KC>::type;
  using BTile = typename TileSel<BN, ELEM, B_KC>::type;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // prologue: the group table (offsets, tiles, dynamic-K order) in LDS
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  const GroupTable tab = carve_table(table_lds, a.E);
  const int err = build_group_table(a.sizes, a.E, a.total_rows, BM, KIND == DYNAMIC_K, tab);
  if (err != 0 && blockIdx.x == 0 && tid == 0 && a.err != nullptr) *a.err = err;

  const int n_tiles = (int)cdiv(a.Nout, BN);
  const int m_tiles_dk = (KIND == DYNAMIC_K) ? (int)cdiv(a.Mout, BM) : 1;
  const int64_t items = (KIND == FIXED_M) ? (int64_t)tab.tstart[a.E] * n_tiles
                                          : (int64_t)a.E * m_tiles_dk * n_tiles;

  // consecutive work items on one XCD (workgroups are dealt round-robin to
  // the 8 XCDs)
  int64_t first = blockIdx.x;
  if ((gridDim.x & 7) == 0) first = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);

  for (int64_t w = first; w < items; w += gridDim.x) {
    int g, m_valid, nt;
    int64_t rowbase, c_lo, c_hi, c_begin;
    if (KIND == FIXED_M) {
      const int64_t mt = w / n_tiles;
      nt = (int)(w - mt * n_tiles);
      const int4 e = fixed_m_entry(tab, a.E, BM, (int32_t)mt);
      g = e.x;
      rowbase = e.y;
      m_valid = e.z;
      c_lo = 0;
      c_hi = a.Kc;
      c_begin = 0;
    } else {
      const int64_t per = (int64_t)m_tiles_dk * n_tiles;
      const int64_t gi = w / per;
      const int64_t rem = w - gi * per;
      const int mt = (int)(rem / n_tiles);
      nt = (int)(rem - (int64_t)mt * n_tiles);
      g = tab.order[gi];
      rowbase = (int64_t)mt * BM;
      m_valid = a.Mout - (int)rowbase;
      c_lo = tab.off[g];
      c_hi = c_lo + tab.eff[g];
      c_begin = tab.eff[g] > 0 ? (c_lo & ~(int64_t)15) : c_hi;
    }
    const int n0 = nt * BN;
    const int n_valid = a.Nout - n0;

    // operand bases
    const uint8_t* a_base;
    const uint8_t* b_base;
    if (A_KC) {
      a_base = reinterpret_cast<const uint8_t*>(a.A) + rowbase * a.a_ld * T::ESZ;
    } else {
      a_base = reinterpret_cast<const uint8_t*>(a.A) + rowbase * T::ESZ;
    }
    if (B_KC) {
      b_base = reinterpret_cast<const uint8_t*>(a.B) + ((int64_t)g * a.b_gs + (int64_t)n0 * a.b_ld) * T::ESZ;
    } else {
      b_base = reinterpret_cast<const uint8_t*>(a.B) + ((int64_t)g * a.b_gs + n0) * T::ESZ;
    }

    const int nsteps = c_hi > c_begin ? (int)cdiv(c_hi - c_begin, BK) : 0;

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    ATile at;
    BTile bt;
    auto load_step = [&](int s) {
      const int64_t c0 = c_begin + (int64_t)s * BK;
      if constexpr (A_KC) at.load(a_base, a.a_ld, m_valid, c0, c_lo, c_hi);
      else at.load(reinterpret_cast<const uint16_t*>(a_base), a.a_ld, m_valid, c0, c_lo, c_hi);
      if constexpr (B_KC) bt.load(b_base, a.b_ld, n_valid, c0, c_lo, c_hi);
      else bt.load(reinterpret_cast<const uint16_t*>(b_base), a.b_ld, n_valid, c0, c_lo, c_hi);
    };

    if (nsteps > 0) {
      load_step(0);
      at.store(smem);
      bt.store(smem + A_BYTES);
      __syncthreads();
      for (int s = 0; s < nsteps; ++s) {
        const int cur = s & 1;
        if (s + 1 < nsteps) load_step(s + 1);
        const uint8_t* As = smem + cur * STAGE;
        const uint8_t* Bs = As + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < T::KSUB; ++ks) {
          if constexpr (ELEM == EL_BF16) {
            bf16x8 af[TI], bfr[TJ];
            const int ch = 2 * ks + (lane >> 5);
#pragma unroll
            for (int i = 0; i < TI; ++i) {
              const int row = wm * WM + i * 32 + (lane & 31);
              af[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(row, ch));
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
              const int row = wn * WN + j * 32 + (lane & 31);
              bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(row, ch));
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
              for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          } else {
            i32x8 af[TI], bfr[TJ];
            const int ch = 4 * ks + 2 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < TI; ++i) {
              const int row = wm * WM + i * 32 + (lane & 31);
              const i32x4 lo = *reinterpret_cast<const i32x4*>(As + lds_off(row, ch));
              const i32x4 hi = *reinterpret_cast<const i32x4*>(As + lds_off(row, ch + 1));
              af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
              const int row = wn * WN + j * 32 + (lane & 31);
              const i32x4 lo = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, ch));
              const i32x4 hi = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, ch + 1));
              bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
              for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[i], bfr[j], acc[i][j], 0, 0, 0, 127, 0, 127);
          }
        }
        if (s + 1 < nsteps) {
          uint8_t* nxt = smem + (cur ^ 1) * STAGE;
          at.store(nxt);
          bt.store(nxt + A_BYTES);
        }
        __syncthreads();
      }
    }

    // ---- epilogue: scales, bf16 rounding, staged coalesced store ----
    __syncthreads();
    uint16_t* stg = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = wn * WN + j * 32 + (lane & 31);
      float cs = 1.f;
      if constexpr (EPI != EPI_NONE) {
        if (col < n_valid) cs = 1.f / a.sb[(int64_t)g * a.Nout + n0 + col];
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          float x = acc[i][j][v];
          if constexpr (EPI == EPI_ROW_COL) {
            if (row < m_valid) x = x * (1.f / a.sa[rowbase + row]) * cs;
          } else if constexpr (EPI == EPI_GROUP) {
            if (row < m_valid) x = x * (1.f / a.sa[(int64_t)g * a.Mout + rowbase + row]) * cs;
          }
          stg[row * SROW + col] = (uint16_t)f32_to_bf16_rne(x);
        }
      }
    }
    __syncthreads();
    {
      constexpr int CPR = BN / 8;                 // 16-byte chunks per row
      constexpr int TOTAL = BM * CPR;
      uint16_t* cbase = reinterpret_cast<uint16_t*>(a.C) + (int64_t)g * a.c_gs + rowbase * a.c_ld + n0;
#pragma unroll
      for (int q0 = 0; q0 < TOTAL; q0 += kThreads) {
        const int q = q0 + tid;
        const int row = q / CPR, ch = q % CPR;
        if (row < m_valid && ch * 8 < n_valid) {
          const uint4 val = *reinterpret_cast<const uint4*>(stg + row * SROW + ch * 8);
          *reinterpret_cast<uint4*>(cbase + (int64_t)row * a.c_ld + ch * 8) = val;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int pick_bm_fixed(int elem, int64_t total_M, int32_t E, int32_t Nout) {
  (void)elem; (void)total_M; (void)E; (void)Nout;
  return 128;
}

int pick_bn_fixed(int elem, int64_t total_M, int32_t E, int32_t Nout, int bm) {
  (void)elem; (void)total_M; (void)E; (void)Nout; (void)bm;
  return 128;
}

template <int BM, int BN, bool A_KC, bool B_KC, int KIND, int ELEM, int EPI>
static hipError_t launch_one(const GemmArgs& a, int64_t max_items, hipStream_t stream) {
  if (max_items <= 0) return hipSuccess;
  auto kern = gmm_kernel<BM, BN, A_KC, B_KC, KIND, ELEM, EPI>;
  const int dyn = table_lds_bytes(a.E);
  static int configured = 0;   // largest dynamic LDS size already allowed
  if (dyn > configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, table_lds_bytes(kMaxExperts));
    if (e != hipSuccess) return e;
    configured = table_lds_bytes(kMaxExperts);
  }
  const int64_t slots = (int64_t)device_cu_count() * 2;
  const int grid = (int)(max_items < slots ? max_items : slots);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), (size_t)dyn, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmLaunch& L, const GemmArgs& a, hipStream_t stream) {
  if (L.bm != 128 || L.bn != 128) return hipErrorInvalidValue;
  if (L.elem == EL_BF16) {
    if (L.kind == FIXED_M) {
      if (!L.a_kc) return hipErrorInvalidValue;
      if (L.b_kc) return launch_one<128, 128, true, true, FIXED_M, EL_BF16, EPI_NONE>(a, L.max_items, stream);
      return launch_one<128, 128, true, false, FIXED_M, EL_BF16, EPI_NONE>(a, L.max_items, stream);
    }
    if (!L.a_kc && !L.b_kc)
      return launch_one<128, 128, false, false, DYNAMIC_K, EL_BF16, EPI_NONE>(a, L.max_items, stream);
    return hipErrorInvalidValue;
  }
  if (L.elem == EL_FP8) {
    if (!L.a_kc || !L.b_kc) return hipErrorInvalidValue;
    if (L.kind == FIXED_M)
      return launch_one<128, 128, true, true, FIXED_M, EL_FP8, EPI_ROW_COL>(a, L.max_items, stream);
    return launch_one<128, 128, true, true, DYNAMIC_K, EL_FP8, EPI_GROUP>(a, L.max_items, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mg
