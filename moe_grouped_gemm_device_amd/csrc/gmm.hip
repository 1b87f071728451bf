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
#include <type_traits>

#include "kernels.h"
#include "worklist.h"

namespace mg {

constexpr int kThreads = 256;   // 4 waves: 2 (M) x 2 (N), 64 x 64 each

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

// Bytes [lo, hi) of a 4-byte word kept, the rest cleared (lo, hi relative
// to the word; any values).
__device__ inline uint32_t byte_range_mask(int64_t lo, int64_t hi) {
  const int l = lo < 0 ? 0 : (lo > 4 ? 4 : (int)lo);
  const int h = hi < 0 ? 0 : (hi > 4 ? 4 : (int)hi);
  if (h <= l) return 0u;
  uint32_t m = l >= 4 ? 0u : (0xFFFFFFFFu << (8 * l));
  if (h < 4) m &= (1u << (8 * h)) - 1u;
  return m;
}

// Keep the bytes of a 16-byte fp8 chunk starting at contraction index c whose
// index lies in [lo, hi); clear the others.
__device__ inline uint4 mask_fp8_chunk(uint4 x, int64_t c, int64_t lo, int64_t hi) {
  x.x &= byte_range_mask(lo - c, hi - c);
  x.y &= byte_range_mask(lo - c - 4, hi - c - 4);
  x.z &= byte_range_mask(lo - c - 8, hi - c - 8);
  x.w &= byte_range_mask(lo - c - 12, hi - c - 12);
  return x;
}

// ---------------------------------------------------------------------------
// Operand tiles are fetched with raw buffer loads.  For every work item and
// operand the workgroup builds a buffer resource in SGPRs whose base is the
// tile origin at the current k-step and whose size ends where the operand's
// valid contraction range ends, so rows past a group's end (or past K) read
// as zeros with no per-load arithmetic.  Each thread keeps one 32-bit offset
// per 16-byte chunk for the whole item; a chunk outside the tile's valid rows
// gets an offset past any buffer size.  Advancing a k-step only moves the
// scalar base.
// ---------------------------------------------------------------------------
constexpr uint32_t kOOB = 0x80000000u;       // offset no buffer below 2 GiB reaches
constexpr int kBufFlags = 0x00020000;        // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, int64_t bytes) {
  const int32_t nr = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, nr, kBufFlags);
}

// Cache policy of a load: operands that are read exactly once (the weights
// of the forward and dX products) are loaded non-temporal, which lets a CU
// keep far more reads in flight than cached loads do (measured: ~7.0 vs
// ~4.8 TB/s for a pure stream on MI355X); operands reused by other tiles keep
// the default policy so they stay in L2.
constexpr int kPolicyCached = 0;
constexpr int kPolicyStream = 2;   // nt

// Build-time knobs (defaults are the measured best on MI355X):
//   MG_GEMM_NPF        k-steps of loads in flight per workgroup (even)
//   MG_GEMM_POL_REUSED cache policy of the operand that other tiles re-read
#ifndef MG_GEMM_NPF
#define MG_GEMM_NPF 6
#endif
#ifndef MG_GEMM_POL_REUSED
#define MG_GEMM_POL_REUSED kPolicyCached
#endif

template <int POL>
__device__ inline uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, POL);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// 16-byte store that does not keep the line in cache (outputs are written once).
__device__ inline void store16_nt(void* p, const uint4& v) {
  i32x4 x;
  x[0] = (int)v.x;
  x[1] = (int)v.y;
  x[2] = (int)v.z;
  x[3] = (int)v.w;
  __builtin_nontemporal_store(x, reinterpret_cast<i32x4*>(p));
}

// Contraction-contiguous operand: tile of R rows x BK contraction elements,
// element (i, c) at base + (i * ld + c) * ESZ.  Thread chunk q: row q >> 3,
// 16-byte chunk q & 7 of the row.
template <int R, int ELEM, int POL>
struct KcTile {
  using T = ElemTraits<ELEM>;
  static constexpr int N = R * 8 / kThreads;   // chunks per thread
  static constexpr int LOADS = N;
  static_assert(N >= 1, "tile too small");
  uint32_t voff[N];

  __device__ inline void setup(int64_t ld, int rows_valid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      voff[i] = row < rows_valid ? (uint32_t)(row * ld * T::ESZ + ch * 16) : kOOB;
    }
  }
  __device__ inline void load(uint4* dst, __amdgpu_buffer_rsrc_t r) const {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = bload<POL>(r, voff[i]);
  }
  // Loads of one k-step starting at contraction index c0, keeping only
  // chunks that meet [c_lo, c_hi): lo = c_lo - c0 and hi = c_hi - c0 are
  // workgroup-uniform, so the test is two compares against scalars.  (fp8 dW
  // chunks that straddle a bound are trimmed to their bytes inside it when
  // they are written to LDS, see store_masked, so no load has to complete
  // early.)
  template <bool BYTES>
  __device__ inline void load_range(uint4* dst, __amdgpu_buffer_rsrc_t r, int lo, int hi) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = ((threadIdx.x + i * kThreads) & 7) * T::EPC;
      const bool ok = (c + T::EPC > lo) & (c < hi);
      dst[i] = bload<POL>(r, ok ? voff[i] : kOOB);
    }
  }
  __device__ static inline void store(uint8_t* lds, const uint4* src) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<uint4*>(lds + lds_off(row, ch)) = src[i];
    }
  }
  // store() keeping only the bytes whose contraction index (relative to the
  // k-step) lies in [lo, hi).
  __device__ static inline void store_masked(uint8_t* lds, const uint4* src, int lo, int hi) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<uint4*>(lds + lds_off(row, ch)) = mask_fp8_chunk(src[i], ch * T::EPC, lo, hi);
    }
  }
};

// bf16 element j (0..7) of a 16-byte chunk.
template <int J>
__device__ inline uint32_t half_of(const uint4& u) {
  const uint32_t d = (J < 2) ? u.x : (J < 4) ? u.y : (J < 6) ? u.z : u.w;
  return (J & 1) ? (d >> 16) : (d & 0xFFFFu);
}

// Row-contiguous bf16 operand (its contraction index is strided: W in
// [K, N] layout for the forward, X and dY for dW): the tile keeps the
// operand's natural layout in LDS -- 64 contraction rows of R values, R * 2
// bytes per row, 16-byte chunks XOR-swizzled by 4 * (row % 4) -- and the MFMA
// fragments are read with gfx950's transposing LDS load (ds_read_b64_tr_b16),
// see frag_nt.  Loads and LDS writes are plain 16-byte chunks.
template <int R, int POL>
struct NtTile {
  static constexpr int CPR = R / 8;                   // 16-byte chunks per row
  static constexpr int N = 64 * CPR / kThreads;       // chunks per thread
  static constexpr int LOADS = N;
  static_assert(N >= 1 && CPR >= 16, "tile shape");
  uint32_t voff[N];

  __device__ inline void setup(int64_t ld, int rows_valid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q / CPR, ch = q % CPR;
      voff[i] = ch * 8 < rows_valid ? (uint32_t)((row * ld + ch * 8) * 2) : kOOB;
    }
  }
  __device__ inline void load(uint4* dst, __amdgpu_buffer_rsrc_t r) const {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = bload<POL>(r, voff[i]);
  }
  __device__ static inline int lds_addr(int row, int col) {
    return row * (R * 2) + (((col >> 3) ^ (4 * (row & 3))) << 4) + (col & 7) * 2;
  }
  __device__ static inline void store(uint8_t* lds, const uint4* src) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q / CPR, ch = q % CPR;
      *reinterpret_cast<uint4*>(lds + lds_addr(row, ch * 8)) = src[i];
    }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA bf16 fragment (lane l: operand row l % 32 of the 32-block at mn0, the
// 8 contraction values 16 * ks + 8 * (l / 32) + 0..7) from an NtTile in LDS.
// Within each 16-lane group, lane s points at row k0 + s / 4, columns
// c0 + 4 * (s % 4) .. +3; the transposing load hands lane t the four rows
// k0..k0+3 of column c0 + t.  Two loads (rows k0 and k0 + 4) make the 8
// values.
template <int R>
__device__ inline bf16x8 frag_nt(const uint8_t* tile, int ks, int mn0, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int k0 = ks * 16 + 8 * (G >> 1) + (sl >> 2);
  const int col = mn0 + 16 * (G & 1) + 4 * (sl & 3);
  const int a0 = NtTile<R, 0>::lds_addr(k0, col);
  const int a1 = a0 + 4 * R * 2;   // row k0 + 4: same swizzle
  auto p = (__attribute__((address_space(3))) uint8_t*)tile;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + a0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + a1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int R, int ELEM, bool KC, int POL> struct TileSel;
template <int R, int ELEM, int POL> struct TileSel<R, ELEM, true, POL> { using type = KcTile<R, ELEM, POL>; };
template <int R, int POL> struct TileSel<R, EL_BF16, false, POL> { using type = NtTile<R, POL>; };

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uni64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// One work item: an output tile and its contraction range.
struct Item {
  int g;            // group (expert)
  int64_t rowbase;  // first output row (token row for FIXED_M, row of C_g for DYNAMIC_K)
  int m_valid;      // rows of the tile that exist
  int n0, n_valid;  // first column, columns that exist
  int64_t c_lo, c_hi, c_begin;
  int nsteps;       // K tiles (>= 1; an empty dW group runs one all-zero step)
};

template <int BM, int BN, int KIND, int ELEM, int BK>
__device__ inline Item get_item(const GemmArgs& a, const GroupTable& tab, int64_t w, int n_tiles, int m_tiles_dk) {
  Item it;
  int nt;
  if (KIND == FIXED_M) {
    const int64_t mt = w / n_tiles;
    nt = (int)(w - mt * n_tiles);
    const int4 e = fixed_m_entry(tab, a.E, BM, (int32_t)mt);
    it.g = e.x;
    it.rowbase = e.y;
    it.m_valid = e.z;
    it.c_lo = 0;
    it.c_hi = a.Kc;
    it.c_begin = 0;
  } else {
    const int64_t per = (int64_t)m_tiles_dk * n_tiles;
    const int64_t gi = w / per;
    const int64_t rem = w - gi * per;
    const int mt = (int)(rem / n_tiles);
    nt = (int)(rem - (int64_t)mt * n_tiles);
    it.g = tab.order[gi];
    it.rowbase = (int64_t)mt * BM;
    it.m_valid = a.Mout - (int)it.rowbase;
    it.c_lo = tab.off[it.g];
    it.c_hi = it.c_lo + tab.eff[it.g];
    // fp8 operands are column-major codes read 16 rows at a time from a
    // 16-aligned row; bf16 operands are read one row at a time
    const int64_t start = (ELEM == EL_FP8) ? (it.c_lo & ~(int64_t)15) : it.c_lo;
    it.c_begin = tab.eff[it.g] > 0 ? start : it.c_hi;
  }
  it.n0 = nt * BN;
  it.n_valid = a.Nout - it.n0;
  const int64_t span = it.c_hi - it.c_begin;
  it.nsteps = span > 0 ? (int)cdiv(span, BK) : 1;
  // every field is the same in all lanes (it comes from LDS reads of the
  // group table, which the compiler cannot see are uniform); say so, so the
  // buffer resources built from them live in SGPRs
  it.g = uni(it.g);
  it.rowbase = uni64(it.rowbase);
  it.m_valid = uni(it.m_valid);
  it.n0 = uni(it.n0);
  it.n_valid = uni(it.n_valid);
  it.c_lo = uni64(it.c_lo);
  it.c_hi = uni64(it.c_hi);
  it.c_begin = uni64(it.c_begin);
  it.nsteps = uni(it.nsteps);
  return it;
}

// The K loop of every work item assigned to a workgroup forms one stream of
// (item, k-step) positions.  Global loads run NPF positions ahead of the
// MFMAs in a ring of register slots -- across item boundaries, so a short
// dW contraction or an epilogue never drains the memory pipeline -- and pass
// through two LDS buffers.  One workgroup per CU; the output tile is staged
// in a separate LDS area so the epilogue does not stall the ring.
template <int BM, int BN, bool A_KC, bool B_KC, int KIND, int ELEM, int EPI>
__global__ void __launch_bounds__(kThreads) gmm_kernel(GemmArgs a) {
  using T = ElemTraits<ELEM>;
  constexpr int BK = T::BK;
  constexpr int NPF = MG_GEMM_NPF;    // positions in flight (even)
  constexpr int WM = BM / 2, WN = BN / 2;   // wave sub-tile (2 x 2 waves)
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int SROW = BN + 8;   // bf16 elements per staged output row
  static_assert(TI >= 1 && TJ >= 1, "tile too small");
  static_assert(NPF % 2 == 0, "ring length must be even");
  // Output staging: bf16 for plain bf16 GEMMs; fp32 when scales follow, so
  // the only rounding is the final one to bf16.
  using StgT = typename std::conditional<EPI == EPI_NONE, uint16_t, float>::type;
  constexpr int SROWT = (EPI == EPI_NONE) ? SROW : BN + 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
  __shared__ __attribute__((aligned(16))) StgT stg[BM * SROWT];

  // Fixed-M bf16 products read each weight element once: stream B.
  constexpr int POL_B = (KIND == FIXED_M && ELEM == EL_BF16) ? kPolicyStream : kPolicyCached;
  using ATile = typename TileSel<BM, ELEM, A_KC, MG_GEMM_POL_REUSED>::type;
  using BTile = typename TileSel<BN, ELEM, B_KC, POL_B>::type;
  constexpr int LA = ATile::LOADS, LB = BTile::LOADS;
  // K-tail chunks of contraction-contiguous operands need masking (fixed-M:
  // the last k-step when K is not a multiple of BK; fp8 dW: the k-steps at
  // the group's two ends).  Row-contiguous bf16 operands are bounded by the
  // buffer size alone.
  constexpr bool MASK_BYTES = (ELEM == EL_FP8) && (KIND == DYNAMIC_K);

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
  if (first >= items) return;
  const int64_t G = gridDim.x;
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(a.B);

  ATile aad;   // per-thread chunk offsets of the load cursor's item
  BTile bad;
  auto setup = [&](const Item& it) {
    aad.setup(a.a_ld, it.m_valid);
    bad.setup(a.b_ld, it.n_valid);
  };

  // Issue the loads of k-step s of item it into (da, db); (mlo, mhi) get the
  // step's contraction range for the byte trimming of fp8 dW.
  auto load_slot = [&](uint4* da, uint4* db, const Item& it, int s, int& mlo, int& mhi) {
    const int64_t c0 = it.c_begin + (int64_t)s * BK;
    const bool empty = it.c_hi <= it.c_lo;
    __amdgpu_buffer_rsrc_t ra, rb;
    if constexpr (A_KC) {
      const uint8_t* base = Ab + (it.rowbase * a.a_ld + c0) * T::ESZ;
      int64_t ext = 0x7FFFFFFF;
      if (KIND == DYNAMIC_K) ext = empty ? 0 : (int64_t)(it.m_valid - 1) * a.a_ld + (a.total_rows - c0);
      ra = make_rsrc(base, ext);
    } else {
      ra = make_rsrc(Ab + (c0 * a.a_ld + it.rowbase) * 2, (it.c_hi - c0) * a.a_ld * 2);
    }
    if constexpr (B_KC) {
      const uint8_t* base = Bb + ((int64_t)it.g * a.b_gs + (int64_t)it.n0 * a.b_ld + c0) * T::ESZ;
      int64_t ext = 0x7FFFFFFF;
      if (KIND == DYNAMIC_K) ext = empty ? 0 : (int64_t)(it.n_valid - 1) * a.b_ld + (a.total_rows - c0);
      rb = make_rsrc(base, ext);
    } else {
      rb = make_rsrc(Bb + ((int64_t)it.g * a.b_gs + c0 * a.b_ld + it.n0) * 2, (it.c_hi - c0) * a.b_ld * 2);
    }
    // contraction range relative to this k-step, clamped to int
    const int64_t lo64 = it.c_lo - c0, hi64 = it.c_hi - c0;
    const int lo = lo64 < -BK ? -BK : (lo64 > 2 * BK ? 2 * BK : (int)lo64);
    const int hi = hi64 < -BK ? -BK : (hi64 > 2 * BK ? 2 * BK : (int)hi64);
    mlo = lo;
    mhi = hi;
    if constexpr (A_KC) aad.template load_range<MASK_BYTES>(da, ra, lo, hi);
    else aad.load(da, ra);
    if constexpr (B_KC) bad.template load_range<MASK_BYTES>(db, rb, lo, hi);
    else bad.load(db, rb);
  };
  auto store_slot = [&](uint8_t* buf, const uint4* da, const uint4* db, int mlo, int mhi) {
    if constexpr (MASK_BYTES) {
      ATile::store_masked(buf, da, mlo, mhi);
      BTile::store_masked(buf + A_BYTES, db, mlo, mhi);
    } else {
      ATile::store(buf, da);
      BTile::store(buf + A_BYTES, db);
    }
  };

  f32x16 acc[TI][TJ];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  };

  auto compute = [&](const uint8_t* As) {
    const uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < T::KSUB; ++ks) {
      if constexpr (ELEM == EL_BF16) {
        bf16x8 af[TI], bfr[TJ];
        const int ch = 2 * ks + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          if constexpr (A_KC) {
            const int row = wm * WM + i * 32 + (lane & 31);
            af[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(row, ch));
          } else {
            af[i] = frag_nt<BM>(As, ks, wm * WM + i * 32, lane);
          }
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if constexpr (B_KC) {
            const int row = wn * WN + j * 32 + (lane & 31);
            bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(row, ch));
          } else {
            bfr[j] = frag_nt<BN>(Bs, ks, wn * WN + j * 32, lane);
          }
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
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0,
                                                                         127, 0, 127);
      }
    }
  };

  // epilogue: column scale, staging, row scale, bf16 rounding, coalesced store
  auto epilogue = [&](const Item& it) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = wn * WN + j * 32 + (lane & 31);
      float cs = 1.f;
      if constexpr (EPI != EPI_NONE) {
        if (col < it.n_valid) cs = 1.f / a.sb[(int64_t)it.g * a.Nout + it.n0 + col];
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if constexpr (EPI == EPI_NONE) {
            stg[row * SROWT + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
          } else {
            stg[row * SROWT + col] = acc[i][j][v] * cs;
          }
        }
      }
    }
    __syncthreads();
    constexpr int CPR = BN / 8;                 // 16-byte output chunks per row
    constexpr int TOTAL = BM * CPR;
    uint16_t* cbase = reinterpret_cast<uint16_t*>(a.C) + (int64_t)it.g * a.c_gs + it.rowbase * a.c_ld + it.n0;
#pragma unroll
    for (int q0 = 0; q0 < TOTAL; q0 += kThreads) {
      const int q = q0 + tid;
      const int row = q / CPR, ch = q % CPR;
      if (row < it.m_valid && ch * 8 < it.n_valid) {
        uint4 val;
        if constexpr (EPI == EPI_NONE) {
          val = *reinterpret_cast<const uint4*>(stg + row * SROWT + ch * 8);
        } else {
          float rs;
          if constexpr (EPI == EPI_ROW_COL) rs = 1.f / a.sa[it.rowbase + row];
          else rs = 1.f / a.sa[(int64_t)it.g * a.Mout + it.rowbase + row];
          const float4 lo = *reinterpret_cast<const float4*>(stg + row * SROWT + ch * 8);
          const float4 hi = *reinterpret_cast<const float4*>(stg + row * SROWT + ch * 8 + 4);
          val.x = pack_bf16x2(lo.x * rs, lo.y * rs);
          val.y = pack_bf16x2(lo.z * rs, lo.w * rs);
          val.z = pack_bf16x2(hi.x * rs, hi.y * rs);
          val.w = pack_bf16x2(hi.z * rs, hi.w * rs);
        }
        store16_nt(cbase + (int64_t)row * a.c_ld + ch * 8, val);
      }
    }
  };

  uint4 da[NPF][LA];
  uint4 db[NPF][LB];
  int mlo[NPF], mhi[NPF];

  // load cursor (runs NPF positions ahead) and compute cursor
  int64_t lw = first;
  int ls = 0;
  Item li = get_item<BM, BN, KIND, ELEM, BK>(a, tab, lw, n_tiles, m_tiles_dk);
  int64_t cw = first;
  int cs = 0;
  Item ci = li;
  setup(li);
  // Past the end of its stream the load cursor keeps re-reading its last
  // item's final k-step (never consumed), so loads need no branch.
  auto advance_load = [&]() {
    if (lw >= items) return;
    if (ls + 1 < li.nsteps) {
      ++ls;
      return;
    }
    if (lw + G < items) {
      lw += G;
      ls = 0;
      li = get_item<BM, BN, KIND, ELEM, BK>(a, tab, lw, n_tiles, m_tiles_dk);
      setup(li);
    } else {
      lw = items;   // finished: stay on the last k-step
    }
  };
  auto advance_compute = [&]() {
    if (++cs >= ci.nsteps) {
      cs = 0;
      cw += G;
      if (cw < items) ci = get_item<BM, BN, KIND, ELEM, BK>(a, tab, cw, n_tiles, m_tiles_dk);
    }
  };

#pragma unroll
  for (int u = 0; u < NPF; ++u) {
    load_slot(da[u], db[u], li, ls, mlo[u], mhi[u]);
    advance_load();
  }
  zero_acc();
  store_slot(smem, da[0], db[0], mlo[0], mhi[0]);
  __syncthreads();

  for (;;) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      load_slot(da[u], db[u], li, ls, mlo[u], mhi[u]);
      advance_load();
      compute(smem + (u & 1) * STAGE);
      if (cs == ci.nsteps - 1) {
        epilogue(ci);
        zero_acc();
      }
      advance_compute();
      if (cw >= items) return;
      const int nx = (u + 1) % NPF;
      store_slot(smem + ((u + 1) & 1) * STAGE, da[nx], db[nx], mlo[nx], mhi[nx]);
      __syncthreads();
    }
  }
}

// Zero n 16-byte words (dW when there are no token rows at all: every group
// is empty, and the GEMM kernel must not run because its operands may be
// empty allocations).
__global__ void __launch_bounds__(256) zero16_kernel(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t stream) {
  const int64_t n = bytes / 16;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = cdiv(n, 256) < 8192 ? cdiv(n, 256) : 8192;
  hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(p), n);
  return hipGetLastError();
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
  const int64_t slots = (int64_t)device_cu_count();
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
