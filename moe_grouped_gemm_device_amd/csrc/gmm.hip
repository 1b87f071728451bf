// Persistent MFMA grouped GEMM for gfx950 (K2): bf16 and fp8-e4m3 operands.
//
// One kernel template covers the three products of the grouped GEMM and its
// backward (grouped_gemm PR "Support GPU-resident batch sizes": gmm forward,
// and the gradient of out.sum() -- dX through W transposed, dW as a
// "dynamic-k" problem whose contraction runs over each group's own rows):
//   FIXED_M   : C[r, :] = A[r, :] . B_g        (forward, dX)
//   DYNAMIC_K : C_g    = A_g^T . B_g           (dW; empty group -> zeros)
// The work list comes from the device group table, so only non-empty groups
// are visited (FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse M").
//
// Design (CDNA4):
//  * 512 threads = 8 waves in a 2 (M) x 4 (N) arrangement over a 128 x 256
//    output tile; a wave owns a 64 x 64 block of 32 x 32 MFMA tiles
//    (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4 with
//    unit block scales for e4m3): 64 fp32 accumulators per lane, so every
//    instantiation fits in the 256 VGPRs a wave gets at two waves per SIMD.
//    Eight waves rather than four: a CU's address unit turns LDS-DMA
//    instructions into memory requests at a bounded rate per wave, and with
//    four waves that rate, not HBM, capped the L2-resident operand streams.
//    (A 256 x 256 tile, which would halve operand traffic per flop, does not
//    fit its accumulators beside the rest without spills at either width.)
//  * Operand tiles move global -> LDS by the buffer unit's LDS-DMA path
//    (buffer_load_dwordx4 ... lds, 16 bytes per lane), never through VGPRs.
//    NS k-steps are in flight in LDS.  Synchronisation is explicit: a vmcnt
//    wait sized to the loads issued after the stage being consumed, then
//    s_barrier.
//  * Operands whose contraction index is contiguous (X rows, W as [N, K],
//    fp8 column-major codes) use 128-byte LDS rows with 16-byte chunks
//    XOR-swizzled by row, read by ds_read_b128; operands whose contraction
//    index is strided (W as [K, N], X and dY for bf16 dW) keep their natural
//    layout, chunks swizzled by 4 * (row % 4), and are read with gfx950's
//    transposing LDS load (ds_read_b64_tr_b16).  Each DMA lane fetches the
//    global chunk that belongs at its LDS slot, so the LDS image comes out
//    swizzled.
//  * The MFMAs take their operands swapped (C^T blocks), so a lane holds four
//    consecutive output columns of one row: the epilogue writes 8-byte runs
//    into an LDS staging area (the stage just consumed), a wave's 32 rows at
//    a time, and 16-byte non-temporal buffer stores write whole 128-byte
//    line segments to HBM.
//  * Fixed-M products run whole tiles, one contiguous run of tiles per XCD,
//    and balance the last round or two stream-K style: the (tile, k-step)
//    positions left form one sequence cut into equal ranges, one per
//    workgroup.  A tile split between workgroups is summed in a fixed
//    order: each piece stores its fp32 partial tile in the workspace and
//    bumps the tile's counter; the piece that arrives last adds all pieces in
//    workgroup order, runs the epilogue and resets the counter.  Nobody waits
//    for anybody, so the persistent grid cannot deadlock.  When whole tiles
//    alone keep most of the grid busy, no tile is split (re-reading a split
//    tile's partials costs more than the idle workgroups).
//  * dW work items are whole tiles dealt round-robin, largest groups first;
//    loads run ahead across item boundaries.  When groups are short (a few
//    k-steps per item) dW uses 256 x 256 tiles with two LDS stages: each
//    wave then owns 128 x 64 outputs (128 accumulators), which fits because
//    the dynamic-K kernel carries no stream-K state.
//  * Consecutive logical workgroups sit on one XCD (dispatch deals
//    workgroups round-robin to the 8 XCDs), so neighbouring tiles share L2.
#include "gemm_dev.h"

namespace mg {

constexpr uint32_t kRasterM = 12;  // most row tiles per raster block (fixed-M item order)
constexpr int64_t kDkMinPieceSteps = 8;   // shortest piece of a split dynamic-K contraction (k-steps)

template <int ELEM> struct ElemTraits;
template <> struct ElemTraits<EL_BF16> {
  static constexpr int EPC = 8;    // elements per 16-byte chunk
  static constexpr int ESZ = 2;    // bytes per element
  static constexpr int BK = 64;    // contraction elements per k-step (128 B per row)
  static constexpr int KSUB = 4;   // MFMA k-steps per k-step
};
template <> struct ElemTraits<EL_FP8> {
  static constexpr int EPC = 16;
  static constexpr int ESZ = 1;
  static constexpr int BK = 128;
  static constexpr int KSUB = 2;
};

// ---------------------------------------------------------------------------
// Operand tiles in LDS.
// ---------------------------------------------------------------------------

// Contraction-contiguous operand: R rows x 128 bytes (BK elements); row r at
// r * 128, its 16-byte chunk c at slot swz_chunk(r, c).  Each 1 KB block
// (8 rows) is one DMA instruction of one wave.
template <int R, int ELEM, int POL, int NW>
struct KcTile {
  using T = ElemTraits<ELEM>;
  static constexpr int BYTES = R * 128;
  static constexpr int LPT = BYTES / (1024 * NW);   // DMA instructions per thread per k-step
  static_assert(LPT >= 1, "tile too small");
  uint32_t voff[LPT];

  __device__ static inline int row_of(int wave, int lane, int i) { return 8 * (wave * LPT + i) + (lane >> 3); }
  // the chunk that belongs at slot lane & 7 of its row (the swizzle is an involution)
  __device__ static inline int chunk_of(int wave, int lane, int i) { return swz_chunk(row_of(wave, lane, i), lane & 7); }

  __device__ inline void setup(int wave, int lane, int64_t ld, int rows_valid) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int row = row_of(wave, lane, i);
      voff[i] = row < rows_valid ? (uint32_t)(row * ld * T::ESZ + chunk_of(wave, lane, i) * 16) : kOOB;
    }
  }
  // Paired rows: the first R / 2 rows of the tile are rows 0.. of the
  // operand (from the tile origin), the last R / 2 are rows half_off + R / 2..
  // (the up rows of a fused gate/up weight stored as [2I, K]); a row pair
  // exists when its first-half row is below rows_valid.
  __device__ inline void setup_paired(int wave, int lane, int64_t ld, int rows_valid, int half_off) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int row = row_of(wave, lane, i);
      const int src = row + (row >= R / 2 ? half_off : 0);
      voff[i] = row % (R / 2) < rows_valid ? (uint32_t)(src * ld * T::ESZ + chunk_of(wave, lane, i) * 16) : kOOB;
    }
  }
  // The same with the tile's rows looked up: row r is source row
  // ids[r] / div, or zeros when ids[r] >= limit (the source holds fewer
  // than 2^31 bytes, checked on the host).  The 8 ids of a DMA block are
  // read with scalar loads (their wait is on the scalar counter, so the
  // LDS-DMA transfers in flight are not drained), from addresses clamped to
  // the tile's valid rows, and each lane picks its row's id.
  __device__ inline void setup_gather(int wave, int lane, int64_t ld, int rows_valid, const int32_t* ids, int div,
                                      int limit) {
    typedef const __attribute__((address_space(4))) int32_t* cptr;
    const cptr cids = (cptr)ids;
    const int sel = lane >> 3;   // the lane's row within its 8-row block
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int r0 = 8 * (wave * LPT + i);
      int id = limit;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rq = r0 + q < rows_valid ? r0 + q : rows_valid - 1;
        const int v = cids[rq];
        id = sel == q ? v : id;
      }
      const int row = row_of(wave, lane, i);
      if (row >= rows_valid) id = limit;
      voff[i] = (id >= 0 && id < limit) ? (uint32_t)((id / div) * ld * T::ESZ + chunk_of(wave, lane, i) * 16) : kOOB;
    }
  }
  // Source offset of transfer i of this thread's k-step share; only chunks
  // meeting the contraction range [lo, hi) (relative to the k-step;
  // workgroup-uniform) are fetched.  (edge: the k-step is cut by the range;
  // otherwise every chunk is inside.)  The transfer lands at LDS byte
  // (wave * LPT + i) * 1024 + 16 * lane of the tile.
  __device__ inline uint32_t offset(int i, int wave, int lane, int lo, int hi, bool edge) const {
    uint32_t vo = voff[i];
    if (edge) {
      const int c = chunk_of(wave, lane, i) * T::EPC;
      vo = ((c + T::EPC > lo) & (c < hi)) ? vo : kOOB;
    }
    return vo;
  }
  __device__ inline void issue(int i, const i32x4& r, uint32_t tile, int wave, int lane, int lo, int hi,
                               bool edge, bool nt) const {
    dma_pol<POL>(r, tile + (wave * LPT + i) * 1024, offset(i, wave, lane, lo, hi, edge), nt);
  }
};

// Row-contiguous bf16 operand (contraction index strided): 64 contraction
// rows of R values in their natural layout, R * 2 bytes per row, 16-byte
// chunk c of row r at slot c ^ (4 * (r % 4)); the MFMA fragments are read
// with the transposing LDS load, see frag_nt.
template <int R, int POL, int NW>
struct NtTile {
  static constexpr int BYTES = 64 * R * 2;
  static constexpr int CPR = R / 8;        // chunks per row
  static constexpr int RPB = 64 / CPR;     // rows per 1 KB block
  static constexpr int LPT = BYTES / (1024 * NW);
  static_assert(CPR >= 16 && CPR <= 64 && LPT >= 1, "tile shape");
  uint32_t voff[LPT];

  __device__ static inline int lds_addr(int row, int col) {
    return row * (R * 2) + (((col >> 3) ^ (4 * (row & 3))) << 4) + (col & 7) * 2;
  }
  __device__ inline void setup(int wave, int lane, int64_t ld, int cols_valid) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int row = (wave * LPT + i) * RPB + lane / CPR;
      const int ch = (lane % CPR) ^ (4 * (row & 3));
      voff[i] = ch * 8 < cols_valid ? (uint32_t)((row * ld + ch * 8) * 2) : kOOB;
    }
  }
  // Paired columns: the first R / 2 columns of the tile are columns 0.. of
  // the operand (from the tile origin), the last R / 2 are columns
  // half_off + R / 2.. (the up block of a fused gate/up weight); a column
  // pair exists when its first-half column is below cols_valid.
  __device__ inline void setup_paired(int wave, int lane, int64_t ld, int cols_valid, int half_off) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int row = (wave * LPT + i) * RPB + lane / CPR;
      const int ch = (lane % CPR) ^ (4 * (row & 3));
      const int hc = ch % (CPR / 2);
      const int col = ch * 8 + (ch >= CPR / 2 ? half_off : 0);
      voff[i] = hc * 8 < cols_valid ? (uint32_t)((row * ld + col) * 2) : kOOB;
    }
  }
  __device__ inline void issue(int i, const i32x4& r, uint32_t tile, int wave, int, int, int, bool, bool nt) const {
    dma_pol<POL>(r, tile + (wave * LPT + i) * 1024, voff[i], nt);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA bf16 fragment (lane l: operand row l % 32 of the 32-block at mn0, the
// 8 contraction values 16 * ks + 8 * (l / 32) + 0..7) from an NtTile.
// Within each 16-lane group, lane s points at row k0 + s / 4, columns
// c0 + 4 * (s % 4) .. +3; the transposing load hands lane t the four rows
// k0..k0+3 of column c0 + t.  Two loads (rows k0 and k0 + 4) make the 8
// values.
template <int R>
__device__ inline bf16x8 frag_nt(const uint8_t* tile, int ks, int mn0, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int k0 = ks * 16 + 8 * (G >> 1) + (sl >> 2);
  const int col = mn0 + 16 * (G & 1) + 4 * (sl & 3);
  const int a0 = NtTile<R, 0, 4>::lds_addr(k0, col);
  const int a1 = a0 + 4 * R * 2;   // row k0 + 4: same swizzle
  auto p = (__attribute__((address_space(3))) uint8_t*)tile;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + a0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + a1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int R, int ELEM, bool KC, int POL, int NW> struct TileSel;
template <int R, int ELEM, int POL, int NW> struct TileSel<R, ELEM, true, POL, NW> { using type = KcTile<R, ELEM, POL, NW>; };
template <int R, int POL, int NW> struct TileSel<R, EL_BF16, false, POL, NW> { using type = NtTile<R, POL, NW>; };

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int BM, int BN, int NS, bool A_KC, bool B_KC, int KIND, int ELEM, int EPI, int NW>
__global__ void __launch_bounds__(NW * 64) gmm_kernel(GemmArgs a) {
  using T = ElemTraits<ELEM>;
  constexpr int BK = T::BK;
  constexpr int kThreads = NW * 64;
  constexpr int WGN = NW / 2;               // waves: 2 along M x NW / 2 along N
  constexpr int WM = BM / 2, WN = BN / WGN; // wave sub-tile
  constexpr int TI = WM / 32, TJ = WN / 32;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int POL_A = kPolicyCached;
  constexpr int POL_B = (KIND == FIXED_M && ELEM == EL_BF16) ? kPolicyStream : kPolicyCached;
  using ATile = typename TileSel<BM, ELEM, A_KC, POL_A, NW>::type;
  using BTile = typename TileSel<BN, ELEM, B_KC, POL_B, NW>::type;
  static_assert(ATile::BYTES == A_BYTES && BTile::BYTES == B_BYTES, "tile bytes");
  constexpr int LPS = ATile::LPT + BTile::LPT;   // DMA instructions per thread per k-step
  // Epilogue staging in the stage just consumed: each wave stages its own
  // WM x WN sub-tile, an ERW x ECW block at a time, in a private region
  // (bf16 rows of ECW + 8 elements), so the waves need no barrier among
  // themselves; then (fp8) the reciprocal row and column scales of the tile.
  // Whole sub-tile rows (ECW = WN) are preferred over whole columns: the
  // stores then write full 128-byte lines.
  // epilogues that apply fp8 scales; EPI_SWIGLU pairs gate and up columns
  constexpr bool SCALED = EPI == EPI_ROW_COL || EPI == EPI_GROUP;
  constexpr bool SWIGLU = EPI == EPI_SWIGLU;
  static_assert(!SWIGLU || (KIND == FIXED_M && ELEM == EL_BF16 && NW == 8 && BN == 256 && BM == 128),
                "the paired gate/up epilogue is built for bf16 fixed-M 128 x 256 tiles with B as [K, N]");
  constexpr int BNE = SWIGLU ? BN / 2 : BN;   // output columns per tile
  constexpr int SC_BYTES = SCALED ? (BM + BN) * 4 : 0;
  constexpr bool FIT_ALL = NW * WM * (WN + 8) * 2 + SC_BYTES <= STAGE;
  constexpr bool FIT_ROWS = NW * 32 * (WN + 8) * 2 + SC_BYTES <= STAGE;
  constexpr int ERW = FIT_ALL ? WM : 32;
  constexpr int ECW = (FIT_ALL || FIT_ROWS) ? WN : (NW * 32 * (WN / 2 + 8) * 2 + SC_BYTES <= STAGE) ? WN / 2 : WN / 4;
  constexpr int SROW = ECW + 8;
  constexpr int WREG = ERW * SROW * 2;           // bytes of one wave's staging region
  constexpr int CPASS = WN / ECW;                // column blocks
  constexpr int PASSES = (WM / ERW) * CPASS;
  constexpr int SPP = ERW * ECW / 8 / kWave;     // 16-byte stores per lane per pass
  constexpr int NST = PASSES * SPP;              // per epilogue
  static_assert(ECW >= 32 && ECW % 32 == 0 && NW * WREG + SC_BYTES <= STAGE, "staging does not fit");
  static_assert(SPP >= 1 && (ERW * ECW / 8) % kWave == 0, "store split");
  static_assert((NS - 2) * LPS + NST <= 63, "vmcnt range");
  // Vector-memory waits count loads and stores on one counter, and a store
  // may retire before older loads.  So no wait relies on stores retiring in
  // order: before an epilogue issues its stores it waits until at most
  // EPI_VM loads are in flight -- the newest NS - 2 stages, which leaves the
  // stage the next k-step reads landed, and (fp8) the tile's scale loads,
  // which only the LPS transfers of its last k-step follow.  The wait at the
  // top of the next k-step may then allow for the NST stores as well.
  constexpr int EPI_VM_STAGES = (NS - 2) * LPS;
  constexpr int EPI_VM = (EPI_VM_STAGES < LPS) ? EPI_VM_STAGES : LPS;
  static_assert(NS >= 2, "at least double buffering");
  static_assert(KIND == DYNAMIC_K || (int64_t)BM * BN * 4 <= kSkPartBytes, "partial tile size");
  // bf16 dynamic-K launches may split long contractions when a partial tile
  // fits a workspace slot (the fp8 dW kernel, with its group-boundary byte
  // masks, has no registers left for the combine)
  constexpr bool DK_SPLIT = KIND == DYNAMIC_K && ELEM == EL_BF16 && (int64_t)BM * BN * 4 <= kSkPartBytes;
  // fp8 dW: chunks straddling a group boundary carry bytes of the next
  // group; they are cleared in the fragments of the boundary k-steps
  constexpr bool MASK_BYTES = (ELEM == EL_FP8) && (KIND == DYNAMIC_K);

  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * STAGE];
  // fp8: the tile's row and column scales, fetched by LDS DMA at the start of
  // its last k-step (a compiler-issued load would make the compiler drain
  // every LDS-DMA transfer in flight before the epilogue could use it)
  __shared__ __attribute__((aligned(16))) float scl[SCALED ? BM + BN : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  // prologue: the group table (offsets, tiles or dynamic-K order) in LDS
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  const GroupTable tab = carve_table(table_lds, a.E);
  const int err = build_group_table(a.sizes, a.E, a.total_rows, BM, KIND == DYNAMIC_K, tab);
  if (err != 0 && blockIdx.x == 0 && tid == 0 && a.err != nullptr) *a.err = err;

  const int n_tiles = (int)cdiv(a.Nout, BNE);
  const int m_tiles_dk = (KIND == DYNAMIC_K) ? (int)cdiv(a.Mout, BM) : 1;
  const int G = gridDim.x;
  // Dynamic-K split plan (grouped_gemm PR review thread: problems sorted by
  // k, descending, so the longest come first): a group whose contraction is
  // longer than a workgroup's share of all k-steps is cut into pieces of at
  // most that share (and of at least kDkMinPieceSteps), so a few very large
  // groups cannot leave the rest of the grid idle.  Each piece stores its
  // fp32 partial tile in the workspace; the last to arrive adds all pieces
  // in piece order (the same bits whatever the arrival order) and writes
  // the tile.  Split tiles are limited by the workspace: one arrival counter
  // each (kSkMaxGrid) and one partial slot per piece (2 kSkMaxGrid).  Every
  // workgroup computes the same plan from the group table.
  __shared__ DkSplit sp;
  if constexpr (DK_SPLIT) {
    auto steps_of = [&](int g) -> int64_t {   // k-steps of group g's contraction
      const int32_t off = tab.off[g], eff = tab.eff[g];
      if (eff <= 0) return 1;
      const int64_t start = (ELEM == EL_FP8) ? ((int64_t)off & ~(int64_t)15) : (int64_t)off;
      return cdiv((int64_t)off + eff - start, BK);
    };
    int64_t mine = 0;
    for (int g = tid; g < a.E; g += kThreads) mine += steps_of(g);
    const int64_t all = block_incl_scan64(mine, tab.scratch);   // the last thread's value is the total
    if (tid == kThreads - 1) tab.scratch[15] = all;
    __syncthreads();
    if (tid == 0) {
      const int per = m_tiles_dk * n_tiles;
      const int64_t total = tab.scratch[15] * per;
      int64_t cap = cdiv(total, G);
      if (cap < kDkMinPieceSteps) cap = kDkMinPieceSteps;
      int ns = 0, slots = 0;
      sp.items_before[0] = 0;
      sp.slot_before[0] = 0;
      while (ns < kDkMaxSplitGroups && ns < a.E) {
        const int64_t st = steps_of(tab.order[ns]);
        int pc = (int)cdiv(st, cap);
        if (pc > st) pc = (int)st;
        if (pc < 2) break;
        if ((ns + 1) * per > kSkMaxGrid) break;            // arrival counters
        if (slots + pc * per > 2 * kSkMaxGrid) break;       // partial slots
        sp.pieces[ns] = pc;
        slots += pc * per;
        sp.items_before[ns + 1] = sp.items_before[ns] + pc * per;
        sp.slot_before[ns + 1] = slots;
        ++ns;
      }
      sp.groups = ns;
    }
  } else {
    if (tid == 0) {
      sp.groups = 0;
      sp.items_before[0] = 0;
    }
  }
  __syncthreads();
  const int64_t items = uni64((KIND == FIXED_M) ? (int64_t)tab.tstart[a.E] * n_tiles
                                                : (int64_t)(a.E - sp.groups) * m_tiles_dk * n_tiles +
                                                      sp.items_before[sp.groups]);
  // logical workgroup index: consecutive indices on one XCD
  int b = blockIdx.x;
  if ((G & 7) == 0) b = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  // Fixed-M schedule: whole tiles first -- workgroups on whole tiles of one
  // XCD run in lockstep, so operand slices they share are fetched once per
  // XCD -- then stream-K over the rest: the L = (items - D) * S (item,
  // k-step) positions of items [D, items) are cut into GS = min(G, L) equal
  // ranges, one per workgroup [p0, p1), so every such range is non-empty and
  // the pieces of a split tile are exactly the workgroups whose ranges meet
  // it.  Splitting a tile costs its last piece a reload of the other pieces'
  // fp32 partial tiles at the end of its range (about as long as 10-15
  // k-steps when the operand streams saturate HBM), so when the last round
  // would still keep at least 5/8 of the grid busy every tile stays whole
  // (D = items); otherwise the last one or two rounds' worth goes to
  // stream-K.  Dynamic-K items are all whole.
  const int S = (KIND == FIXED_M) ? (int)cdiv(a.Kc, BK) : 1;
  const int64_t full = items / G, rem = items - full * G;
  const bool whole = rem == 0 || rem * 8 >= (int64_t)G * 5;
  const int64_t D = (KIND != FIXED_M || whole) ? items : (full >= 2 ? (full - 1) * G : 0);
  const int64_t L = (items - D) * S;
  const int64_t GS = L < G ? L : G;
  // Whole items [0, D) of equal length (fixed-M tiles; dynamic-K tiles when
  // every group has the same size): XCD x owns the contiguous eighth
  // [c0, c1) and its G / 8 workgroups take it round-robin, so each XCD's L2
  // serves one run of consecutive items (for a balanced dW, one expert's X
  // and dY rows per XCD) and a partial last round is spread evenly over the
  // XCDs.  Dynamic-K items of unequal length (groups come largest first) are
  // dealt over the whole grid, longest first, in snake order.  dp_item(k) is
  // the workgroup's k-th whole item, or -1.
  bool equal_items = KIND == FIXED_M;
  if constexpr (KIND == DYNAMIC_K)
    equal_items = uni(sp.groups) == 0 && uni(tab.eff[uni(tab.order[0])]) == uni(tab.eff[uni(tab.order[a.E - 1])]);
  const bool xcd_split = equal_items && (G & 7) == 0;
  const int64_t gx = xcd_split ? (G >> 3) : G;
  const int64_t dj = xcd_split ? (int64_t)(blockIdx.x >> 3) : b;
  const int64_t c0 = xcd_split ? ((int64_t)(blockIdx.x & 7) * D) >> 3 : 0;
  const int64_t c1 = xcd_split ? ((int64_t)((blockIdx.x & 7) + 1) * D) >> 3 : D;
  auto dp_item = [&](int64_t k) -> int64_t {
    // dynamic-K: odd rounds run backwards (snake), so the workgroups that
    // drew the longest items of one round draw the shortest of the next
    const int64_t w = (KIND == DYNAMIC_K && !xcd_split && (k & 1)) ? k * G + (G - 1 - b) : c0 + dj + k * gx;
    return w < c1 ? w : -1;
  };
  auto dp_next = [&](int64_t w) -> int64_t {   // whole item after w (w from dp_item)
    if (KIND == DYNAMIC_K && !xcd_split) {
      const int64_t k = (w >> 32) == 0 ? (int64_t)((uint32_t)w / (uint32_t)G) : w / G;
      return dp_item(k + 1);
    }
    const int64_t nw = w + gx;
    return nw < c1 ? nw : -1;
  };
  const int64_t dp0 = dp_item(0);
  if (dp0 < 0 && b >= GS) return;
  const int64_t p0 = (KIND == FIXED_M && b < GS) ? D * S + (int64_t)b * L / GS : 0;
  const int64_t p1 = (KIND == FIXED_M && b < GS) ? D * S + (int64_t)(b + 1) * L / GS : 0;
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(a.B);
  auto fetch = [&](int64_t w, const Item* prev) {
    return get_item<BM, BNE, KIND, ELEM, BK, DK_SPLIT, kRasterM>(a, tab, w, n_tiles, m_tiles_dk, prev, sp);
  };
  // The workgroup's sequence of (item, first k-step, end k-step); the end of
  // a dynamic-K item comes from the item (-1 here).
  struct Pos {
    int64_t w;
    int s, e;
  };
  auto sk_pos = [&](int64_t w, int64_t from) -> Pos {
    const int64_t e = p1 - w * S;
    return Pos{w, (int)(from - w * S), (int)(e < S ? e : S)};
  };
  auto first_pos = [&]() -> Pos {
    if (dp0 >= 0) return Pos{dp0, 0, KIND == FIXED_M ? S : -1};
    return sk_pos(p0 / S, p0);
  };
  auto next_pos = [&](int64_t w, Pos& out) -> bool {
    if (w < D) {
      const int64_t nw = dp_next(w);
      if (nw >= 0) {
        out = Pos{nw, 0, KIND == FIXED_M ? S : -1};
        return true;
      }
      if (b >= GS) return false;
      out = sk_pos(p0 / S, p0);
      return true;
    }
    if ((w + 1) * S >= p1) return false;
    out = sk_pos(w + 1, (w + 1) * S);
    return true;
  };

  // load cursor (NS - 1 positions ahead of the compute cursor)
  const Pos fp = first_pos();
  int64_t lw = fp.w;
  int ls = fp.s;
  Item li = fetch(lw, nullptr);
  int lend = fp.e < 0 ? li.nsteps : fp.e;
  bool ldone = false;
  ATile at;
  BTile bt;
  // fixed-M products with a contraction-contiguous bf16 A may take their A
  // rows through a gather index (workgroup-uniform choice)
  constexpr bool CAN_GATHER = KIND == FIXED_M && A_KC && ELEM == EL_BF16;
  const bool gather = CAN_GATHER && a.gather != nullptr;
  auto setup = [&](const Item& it) {
    if constexpr (CAN_GATHER) {
      if (gather) at.setup_gather(wave, lane, a.a_ld, it.m_valid, a.gather + it.rowbase, a.gather_div, a.gather_limit);
      else at.setup(wave, lane, a.a_ld, it.m_valid);
    } else {
      at.setup(wave, lane, a.a_ld, it.m_valid);
    }
    if constexpr (SWIGLU) bt.setup_paired(wave, lane, a.b_ld, it.n_valid, a.Nout - BNE);
    else bt.setup(wave, lane, a.b_ld, it.n_valid);
  };
  setup(li);
  // compute cursor
  int64_t cw = lw;
  int cs = ls, cend = lend;
  Item ci = li;

  // DMA of the load cursor's k-step into an LDS stage: prepare_loads builds
  // the descriptors, issue_one(q) sends the thread's q-th 16-byte transfer
  // (q < LA: operand A, then B).  The transfers are spread over the MFMA
  // sub-steps of the k-step being computed, so their issue overlaps MFMA
  // execution.  Past the end of the workgroup's positions the loads still
  // issue (all out of range: no traffic), so every k-step has the same
  // number of vector-memory instructions, which the waits count on.
  struct LoadCtx {
    i32x4 ra, rb;
    int lo, hi;
    bool edge, nt;
    uint32_t st;
  };
  auto prepare_loads = [&](uint8_t* st) -> LoadCtx {
    const Item& it = li;
    const int64_t c0 = it.c_begin + (int64_t)ls * BK;
    LoadCtx x;
    if constexpr (A_KC) {
      int64_t ext = 0x7FFFFFFF;
      if (KIND == DYNAMIC_K) ext = it.c_hi <= it.c_lo ? 0 : (int64_t)(it.m_valid - 1) * a.a_ld + (a.total_rows - c0);
      const int64_t arow = gather ? 0 : it.rowbase;   // gathered rows carry their row in the offset
      x.ra = make_rsrc_words(Ab + (arow * a.a_ld + c0) * T::ESZ, ldone ? 0 : ext);
    } else {
      x.ra = make_rsrc_words(Ab + (c0 * a.a_ld + it.rowbase) * 2, ldone ? 0 : (it.c_hi - c0) * a.a_ld * 2);
    }
    if constexpr (B_KC) {
      int64_t ext = 0x7FFFFFFF;
      if (KIND == DYNAMIC_K) ext = it.c_hi <= it.c_lo ? 0 : (int64_t)(it.n_valid - 1) * a.b_ld + (a.total_rows - c0);
      x.rb = make_rsrc_words(Bb + ((int64_t)it.g * a.b_gs + (int64_t)it.n0 * a.b_ld + c0) * T::ESZ, ldone ? 0 : ext);
    } else {
      x.rb = make_rsrc_words(Bb + ((int64_t)it.g * a.b_gs + c0 * a.b_ld + it.n0) * 2, ldone ? 0 : (it.c_hi - c0) * a.b_ld * 2);
    }
    // contraction range relative to this k-step, clamped to int
    const int64_t lo64 = it.c_lo - c0, hi64 = it.c_hi - c0;
    x.lo = lo64 < -BK ? -BK : (lo64 > 2 * BK ? 2 * BK : (int)lo64);
    x.hi = hi64 < -BK ? -BK : (hi64 > 2 * BK ? 2 * BK : (int)hi64);
    x.edge = x.lo > 0 || x.hi < BK;
    x.nt = it.b_stream;
    x.st = lds_address(st);
    return x;
  };
  constexpr int LA = ATile::LPT;
  auto issue_one = [&](const LoadCtx& x, int q) {
    if (q < LA) at.issue(q, x.ra, x.st, wave, lane, x.lo, x.hi, x.edge, false);
    else bt.issue(q - LA, x.rb, x.st + A_BYTES, wave, lane, x.lo, x.hi, x.edge, x.nt);
  };
  // Scale DMAs for the compute cursor's tile (EPI != NONE): BM row scales,
  // then BN column scales, 64 floats per instruction; instruction k goes to
  // wave k % 4.  Rows and columns outside the tile read as 0.
  constexpr int NSC = (BM + BN) / 64;
  auto issue_scales = [&](const Item& it) {
    if constexpr (SCALED) {
      const float* rows = a.sa + ((EPI == EPI_ROW_COL) ? it.rowbase : (int64_t)it.g * a.Mout + it.rowbase);
      const float* cols = a.sb + (int64_t)it.g * a.Nout + it.n0;
      const i32x4 rr = make_rsrc_words(rows, (int64_t)it.m_valid * 4);
      const i32x4 rc = make_rsrc_words(cols, (int64_t)it.n_valid * 4);
      const uint32_t base = lds_address(reinterpret_cast<uint8_t*>(scl));
#pragma unroll
      for (int k = 0; k < (NSC + NW - 1) / NW; ++k) {
        const int ins = wave + NW * k;
        if (ins < NSC) {
          const bool is_row = ins < BM / 64;
          const int first = is_row ? ins * 64 : ins * 64 - BM;
          dma4(is_row ? rr : rc, base + ins * 256, (uint32_t)((first + lane) * 4));
        }
      }
    }
  };

  auto advance_load = [&]() {
    if (ldone) return;
    if (ls + 1 < lend) {
      ++ls;
      return;
    }
    Pos np;
    if (!next_pos(lw, np)) {
      ldone = true;
      return;
    }
    lw = np.w;
    ls = np.s;
    li = fetch(np.w, &li);
    lend = np.e < 0 ? li.nsteps : np.e;
    setup(li);
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

  // acc[i][j] holds the transposed 32 x 32 block: lane l has output row
  // wm * WM + 32 i + l % 32 and columns wn * WN + 32 j + 8 q + 4 (l / 32) + r
  // in element 4 q + r.
  // transfers issued in MFMA sub-step ks: [ks * LPS / KSUB, (ks + 1) * LPS / KSUB)
  // The k-step body, in two instantiations: EDGE (fp8 dW, a k-step cut by
  // the group's contraction range: bytes outside it are cleared in the
  // fragments) and the plain one every other k-step runs, which then carries
  // none of the masking arithmetic.
  auto compute_body = [&](const uint8_t* As, const LoadCtx& lx, auto edge_c, int mlo, int mhi) {
    constexpr bool EDGE = decltype(edge_c)::value;
    const uint8_t* Bs = As + A_BYTES;
    // The fragment addresses below are loop-invariant; hoisted, they would
    // hold 24-48 VGPRs across the K loop and push the kernel into spills.
    // An opaque copy of the lane index makes them cheap per-step arithmetic.
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
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
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int q = ks * LPS / T::KSUB; q < (ks + 1) * LPS / T::KSUB; ++q) issue_one(lx, q);
      } else {
        i32x8 af[TI], bfr[TJ];
        const int ch = 4 * ks + 2 * (lane >> 5);
        const int k0 = 16 * ch;   // contraction index of the fragment's first byte
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int row = wm * WM + i * 32 + (lane & 31);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(As + lds_off(row, ch));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(As + lds_off(row, ch + 1));
          af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          if constexpr (EDGE) af[i] = mask_frag8(af[i], k0, mlo, mhi);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int row = wn * WN + j * 32 + (lane & 31);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, ch));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(Bs + lds_off(row, ch + 1));
          bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          if constexpr (EDGE) bfr[j] = mask_frag8(bfr[j], k0, mlo, mhi);
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0, 0,
                                                                         127, 0, 127);
#pragma unroll
        for (int q = ks * LPS / T::KSUB; q < (ks + 1) * LPS / T::KSUB; ++q) issue_one(lx, q);
      }
    }
  };
  auto compute = [&](const uint8_t* As, const LoadCtx& lx) {
    if constexpr (MASK_BYTES) {
      const int64_t c0 = ci.c_begin + (int64_t)cs * BK;
      const int64_t lo64 = ci.c_lo - c0, hi64 = ci.c_hi - c0;
      const int mlo = lo64 < 0 ? 0 : (lo64 > BK ? BK : (int)lo64);
      const int mhi = hi64 < 0 ? 0 : (hi64 > BK ? BK : (int)hi64);
      if (mlo > 0 || mhi < BK) {
        compute_body(As, lx, BoolConst<true>{}, mlo, mhi);
        return;
      }
    }
    compute_body(As, lx, BoolConst<false>{}, 0, BK);
  };

  // Epilogue into the stage st just consumed: (fp8: scales), bf16 rounding,
  // per-wave staging, 16-byte stores of whole 128-byte row segments.  Issues
  // exactly NST vector-memory stores per lane (lanes outside the tile store
  // out of range).
  auto epilogue = [&](uint8_t* st, const Item& it) {
    if constexpr (SWIGLU) {
      // Waves 0-1 of each row half hold gate columns, waves 2-3 the up
      // columns at the same positions (same lane layout).  Per 32-row block:
      // the gate waves hand their bf16-rounded values to the up waves
      // through LDS (lane-contiguous dwords, conflict-free), the up waves
      // form act = silu(g) * u in fp32 from the bf16 values, round it and
      // stage it for 16-byte stores of whole row segments.  Every wave
      // issues the same NST stores (the gate waves' out of range), so the
      // main loop's vector-memory waits count alike in all waves.
      static_assert(NST == TI * 4 && WGN == 4 && TJ == 2 && WN == 64, "paired epilogue shape");
      // every wave is done reading st, and the next k-step's stage has landed
      wait_vm_sync<EPI_VM_STAGES>();
      uint32_t* xch = reinterpret_cast<uint32_t*>(st);   // [4 gate waves][16 dwords][64 lanes]
      const bool up = wn >= 2;
      const int pair = wm * 2 + (wn & 1);
      uint16_t* stg_up = reinterpret_cast<uint16_t*>(st + 4 * 16 * 64 * 4) + pair * 32 * SROW;
      const __amdgpu_buffer_rsrc_t cr =
          make_rsrc(reinterpret_cast<uint16_t*>(a.C) + it.rowbase * a.c_ld + it.n0, 0x7FFFFFFF);
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if (!up) {
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int d = 0; d < 8; ++d)
              xch[(pair * 16 + j * 8 + d) * 64 + lane] = pack_bf16x2_hw(acc[i][j][2 * d], acc[i][j][2 * d + 1]);
        }
        lds_sync();
        if (up) {
#pragma unroll
          for (int j = 0; j < TJ; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t g01 = xch[(pair * 16 + j * 8 + 2 * q) * 64 + lane];
              const uint32_t g23 = xch[(pair * 16 + j * 8 + 2 * q + 1) * 64 + lane];
              const uint32_t u01 = pack_bf16x2_hw(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
              const uint32_t u23 = pack_bf16x2_hw(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              const float g[4] = {bf16_to_f32(g01 & 0xFFFFu), bf16_to_f32(g01 >> 16), bf16_to_f32(g23 & 0xFFFFu),
                                  bf16_to_f32(g23 >> 16)};
              const float u[4] = {bf16_to_f32(u01 & 0xFFFFu), bf16_to_f32(u01 >> 16), bf16_to_f32(u23 & 0xFFFFu),
                                  bf16_to_f32(u23 >> 16)};
              float v[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = g[r] / (1.f + expf(-g[r])) * u[r];
              uint2 pk;
              pk.x = pack_bf16x2(v[0], v[1]);
              pk.y = pack_bf16x2(v[2], v[3]);
              const int cw = 32 * j + 8 * q + 4 * (lane >> 5);
              *reinterpret_cast<uint2*>(stg_up + (lane & 31) * SROW + cw) = pk;
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int q = lane + k * kWave;
          const int rw = q >> 3, ch = q & 7;
          uint4 v = make_uint4(0, 0, 0, 0);
          uint32_t vo = kOOB;
          if (up) {
            v = *reinterpret_cast<const uint4*>(stg_up + rw * SROW + ch * 8);
            const int row = wm * WM + 32 * i + rw, col = (wn - 2) * WN + ch * 8;
            vo = (row < it.m_valid && col < it.n_valid) ? (uint32_t)((row * a.c_ld + col) * 2) : kOOB;
          }
          i32x4 d;
          d[0] = (int)v.x;
          d[1] = (int)v.y;
          d[2] = (int)v.z;
          d[3] = (int)v.w;
          __builtin_amdgcn_raw_buffer_store_b128(d, cr, (int)vo, 0, kPolicyStream);
        }
        lds_sync();   // exchange and staging are free for the next block
      }
      return;
    }
    uint16_t* stg = reinterpret_cast<uint16_t*>(st + wave * WREG);
    float* rsc = reinterpret_cast<float*>(st + NW * WREG);  // [BM] 1 / row scale
    float* csc = rsc + BM;                                  // [BN] 1 / column scale
    if constexpr (SCALED) {
      // every wave is done reading st; the scale DMAs, which only this
      // k-step's LPS tile transfers follow, and the next k-step's stage have
      // landed (the stream-K combine waited for whatever it issued since)
      wait_vm_sync<EPI_VM>();
      for (int idx = tid; idx < BM + BN; idx += kThreads) {
        const float v = scl[idx];
        if (idx < BM) rsc[idx] = v != 0.f ? 1.f / v : 0.f;
        else csc[idx - BM] = v != 0.f ? 1.f / v : 0.f;
      }
      lds_sync();
    } else {
      // every wave is done reading st, and the next k-step's stage has landed
      wait_vm_sync<EPI_VM_STAGES>();
    }
    const __amdgpu_buffer_rsrc_t cr =
        make_rsrc(reinterpret_cast<uint16_t*>(a.C) + (int64_t)it.g * a.c_gs + it.rowbase * a.c_ld + it.n0, 0x7FFFFFFF);
    const int r0 = wm * WM, c0 = wn * WN;   // the wave's sub-tile
#pragma unroll
    for (int e = 0; e < PASSES; ++e) {
      const int er = e / CPASS, ec = e % CPASS;   // row block, column block of the pass
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if (32 * j / ECW != ec) continue;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          if (32 * i / ERW != er) continue;
          const int rw = 32 * i + (lane & 31);
          float rs = 1.f;
          if constexpr (SCALED) rs = rsc[r0 + rw];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cw = 32 * j + 8 * q + 4 * (lane >> 5);   // column in the sub-tile
            float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
            float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
            if constexpr (SCALED) {
              const f32x4 cs4 = *reinterpret_cast<const f32x4*>(csc + c0 + cw);
              v0 = (v0 * cs4[0]) * rs;
              v1 = (v1 * cs4[1]) * rs;
              v2 = (v2 * cs4[2]) * rs;
              v3 = (v3 * cs4[3]) * rs;
            }
            uint2 pk;
            pk.x = pack_bf16x2_hw(v0, v1);
            pk.y = pack_bf16x2_hw(v2, v3);
            *reinterpret_cast<uint2*>(stg + (rw - er * ERW) * SROW + (cw - ec * ECW)) = pk;
          }
        }
      }
      // the wave reads back what its own lanes wrote: LDS executes a wave's
      // accesses in order, so a wait for the writes is all it takes
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < SPP; ++k) {
        const int q = lane + k * kWave;
        const int rw = q / (ECW / 8), ch = q % (ECW / 8);
        const uint4 v = *reinterpret_cast<const uint4*>(stg + rw * SROW + ch * 8);
        const int row = r0 + er * ERW + rw, col = c0 + ec * ECW + ch * 8;
        const uint32_t vo = (row < it.m_valid && col < it.n_valid) ? (uint32_t)((row * a.c_ld + col) * 2) : kOOB;
        i32x4 d;
        d[0] = (int)v.x;
        d[1] = (int)v.y;
        d[2] = (int)v.z;
        d[3] = (int)v.w;
        __builtin_amdgcn_raw_buffer_store_b128(d, cr, (int)vo, 0, kPolicyStream);
      }
      // the next pass overwrites the region only after these reads returned
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  };

  // Stream-K combination of a fixed-M tile (FIXED_M only).  Returns true when
  // acc holds the whole tile's sum afterwards and this workgroup must write it.
  // Partial tiles are stored and loaded with device-scope coherence (sc1:
  // written through to, and read from, the point where all XCDs agree), so
  // no L2-wide writeback or invalidate is needed: a wait for the stores to
  // complete orders them before the counter update, and the loads after the
  // counter update cannot hit stale lines.  (A __threadfence() here would
  // write back and invalidate the whole L2 of the XCD, and every later
  // operand load on that XCD would go back to HBM.)
  constexpr int PART_BYTES = BM * BN * 4;
  constexpr int WAVE_BYTES = TI * TJ * 4096;   // 16 floats x 64 lanes per block
  // (positions here are absolute; the stream-K ranges start at D * S)
  auto wg_of = [&](int64_t pos) -> int { return (int)(((pos - D * S + 1) * GS - 1) / L); };
  auto part_rsrc = [&](int bb, int64_t w) {
    const int64_t first = (D * S + (int64_t)bb * L / GS) / S;   // first item in bb's range
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sk_part) +
                          (int64_t)(2 * bb + (first == w ? 0 : 1)) * PART_BYTES + wave * WAVE_BYTES;
    return make_rsrc(base, WAVE_BYTES);
  };
  // Partial tiles in the MFMA register layout: 16 bytes per lane and
  // element quad, a 1 KB block per (i, j, q).  The block offset goes in the
  // instruction's scalar offset, so no per-block address stays live in a
  // VGPR across the K loop.
  auto part_io = [&](bool store, const __amdgpu_buffer_rsrc_t& r, const Item& it, bool add) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const bool ok = wm * WM + 32 * i + (lane & 31) < it.m_valid;
      const uint32_t vo = ok ? (uint32_t)(lane * 16) : kOOB;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int so = ((i * TJ + j) * 4 + q) * 1024;
          if (store) {
            i32x4 v;
            v[0] = __float_as_int(acc[i][j][4 * q]);
            v[1] = __float_as_int(acc[i][j][4 * q + 1]);
            v[2] = __float_as_int(acc[i][j][4 * q + 2]);
            v[3] = __float_as_int(acc[i][j][4 * q + 3]);
            __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)vo, so, kPolicyDevice);
          } else {
            const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, so, kPolicyDevice);
            if (add) {
              acc[i][j][4 * q] += __int_as_float(v[0]);
              acc[i][j][4 * q + 1] += __int_as_float(v[1]);
              acc[i][j][4 * q + 2] += __int_as_float(v[2]);
              acc[i][j][4 * q + 3] += __int_as_float(v[3]);
            } else {
              acc[i][j][4 * q] = __int_as_float(v[0]);
              acc[i][j][4 * q + 1] = __int_as_float(v[1]);
              acc[i][j][4 * q + 2] = __int_as_float(v[2]);
              acc[i][j][4 * q + 3] = __int_as_float(v[3]);
            }
          }
        }
    }
  };
  auto sk_combine = [&](const Item& it, int64_t w) -> bool {
    const int bf = wg_of(w * S), bl = wg_of(w * S + S - 1);
    if (bf == bl) return true;
    int32_t* flag = reinterpret_cast<int32_t*>(tab.scratch);
    if (bl - bf == 1) {
      // Two pieces (the usual split): the tile is own + other, and fp32
      // addition is commutative, so whichever piece finishes second adds the
      // other's partial to its registers -- the same bits either way.  A
      // piece that finds the other already published skips storing its own.
      const int other = b == bf ? bl : bf;
      if (tid == 0) *flag = __hip_atomic_load(a.sk_ctr + bf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_sync();
      if (uni(*flag) == 1) {
        if (tid == 0) __hip_atomic_store(a.sk_ctr + bf, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        part_io(false, part_rsrc(other, w), it, true);
        return true;
      }
      lds_sync();   // the peek is read by every wave before the flag is reused
      part_io(true, part_rsrc(b, w), it, false);
      wait_vm_all();   // this wave's partial has reached the coherence point
      lds_sync();
      if (tid == 0) {
        const int last = __hip_atomic_fetch_add(a.sk_ctr + bf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
        if (last) __hip_atomic_store(a.sk_ctr + bf, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
      }
      lds_sync();
      if (!uni(*flag)) return false;
      part_io(false, part_rsrc(other, w), it, true);
      return true;
    }
    // Three or more pieces: every piece stores its partial; the last to
    // arrive adds them all in workgroup order.
    part_io(true, part_rsrc(b, w), it, false);
    wait_vm_all();
    lds_sync();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(a.sk_ctr + bf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == bl - bf;
      if (last) __hip_atomic_store(a.sk_ctr + bf, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = last;
    }
    lds_sync();
    if (!uni(*flag)) return false;
    for (int bb = bf; bb <= bl; ++bb) part_io(false, part_rsrc(bb, w), it, bb != bf);
    return true;
  };

  // Dynamic-K split tile: every piece stores its partial (slot ci.slot +
  // piece); the last to arrive sums the pieces in order and writes the tile.
  // The same device-coherent protocol as the stream-K combine.
  auto slot_rsrc = [&](int slot) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sk_part) + (int64_t)slot * PART_BYTES + wave * WAVE_BYTES;
    return make_rsrc(base, WAVE_BYTES);
  };
  auto dk_combine = [&](const Item& it) -> bool {
    int32_t* flag = reinterpret_cast<int32_t*>(tab.scratch);
    part_io(true, slot_rsrc(it.slot() + it.piece()), it, false);
    wait_vm_all();   // this wave's partial has reached the coherence point
    lds_sync();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(a.sk_ctr + it.ctr(), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == it.pieces() - 1;
      if (last) __hip_atomic_store(a.sk_ctr + it.ctr(), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = last;
    }
    lds_sync();
    if (!uni(*flag)) return false;
    const int pc = it.pieces();
    for (int j = 0; j < pc; ++j) part_io(false, slot_rsrc(it.slot() + j), it, j != 0);
    return true;
  };

  // ---- main loop ----------------------------------------------------------
  // NS - 1 k-steps are loaded ahead; stages are used round-robin.
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) {
    const LoadCtx lx = prepare_loads(smem + u * STAGE);
#pragma unroll
    for (int q = 0; q < LPS; ++q) issue_one(lx, q);
    advance_load();
  }
  int stage = 0;            // stage holding the compute cursor's k-step
  int lstage = NS - 1;      // stage the next load goes to
  bool epi_prev = false;    // the last epilogue's NST stores follow the newest loads
  zero_acc();
  for (;;) {
    int last_stage = stage;
    for (; cs < cend; ++cs) {
      // this thread's DMA for the current stage has landed (only the next
      // NS - 2 stages' loads and the last epilogue's stores may be in
      // flight; after an epilogue the stage had landed before its stores
      // were issued), and every wave is past the previous k-step
      if (epi_prev) wait_vm_sync<(NS - 2) * LPS + NST>();
      else wait_vm_sync<(NS - 2) * LPS>();
      epi_prev = false;
      if (SCALED && cs + 1 == cend) issue_scales(ci);
      const LoadCtx lx = prepare_loads(smem + lstage * STAGE);
      lstage = lstage + 1 == NS ? 0 : lstage + 1;
      compute(smem + stage * STAGE, lx);   // also issues the loads of lx
      advance_load();                      // only now: setup() replaces the tiles' offsets
      last_stage = stage;
      stage = stage + 1 == NS ? 0 : stage + 1;
    }
    bool write = true;
    if constexpr (KIND == FIXED_M) write = cw < D || sk_combine(ci, cw);
    if constexpr (DK_SPLIT) {
      if (ci.pieces() > 1) write = dk_combine(ci);
    }
    if (write) {
      epilogue(smem + last_stage * STAGE, ci);
      epi_prev = true;
    }
    zero_acc();
    Pos np;
    if (!next_pos(cw, np)) break;
    cw = np.w;
    cs = np.s;
    ci = fetch(np.w, &ci);
    cend = np.e < 0 ? ci.nsteps : np.e;
  }
  wait_vm_all();   // no LDS-DMA transfer may outlive the workgroup
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

constexpr int kGemmWaves = 8;   // waves per workgroup

int gemm_tile_m(int kind) { (void)kind; return 128; }
int gemm_tile_n(int kind) { (void)kind; return 256; }

template <int BM, int BN, int NS, bool A_KC, bool B_KC, int KIND, int ELEM, int EPI, int NW>
static hipError_t launch_one(const GemmArgs& a, hipStream_t stream) {
  using T = ElemTraits<ELEM>;
  // host bound on the work: fixed-M tiles cover at most
  // floor(total_M / BM) + min(total_M, E) row slices
  int64_t work;
  if (KIND == FIXED_M) work = fixed_m_capacity(a.total_rows, a.E, BM) * cdiv(a.Nout, EPI == EPI_SWIGLU ? BN / 2 : BN) * cdiv(a.Kc, T::BK);
  else work = (int64_t)a.E * cdiv(a.Mout, BM) * cdiv(a.Nout, BN);
  if (work <= 0) return hipSuccess;
  // a dynamic-K launch whose tiles may be split takes up to 8 workgroups per
  // tile, so the pieces of a long contraction find idle workgroups
  if (KIND == DYNAMIC_K && ELEM == EL_BF16 && (int64_t)BM * BN * 4 <= kSkPartBytes) work *= 8;
  auto kern = gmm_kernel<BM, BN, NS, A_KC, B_KC, KIND, ELEM, EPI, NW>;
  const int dyn = table_lds_bytes(a.E);
  static int configured = 0;   // dynamic LDS size already allowed
  if (configured == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, table_lds_bytes(kMaxExperts));
    if (e != hipSuccess) return e;
    configured = 1;
  }
  int64_t slots = device_cu_count();
  if (KIND == FIXED_M && slots > kSkMaxGrid) slots = kSkMaxGrid;
  const int grid = (int)(work < slots ? work : slots);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), (size_t)dyn, stream, a);
  return hipGetLastError();
}

namespace {
thread_local int t_last_tile_m = 0;
}
int last_gemm_tile_m() { return t_last_tile_m; }

hipError_t launch_gemm(const GemmLaunch& L, const GemmArgs& a, hipStream_t stream) {
  if (gemm256_eligible(L, a)) {
    t_last_tile_m = 256;
    return launch_gemm256(L, a, stream);
  }
  t_last_tile_m = (L.kind == DYNAMIC_K && L.elem == EL_BF16 && !L.a_kc && !L.b_kc &&
                   a.total_rows <= 256 * (int64_t)a.E) ? 256 : 128;
  if (L.elem == EL_BF16) {
    if (L.kind == FIXED_M) {
      if (!L.a_kc) return hipErrorInvalidValue;
      if (L.swiglu) {
        if (L.b_kc) return launch_one<128, 256, 3, true, true, FIXED_M, EL_BF16, EPI_SWIGLU, kGemmWaves>(a, stream);
        return launch_one<128, 256, 3, true, false, FIXED_M, EL_BF16, EPI_SWIGLU, kGemmWaves>(a, stream);
      }
      if (L.b_kc) return launch_one<128, 256, 3, true, true, FIXED_M, EL_BF16, EPI_NONE, kGemmWaves>(a, stream);
      return launch_one<128, 256, 3, true, false, FIXED_M, EL_BF16, EPI_NONE, kGemmWaves>(a, stream);
    }
    if (!L.a_kc && !L.b_kc) {
      // Short contractions (at most 256 rows per group on average, so a few
      // k-steps per item): 256 x 256 tiles, two stages.  Every item's
      // operands then cross from L2 to LDS once per 256 x 256 outputs
      // instead of once per 128 x 256, and the one k-step in flight costs
      // little when items are that short.  Long contractions keep three
      // stages, which 256 x 256 tiles cannot fit in LDS.
      if (a.total_rows <= 256 * (int64_t)a.E)
        return launch_one<256, 256, 2, false, false, DYNAMIC_K, EL_BF16, EPI_NONE, kGemmWaves>(a, stream);
      return launch_one<128, 256, 3, false, false, DYNAMIC_K, EL_BF16, EPI_NONE, kGemmWaves>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  if (L.elem == EL_FP8) {
    if (!L.a_kc || !L.b_kc) return hipErrorInvalidValue;
    if (L.kind == FIXED_M) return launch_one<128, 256, 3, true, true, FIXED_M, EL_FP8, EPI_ROW_COL, kGemmWaves>(a, stream);
    return launch_one<128, 256, 3, true, true, DYNAMIC_K, EL_FP8, EPI_GROUP, kGemmWaves>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace mg
