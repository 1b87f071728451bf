// Persistent grouped GEMM for the compute-bound launches on gfx950: 256 x 256
// output tiles on four waves.
//
// The products are those of gmm.hip (grouped_gemm PR "Support GPU-resident
// batch sizes": the grouped forward and its dX; FBGEMM PR "F8I4 Grouped Gemm
// Optimization for Sparse M": only non-empty groups own work), for launches
// with enough rows per group that 256-row tiles stay mostly full:
//   bf16 fixed-M, B as [K, N] or [N, K], optionally with the A rows taken
//   through the token-sorted index and/or the SiLU*mul epilogue
//   (applied-ai issue "Column-major fused MoE": fused_moe_kernel and
//   silu_and_mul), the gate and up halves of B as column or row blocks;
//   e4m3 fixed-M with per-row and per-column scales (torchao commit
//   "Optimize FP8 MoE backward pass": the rowwise scaled operands).
//
// Design (CDNA4):
//  * 256 threads = 4 waves in a 2 x 2 arrangement; a wave owns a 128 x 128
//    block of 32 x 32 MFMA tiles, 256 fp32 accumulators per lane, which the
//    compiler keeps in AGPRs at one wave per SIMD.  Per flop this halves the
//    operand bytes that cross from L2 into LDS against a 128 x 256 tile, and
//    that stream, not the matrix cores, bounds the smaller tile.
//  * A k-step covers 64 contraction bytes of every operand row (32 bf16 or
//    64 e4m3 values); four LDS stages of 32 KB, filled by LDS-DMA
//    (buffer_load_dwordx4 ... lds), keep three k-steps in flight.
//  * Contraction-contiguous operands: two 64-byte rows per 128-byte LDS
//    line, 16-byte chunk position (row % 2) * 4 + chunk XOR-swizzled by the
//    line index, so the 32 rows a fragment read touches hit distinct banks.
//    Contraction-strided bf16 operands (B as [K, N]) keep their natural
//    layout, 32 rows of 512 bytes, chunks swizzled by 4 * (row % 4), and are
//    read with the transposing LDS load.
//  * Each wave reads the fragments of MFMA sub-step s + 1 while the MFMAs
//    of sub-step s run; the order of reads, transfers and MFMAs is pinned by
//    scheduling fences.  One barrier per k-step: before the first fragment
//    read of k-step j, every wave has its own transfers of k-step j landed
//    (vmcnt: only the newer NS - 2 batches may still be in flight -- loads
//    retire in order, and anything else in flight only makes the wait
//    stricter), and every wave is done reading stage j - 1, which then
//    takes k-step j - 1 + NS.
//  * Items run ahead across item boundaries; an item's epilogue stages its
//    output in the stage its last k-step used (each wave its own region,
//    32 rows x 64 columns at a time) and writes whole 128-byte row segments;
//    the transfer that would refill that stage is issued after the
//    epilogue and a barrier.
//  * Each XCD owns a contiguous eighth of the tiles and its workgroups take
//    them round-robin; tiles come in raster blocks of up to 5 row tiles, so
//    the 32 tiles an XCD runs at once cover about 5 row tiles x 6 column
//    tiles and share their operand slices in its L2.  When the XCD's last
//    round would leave most of its workgroups idle (at most a quarter of
//    them busy), each of that round's tiles is cut along the contraction
//    into P pieces, one per workgroup: the pieces store fp32 partial tiles
//    in the workspace and the last to arrive sums them in piece order.
#include "gemm_dev.h"

namespace mg {

namespace g256 {
constexpr int BM = 256, BN = 256;
constexpr int NW = 4;
constexpr int RB = 64;                // contraction bytes per operand row per k-step
constexpr int NS = 4;                 // LDS stages
constexpr int OPB = 256 * RB;         // bytes of one operand per stage (16 KB)
constexpr int STAGE = 2 * OPB;        // 32 KB
constexpr int LPW = 8;                // 16-byte transfers per lane per k-step (4 A + 4 B)
constexpr uint32_t RASTER = 5;        // row tiles per raster block
constexpr int NSCB = NS + 1;          // fp8 scale buffers, used round-robin by item
constexpr int SROW = 64 + 8;          // epilogue staging row (bf16 elements)
static_assert(NW * 32 * SROW * 2 <= STAGE, "epilogue staging fits a stage");
static_assert((NS - 2) * LPW <= 63, "vmcnt range");
constexpr int64_t PART = 256LL * 256 * 4;   // one fp32 partial tile (split dynamic-K contraction)
constexpr int PART_SLOTS = (int)(2 * kSkMaxGrid * kSkPartBytes / PART);   // partial slots in the workspace
constexpr int64_t MIN_PIECE = 8;            // shortest piece of a split dynamic-K contraction (k-steps)
constexpr int64_t TAIL_PIECE = 32;          // shortest piece of a split fixed-M last-round tile (k-steps)
constexpr int64_t DK_CAP_DIV = 1;           // dynamic-K split: pieces of at most a workgroup's share / this
constexpr int64_t HEAD_PCT = 60;            // unequal dynamic-K items: percent of the work dealt by XCD

// chunk swizzle of a contraction-contiguous tile: line L holds rows 2L, 2L+1
__device__ inline int kc_swz(int L) { return (L ^ (L >> 1)) & 3; }
// byte offset of (row, 16-byte chunk c in 0..3) in a contraction-contiguous tile
__device__ inline int kc_off(int row, int c) {
  const int L = row >> 1;
  return L * 128 + ((((row & 1) << 2) | c) ^ kc_swz(L)) * 16;
}
// byte offset of (contraction row r in 0..31, column c in 0..255) in a
// contraction-strided bf16 tile
__device__ inline int nt_off(int r, int c) { return r * 512 + (((c >> 3) ^ (4 * (r & 3))) << 4) + (c & 7) * 2; }
}  // namespace g256

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int ELEM> struct Frag256;
template <> struct Frag256<EL_BF16> {
  bf16x8 a[4], b[4];
};
template <> struct Frag256<EL_FP8> {
  i32x8 a[4], b[4];
};

#define G256_FENCE() __builtin_amdgcn_sched_barrier(0)

// The LDS-DMA asm takes its resource and LDS address in SGPRs; both are
// workgroup-uniform here, which readfirstlane states for the compiler.
__device__ inline i32x4 uni4(i32x4 r) {
  i32x4 u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

template <bool B_KC, int ELEM, int EPI, int KIND>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) gmm256_kernel(GemmArgs a) {
  using namespace g256;
  constexpr int ESZ = ELEM == EL_FP8 ? 1 : 2;
  constexpr int EPC = 16 / ESZ;                    // elements per 16-byte chunk
  constexpr int BK = RB / ESZ;                     // contraction elements per k-step
  constexpr int KSUB = ELEM == EL_FP8 ? 1 : 2;     // MFMA sub-steps per k-step
  constexpr bool SCALED = EPI == EPI_ROW_COL || EPI == EPI_GROUP;
  constexpr bool DK = KIND == DYNAMIC_K;
  constexpr bool SWIGLU = EPI == EPI_SWIGLU;
  constexpr int BNE = SWIGLU ? BN / 2 : BN;        // output columns per tile
  constexpr bool TSPLIT = KIND == FIXED_M && !SWIGLU;   // last-round tiles may be cut into pieces
  constexpr bool PIECES = DK || TSPLIT;
  static_assert(ELEM == EL_BF16 || (B_KC && SCALED), "fp8: both operands k-contiguous, scaled");
  static_assert(!DK || (ELEM == EL_FP8 && EPI == EPI_GROUP), "dynamic-K: e4m3 with per-group scales");
  static_assert(!SWIGLU || ELEM == EL_BF16, "paired gate/up epilogue: bf16");
  static_assert(ELEM == EL_FP8 || EPI == EPI_NONE || SWIGLU, "bf16 epilogues");

  __shared__ __attribute__((aligned(16))) uint8_t smem[NS * STAGE];
  // fp8: the row and column scales of the last NSCB items (row scales, then
  // column scales, 256 each), and the reciprocals the epilogue applies
  __shared__ __attribute__((aligned(16))) float scl[SCALED ? NSCB * 512 : 4];
  __shared__ __attribute__((aligned(16))) float rcp[SCALED ? 512 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l31 = lane & 31, hi = lane >> 5;

  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  const GroupTable tab = carve_table(table_lds, a.E);
  const int err = build_group_table(a.sizes, a.E, a.total_rows, BM, DK, tab);
  if (err != 0 && blockIdx.x == 0 && tid == 0 && a.err != nullptr) *a.err = err;

  const int n_tiles = (int)cdiv(a.Nout, BNE);
  const int G = gridDim.x;
  const int m_tiles_dk = DK ? (int)cdiv(a.Mout, BM) : 1;
  // Dynamic-K split plan (grouped_gemm PR review thread: problems sorted by
  // k, descending): a group whose contraction is longer than a workgroup's
  // share of all k-steps is cut into pieces of at most that share (and of
  // at least MIN_PIECE), so a few large groups cannot leave most of the
  // grid idle.  Each piece stores its fp32 partial tile in the workspace;
  // the last to arrive adds all pieces in piece order (the same bits
  // whatever the arrival order) and writes the tile.  Limits: one arrival
  // counter per split tile (kSkMaxGrid), one partial slot per piece
  // (PART_SLOTS).  Every workgroup computes the same plan from the table.
  __shared__ DkSplit sp;
  auto steps_of = [&](int g) -> int64_t {   // k-steps of group g's contraction (dynamic-K)
    const int32_t off = tab.off[g], eff = tab.eff[g];
    if (eff <= 0) return 1;
    const int64_t start = (int64_t)off & ~(int64_t)15;
    return cdiv((int64_t)off + eff - start, BK);
  };
  if constexpr (DK) {
    int64_t mine = 0;
    for (int g = tid; g < a.E; g += 256) mine += steps_of(g);
    const int64_t all = block_incl_scan64(mine, tab.scratch);   // the last thread's value is the total
    if (tid == 255) tab.scratch[15] = all;
    __syncthreads();
    if (tid == 0) {
      const int per = m_tiles_dk * n_tiles;
      int64_t cap = cdiv(tab.scratch[15] * per, (int64_t)G * DK_CAP_DIV);
      if (cap < MIN_PIECE) cap = MIN_PIECE;
      int ns = 0, slots = 0;
      sp.items_before[0] = 0;
      sp.slot_before[0] = 0;
      while (ns < kDkMaxSplitGroups && ns < a.E) {
        const int64_t st = steps_of(tab.order[ns]);
        int pc = (int)cdiv(st, cap);
        if (pc > st) pc = (int)st;
        if (pc < 2) break;
        if ((ns + 1) * per > kSkMaxGrid) break;            // arrival counters
        if (slots + pc * per > PART_SLOTS) break;           // partial slots
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
  const int64_t items = uni64(DK ? (int64_t)(a.E - sp.groups) * m_tiles_dk * n_tiles + sp.items_before[sp.groups]
                                 : (int64_t)tab.tstart[a.E] * n_tiles);
  // Items of equal length (fixed-M tiles; dynamic-K tiles when every group
  // has the same size): XCD x (workgroups are dealt round-robin to the 8
  // XCDs) owns items [x D / 8, (x + 1) D / 8), taken round-robin by its G / 8
  // workgroups.
  bool equal_items = true;
  if constexpr (DK)
    equal_items = uni(sp.groups) == 0 && uni(tab.eff[uni(tab.order[0])]) == uni(tab.eff[uni(tab.order[a.E - 1])]);
  const bool xcd_split = equal_items && (G & 7) == 0;
  // Dynamic-K items of unequal length (groups come largest first) come from
  // a work queue: a workgroup's first item is its own index, and every
  // further one the next index handed out by an atomic counter in the
  // workspace, so a workgroup that drew long items draws fewer -- the
  // longest-first greedy deal.  Thread 0 requests items into a ring in LDS
  // six ahead of the compute cursor (the load cursor runs at most four
  // ahead), right after an epilogue: waiting there for the counter's reply
  // waits for little else, since the next item's loads had the epilogue's
  // time to land.  The last workgroup to finish resets the counters.
  // (Tiles handed out this way share no L2 by XCD, which costs against the
  // static deal when the groups are equal; measured on MI355X with the
  // Zipf-skewed groups of a DeepSeek-MoE layer share, it still beats a
  // static longest-first deal.)
  const bool dyn = DK && !equal_items;
  // With a grid of whole XCD rounds, the queue has two levels.  The first
  // HEAD_PCT percent of the work (the longest items) is cut into 8 runs of
  // equal work, one per XCD, each handed out by that XCD's own counter.
  // The tiles of one group share their operand slabs, and a run keeps them
  // in one L2: measured on the Zipf-skewed groups of a DeepSeek-MoE layer
  // share, a single queue spread every group over all 8 L2s and fetched
  // 8 times the operand bytes.  The rest, the short items, comes from one
  // counter shared by all, which evens out the finish.
  const bool xq = HEAD_PCT > 0 && dyn && (G & 7) == 0;
  __shared__ int32_t seg[9];   // XCD x's run: items [seg[x], seg[x + 1]); seg[8]: the first shared item
  if (xq) {
    const int per_t = m_tiles_dk * n_tiles;
    const int ns = sp.groups;
    const int pp = (a.E + 255) / 256;   // group-order positions per thread (<= 4)
    const int q0 = tid * pp;
    int64_t wl = 0;   // work (k-steps x tiles) of this thread's positions
    for (int i = 0; i < pp; ++i)
      if (q0 + i < a.E) wl += steps_of(tab.order[q0 + i]) * per_t;
    const int64_t incl = block_incl_scan64(wl, tab.scratch);
    const int64_t head = tab.scratch[15] * per_t * HEAD_PCT / 100;   // of all the work
    int64_t before = incl - wl;
    for (int i = 0; i < pp; ++i) {
      const int q = q0 + i;
      if (q >= a.E) break;
      const int64_t wq_ = steps_of(tab.order[q]) * per_t;
      const int64_t n = q < ns ? (int64_t)sp.pieces[q] * per_t : per_t;   // its items, of equal work
      const int64_t ib = q < ns ? sp.items_before[q] : sp.items_before[ns] + (int64_t)(q - ns) * per_t;
      for (int x = 1; x <= 8; ++x) {   // the item where work head * x / 8 falls
        const int64_t t = head * x / 8;
        if (t >= before && t < before + wq_) seg[x] = (int32_t)(ib + (t - before) * n / wq_);
      }
      before += wq_;
    }
    if (tid == 0) seg[0] = 0;
    __syncthreads();
  }
  __shared__ int32_t qring[16];   // the workgroup's n-th item at [n % 16] (-1: none)
  bool own_left = true;           // (thread 0) the XCD's run may hold more items
  auto grab = [&](int64_t n) __attribute__((always_inline)) {
    if (tid == 0) {
      int code = -1;
      if (xq) {
        const int x = blockIdx.x & 7;
        if (own_left) {
          const int l = n == 0 ? (int)(blockIdx.x >> 3)
                               : (G >> 3) + __hip_atomic_fetch_add(a.wq + 16 + x, 1, __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_AGENT);
          if (l >= 0 && l < seg[x + 1] - seg[x]) code = seg[x] + l;
          else own_left = false;
        }
        if (code < 0) {
          const int l = __hip_atomic_fetch_add(a.wq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (l >= 0 && l < items - seg[8]) code = seg[8] + l;
        }
      } else if (n == 0) {
        code = (int)blockIdx.x;
      } else {
        const int l = G + __hip_atomic_fetch_add(a.wq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (l >= 0 && l < items) code = l;
      }
      qring[n & 15] = code;
    }
  };
  // counts this workgroup out; the last one resets the counters
  auto queue_exit = [&]() __attribute__((always_inline)) {
    if (dyn && tid == 0) {
      const int done = __hip_atomic_fetch_add(a.wq + 8, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == G - 1) {
        __hip_atomic_store(a.wq, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.wq + 8, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int x = 0; x < 8; ++x) __hip_atomic_store(a.wq + 16 + x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  if (dyn) {
    for (int n = 0; n <= 6; ++n) grab(n);
    __syncthreads();
  }
  const int64_t gx = xcd_split ? (G >> 3) : G;
  const int64_t dj = xcd_split ? (int64_t)(blockIdx.x >> 3) : blockIdx.x;
  const int64_t c0 = xcd_split ? ((int64_t)(blockIdx.x & 7) * items) >> 3 : 0;
  const int64_t c1 = xcd_split ? ((int64_t)((blockIdx.x & 7) + 1) * items) >> 3 : items;
  // Fixed-M last round: the XCD's n tiles run as floor(n / gx) full rounds
  // and a last round of r = n % gx tiles, which at 256 x 256 tiles and long
  // contractions (the second FFN GEMM) can idle most of the XCD for a whole
  // tile's time.  With r <= gx / 4, each of those r tiles is cut into P
  // = min(8, gx / r) pieces of at least TAIL_PIECE k-steps, one piece per
  // workgroup (piece j of last-round tile t is item code D + j r + t, D the
  // tile count).  Tile t's arrival counter is x gx + t, its piece j's
  // partial slot x gx + t P + j: with gx <= 32 every XCD stays inside its
  // own 32 counters and slots.  (Measured on MI355X: with a quarter of the
  // XCD or more busy, a last round of whole tiles runs about as fast as the
  // same work in pieces -- the k-steps of the few busy workgroups speed up
  // -- and short pieces lose to the partials' round trip.)
  int64_t whole = c1 - c0;   // the XCD's tiles that run whole
  int64_t tail_r = 0, tail_p = 1;
  if constexpr (TSPLIT) {
    const int64_t r = (c1 - c0) % gx;
    if (xcd_split && G <= kSkMaxGrid && G <= PART_SLOTS && r > 0 && 4 * r <= gx) {
      int64_t p = gx / r;
      if (p > 8) p = 8;
      const int64_t steps = cdiv(a.Kc, BK);
      if (p > steps / TAIL_PIECE) p = steps / TAIL_PIECE;
      if (p >= 2) {
        tail_r = r;
        tail_p = p;
        whole = c1 - c0 - r;
      }
    }
  }
  // the workgroup's k-th item code (-1: none)
  auto item_of = [&](int64_t k) __attribute__((always_inline)) -> int64_t {
    if (dyn) {
      const int code = uni(qring[k & 15]);
      return code < 0 ? -1 : code;   // none left (or the counter was not zeroed)
    }
    const int64_t u = dj + k * gx;
    if (u < whole) return c0 + u;
    const int64_t v = u - whole;
    return TSPLIT && v < tail_r * tail_p ? items + v : -1;
  };
  if (item_of(0) < 0) {
    queue_exit();
    return;
  }
  // (every field is workgroup-uniform; said so, so that items live in SGPRs)
  auto fetch = [&](int64_t w) __attribute__((always_inline)) {
    int64_t t = 0, j = 0;
    if (TSPLIT && w >= items) {   // piece j of the XCD's last-round tile t
      t = (w - items) % tail_r;
      j = (w - items) / tail_r;
    }
    Item it = get_item<BM, BNE, KIND, ELEM, BK, DK, RASTER>(a, tab, TSPLIT && w >= items ? c0 + whole + t : w,
                                                           n_tiles, m_tiles_dk, nullptr, sp);
    if (TSPLIT && w >= items) {   // k-steps [j S / P, (j + 1) S / P) of the tile's S
      const int s0 = (int)(j * it.nsteps / tail_p), s1 = (int)((j + 1) * it.nsteps / tail_p);
      const int base = (int)((blockIdx.x & 7) * gx);
      it.c_begin = (int64_t)s0 * BK;
      it.nsteps = s1 - s0;
      it.split = ((int)tail_p << 16) | (int)j;
      it.sloc = ((base + (int)t) << 16) | (base + (int)(t * tail_p));
    }
    it.g = uni(it.g);
    it.rowbase = uni64(it.rowbase);
    it.m_valid = uni(it.m_valid);
    it.n0 = uni(it.n0);
    it.n_valid = uni(it.n_valid);
    it.c_lo = uni64(it.c_lo);
    it.c_hi = uni64(it.c_hi);
    it.c_begin = uni64(it.c_begin);
    it.nsteps = uni(it.nsteps);
    it.split = uni(it.split);
    it.sloc = uni(it.sloc);
    return it;
  };
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(a.B);
  const bool gather = ELEM == EL_BF16 && a.gather != nullptr;

  // ---- transfers: this wave's 4 A and 4 B instructions of a k-step ----
  // A (contraction-contiguous): instruction i = 4 wave + q covers tile rows
  // 16 i .. 16 i + 15; lane l lands at LDS line 8 i + l / 8, chunk position
  // l % 8, which holds row 2 L + p / 4, chunk p % 4 (p = l % 8 ^ swizzle).
  uint32_t voA[4], voB[4];
  // the chunk index (0..3) each of the lane's 8 transfers fetches, 2 bits
  // each (A 0..3, B 4..7): only the k-step that the contraction's end cuts
  // needs them
  uint32_t chunks = 0;
  auto kc_row = [&](int ln, int q, int& c) __attribute__((always_inline)) {
    const int i = 4 * wave + q;
    const int L = 8 * i + (ln >> 3);
    const int p = (ln & 7) ^ kc_swz(L);
    c = p & 3;
    return 2 * L + (p >> 2);
  };
  // (offsets in 32 bits: every operand is below 2 GiB, checked on the host)
  const uint32_t a_row = (uint32_t)(a.a_ld * ESZ), b_row = (uint32_t)(a.b_ld * ESZ);
  auto setup = [&](const Item& it) __attribute__((always_inline)) {
    // per-lane offsets from an opaque copy of the lane index: recomputed at
    // each item (cheap), never hoisted into registers held across the loop
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
    chunks = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int c;
      const int row = kc_row(ln, q, c);
      chunks |= (uint32_t)c << (2 * q);
      if (gather) {
        // the 16 rows of the instruction: ids read as scalars from clamped
        // addresses, each lane picking its own
        typedef const __attribute__((address_space(4))) int32_t* cptr;
        const cptr ids = (cptr)(a.gather + it.rowbase);
        const int r0 = 16 * (4 * wave + q);
        int id = a.gather_limit;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          const int rs = r0 + s < it.m_valid ? r0 + s : it.m_valid - 1;
          const int v = ids[rs];
          id = (row - r0 == s) ? v : id;
        }
        if (row >= it.m_valid) id = a.gather_limit;
        voA[q] = (id >= 0 && id < a.gather_limit) ? (uint32_t)(id / a.gather_div) * a_row + (uint32_t)(c * 16) : kOOB;
      } else {
        voA[q] = row < it.m_valid ? (uint32_t)row * a_row + (uint32_t)(c * 16) : kOOB;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (B_KC) {
        int c;
        const int row = kc_row(ln, q, c);
        chunks |= (uint32_t)c << (2 * (4 + q));
        if constexpr (SWIGLU) {
          // gate rows n0.. in tile rows 0..127, up rows I + n0.. in 128..255
          const int src = row + (row >= BNE ? a.Nout - BNE : 0);
          voB[q] = (row & (BNE - 1)) < it.n_valid ? (uint32_t)src * b_row + (uint32_t)(c * 16) : kOOB;
        } else {
          voB[q] = row < it.n_valid ? (uint32_t)row * b_row + (uint32_t)(c * 16) : kOOB;
        }
      } else {
        // 32 contraction rows of 512 bytes; instruction i covers rows 2i, 2i+1
        const int i = 4 * wave + q;
        const int r = 2 * i + (ln >> 5);
        const int ch = (ln & 31) ^ (4 * (r & 3));   // the column chunk that belongs at this slot
        int col, ok;
        if constexpr (SWIGLU) {
          const int hc = ch & 15;   // gate chunks 0..15, up chunks 16..31 (columns I + n0 ..)
          col = ch * 8 + (ch >= 16 ? a.Nout - BNE : 0);
          ok = hc * 8 < it.n_valid;
        } else {
          col = ch * 8;
          ok = col < it.n_valid;
        }
        voB[q] = ok ? (uint32_t)r * b_row + (uint32_t)(col * 2) : kOOB;
      }
    }
  };

  // load cursor: item lw, k-step ls
  int64_t lk = 0;               // load cursor: the workgroup's lk-th item, k-step ls
  int64_t lw = item_of(0);
  int ls = 0;
  Item li = fetch(lw);
  bool ldone = false;
  int lseq = 0;                 // items started by the load cursor
  setup(li);
  const uint32_t lbase = lds_address(smem);
  const uint32_t sbase = lds_address(reinterpret_cast<uint8_t*>(scl));

  // the scale transfers of item it into buffer b: 256 row scales, then 256
  // column scales, 64 per instruction, two instructions per wave
  auto issue_scales = [&](const Item& it, int b) __attribute__((always_inline)) {
    if constexpr (SCALED) {
      const float* rows = a.sa + (DK ? (int64_t)it.g * a.Mout + it.rowbase : it.rowbase);
      const i32x4 rr = uni4(make_rsrc_words(rows, (int64_t)it.m_valid * 4));
      const i32x4 rc = uni4(make_rsrc_words(a.sb + (int64_t)it.g * a.Nout + it.n0, (int64_t)it.n_valid * 4));
      dma4(rr, sbase + (b * 512 + 64 * wave) * 4, (uint32_t)((64 * wave + lane) * 4));
      dma4(rc, sbase + (b * 512 + 256 + 64 * wave) * 4, (uint32_t)((64 * wave + lane) * 4));
    }
  };

  // One batch: the load cursor's k-step into stage st (past the last item:
  // zero-size resources, so every batch is LPW transfers per lane).
  // prepare() builds the resources (SGPRs) and this lane's 8 offsets, with
  // chunks past the contraction's end sent out of range.
  struct Batch {
    i32x4 ra, rb;
    uint32_t st;
    uint32_t vo[LPW];
  };
  auto prepare = [&](int st) __attribute__((always_inline)) -> Batch {
    Batch x;
    // contraction index of the k-step's first element, and the item's range
    // relative to it (clamped to int)
    const int64_t cb = li.c_begin + (int64_t)ls * BK;
    const int64_t lo64 = li.c_lo - cb, hi64 = li.c_hi - cb;
    const int lo = lo64 < -BK ? -BK : (lo64 > 2 * BK ? 2 * BK : (int)lo64);
    const int hi = hi64 < -BK ? -BK : (hi64 > 2 * BK ? 2 * BK : (int)hi64);
    // dynamic-K operands end where the matrix ends; an empty group reads nothing
    int64_t a_ext = 0x7FFFFFFF, b_ext = 0x7FFFFFFF;
    if constexpr (DK) {
      a_ext = li.c_hi <= li.c_lo ? 0 : (int64_t)(li.m_valid - 1) * a.a_ld + (a.total_rows - cb);
      b_ext = li.c_hi <= li.c_lo ? 0 : (int64_t)(li.n_valid - 1) * a.b_ld + (a.total_rows - cb);
    }
    const uint8_t* abase = gather ? Ab + cb * ESZ : Ab + (li.rowbase * a.a_ld + cb) * ESZ;
    x.ra = uni4(make_rsrc_words(abase, ldone ? 0 : a_ext));
    if constexpr (B_KC)
      x.rb = uni4(make_rsrc_words(Bb + ((int64_t)li.g * a.b_gs + (int64_t)li.n0 * a.b_ld + cb) * ESZ,
                                  ldone ? 0 : b_ext));
    else
      x.rb = uni4(make_rsrc_words(Bb + ((int64_t)li.g * a.b_gs + cb * a.b_ld + li.n0) * 2,
                                  ldone ? 0 : ((int64_t)a.Kc - cb) * a.b_ld * 2));
    x.st = (uint32_t)uni((int)(lbase + st * STAGE));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x.vo[q] = voA[q];
      x.vo[4 + q] = voB[q];
    }
    if (lo > 0 || hi < BK) {   // a k-step the contraction range cuts: chunks outside it read zeros
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const int c = (int)((chunks >> (2 * q)) & 3u);
        if (q < 4 || B_KC) x.vo[q] = (c * EPC + EPC > lo && c * EPC < hi) ? x.vo[q] : kOOB;
      }
    }
    return x;
  };
  auto issue_one = [&](const Batch& x, int q) __attribute__((always_inline)) {
    if (q < 4) dma16<kPolicyCached>(x.ra, x.st + (4 * wave + q) * 1024, x.vo[q]);
    else dma16<kPolicyCached>(x.rb, x.st + OPB + (4 * wave + q - 4) * 1024, x.vo[q]);
  };
  auto advance_load = [&]() __attribute__((always_inline)) {
    if (ldone) return;
    if (ls + 1 < li.nsteps) {
      ++ls;
      return;
    }
    const int64_t nw = item_of(++lk);
    if (nw < 0) {
      ldone = true;
      return;
    }
    lw = nw;
    ls = 0;
    li = fetch(lw);
    setup(li);
    ++lseq;
  };
  // a whole batch for the load cursor into stage st, with the scales of the
  // item it starts
  auto load_step = [&](int st) __attribute__((always_inline)) {
    if (SCALED && ls == 0 && !ldone) issue_scales(li, lseq % NSCB);
    const Batch x = prepare(st);
#pragma unroll
    for (int q = 0; q < LPW; ++q) issue_one(x, q);
    advance_load();
  };

  // ---- fragments ----
  const int Ll = l31 >> 1;
  auto kc_frag_off = [&](int c) __attribute__((always_inline)) -> int { return Ll * 128 + ((((l31 & 1) << 2) | (c ^ kc_swz(Ll))) * 16); };
  // one LDS read of fragment piece n of sub-step ks of stage st: bf16 n =
  // 0..7 in the order a0 b0 b1 b2 b3 a1 a2 a3, e4m3 n = 0..15 (the same
  // order, low then high 16 bytes)
  constexpr int ORD_A[8] = {1, 0, 0, 0, 0, 1, 1, 1};
  constexpr int ORD_X[8] = {0, 0, 1, 2, 3, 1, 2, 3};
  constexpr int NREAD = ELEM == EL_FP8 ? 16 : 8;
  auto read_one = [&](Frag256<ELEM>& f, int st, int ks, int n) __attribute__((always_inline)) {
    const uint8_t* As = smem + st * STAGE;
    const uint8_t* Bs = As + OPB;
    if constexpr (ELEM == EL_BF16) {
      const int x = ORD_X[n];
      if (ORD_A[n]) {
        f.a[x] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + 32 * x) * 64 + kc_frag_off(2 * ks + hi));
      } else if constexpr (B_KC) {
        f.b[x] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 128 + 32 * x) * 64 + kc_frag_off(2 * ks + hi));
      } else {
        // transposing read: within each 16-lane group, lane s addresses
        // contraction row k0 + s / 4, columns c + 4 (s % 4) .. + 3; two reads
        // (rows k0 and k0 + 4) give the lane its column's 8 values
        const int Gq = lane >> 4, sl = lane & 15;
        const int k0 = ks * 16 + 8 * (Gq >> 1) + (sl >> 2);
        const int col = wn * 128 + 32 * x + 16 * (Gq & 1) + 4 * (sl & 3);
        auto p = (__attribute__((address_space(3))) uint8_t*)Bs;
        const int a0 = nt_off(k0, col);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + a0));
        const s16x4 hh = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + a0 + 4 * 512));
        f.b[x] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hh, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
      const int half = n & 1, x = ORD_X[n >> 1];
      const int o = kc_frag_off(2 * hi + half);
      if (ORD_A[n >> 1]) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(As + (wm * 128 + 32 * x) * 64 + o);
        if (half) f.a[x].hi = v; else f.a[x].lo = v;
      } else {
        const i32x4 v = *reinterpret_cast<const i32x4*>(Bs + (wn * 128 + 32 * x) * 64 + o);
        if (half) f.b[x].hi = v; else f.b[x].lo = v;
      }
    }
  };

  f32x16 acc[4][4];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  };
  // MFMA n (0..15) of a sub-step: block (n / 4, n % 4).  Operands swapped,
  // so acc[i][j] holds the transposed 32 x 32 block: lane l has output row
  // 32 i + l % 32 of the wave's block and columns 32 j + 8 q + 4 (l / 32) + r
  // in element 4 q + r.
  // LIVE false: the wave's 128 x 128 quadrant lies wholly outside the
  // tile's valid rows or columns, and its MFMAs are left out (the transfers,
  // fragment reads and barriers stay, so every wave follows one schedule).
  auto mfma_one = [&](const Frag256<ELEM>& f, int n, auto live_c) __attribute__((always_inline)) {
    if constexpr (!decltype(live_c)::value) return;
    const int i = n >> 2, j = n & 3;
    if constexpr (ELEM == EL_BF16)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], 0, 0, 0, 127, 0, 127);
  };
  constexpr int RPG = NREAD / 8;
  // A sub-step inside a k-step (bf16 only): the 16 MFMAs on cur, the reads
  // of nxt (the k-step's second sub-step) interleaved, one read per 2 MFMAs.
  auto inner_sub = [&](const Frag256<ELEM>& cur, Frag256<ELEM>& nxt, int st, auto live_c)
      __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int r = 0; r < RPG; ++r) read_one(nxt, st, 1, t * RPG + r);
      mfma_one(cur, 2 * t, live_c);
      mfma_one(cur, 2 * t + 1, live_c);
      G256_FENCE();
    }
  };
  // The last sub-step of k-step j: 2 MFMAs, barrier B(j + 1), then the batch
  // that refills stage j and the reads of nxt from stage j + 1 interleaved
  // with the other 14 MFMAs.  At an item's last k-step (LAST) neither: the
  // refill waits for the epilogue, which stages the output in stage j, and
  // the next k-step's fragments are read after it.
  auto boundary_sub = [&](const Frag256<ELEM>& cur, Frag256<ELEM>& nxt, int stj, auto last_c, auto live_c)
      __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_c)::value;
    const int stn = stj + 1 == NS ? 0 : stj + 1;
    mfma_one(cur, 0, live_c);
    mfma_one(cur, 1, live_c);
    G256_FENCE();
    wait_vm_sync<(NS - 2) * LPW>();
    if constexpr (!LAST) {
      if (SCALED && ls == 0 && !ldone) issue_scales(li, lseq % NSCB);
      const Batch x = prepare(stj);
      advance_load();   // (x holds all this batch needs)
      G256_FENCE();
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        issue_one(x, t);
#pragma unroll
        for (int r = 0; r < RPG; ++r) read_one(nxt, stn, 0, t * RPG + r);
        if (t < 7) {
          mfma_one(cur, 2 + 2 * t, live_c);
          mfma_one(cur, 3 + 2 * t, live_c);
        }
        G256_FENCE();
      }
    } else {
      G256_FENCE();
#pragma unroll
      for (int n = 2; n < 16; ++n) mfma_one(cur, n, live_c);
      G256_FENCE();
    }
  };

  // partial slot of a split dynamic-K tile, this wave's 64 KB of it
  auto slot_rsrc = [&](int slot) __attribute__((always_inline)) {
    return make_rsrc(reinterpret_cast<const uint8_t*>(a.sk_part) + (int64_t)slot * PART + wave * (PART / 4), PART / 4);
  };

  // ---- epilogue: the item's output through stage st ----
  // With npieces > 0 (the last-arriving piece of a split dynamic-K tile)
  // the values are the sums, in piece order, of the pieces' partial tiles in
  // slots slot0 .. slot0 + npieces - 1, and acc (already zero) is not read.
  auto epilogue = [&](int st, const Item& it, int sb, int npieces, int slot0) __attribute__((always_inline)) {
    uint8_t* stg_base = smem + st * STAGE;
    // lane-derived addresses from an opaque copy of the lane index, so they
    // are computed here rather than hoisted and held across the k-loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int l31 = lane & 31, hi = lane >> 5;
    if constexpr (SCALED) {
      // reciprocals of the item's scales (exact: the scales are powers of two
      // or zero) for every wave
      for (int idx = tid; idx < 512; idx += 256) {
        const float v = scl[sb * 512 + idx];
        rcp[idx] = v != 0.f ? 1.f / v : 0.f;
      }
      lds_sync();
    }
    if constexpr (SWIGLU) {
      // gate wave (wm, 0) and up wave (wm, 1) hold the same rows and
      // matching columns; per 32-row block and 64-column half the gate wave
      // hands its bf16-rounded values over (lane-contiguous dwords), the up
      // wave forms act = silu(g) * u in fp32 from the bf16 values and stages
      // it for 16-byte stores of whole 128-byte row segments
      uint32_t* xch = reinterpret_cast<uint32_t*>(stg_base) + wm * 16 * 64;   // [2 wm][16 dwords][64 lanes]
      uint16_t* stg = reinterpret_cast<uint16_t*>(stg_base + 2 * 16 * 64 * 4) + wm * 32 * SROW;
      const __amdgpu_buffer_rsrc_t cr =
          make_rsrc(reinterpret_cast<uint16_t*>(a.C) + it.rowbase * a.c_ld + it.n0, 0x7FFFFFFF);
      const bool up = wn == 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = e >> 1, h = e & 1;
        if (!up) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int d = 0; d < 8; ++d)
              xch[(jj * 8 + d) * 64 + lane] =
                  pack_bf16x2_hw(acc[i][2 * h + jj][2 * d], acc[i][2 * h + jj][2 * d + 1]);
        }
        lds_sync();
        if (up) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int j = 2 * h + jj;
              const uint32_t g01 = xch[(jj * 8 + 2 * q) * 64 + lane];
              const uint32_t g23 = xch[(jj * 8 + 2 * q + 1) * 64 + lane];
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
              *reinterpret_cast<uint2*>(stg + l31 * SROW + 32 * jj + 8 * q + 4 * hi) = pk;
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int qq = lane + k * 64;
            const int rw = qq >> 3, ch = qq & 7;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + rw * SROW + ch * 8);
            const int row = wm * 128 + 32 * i + rw, col = 64 * h + ch * 8;
            const uint32_t vo = (row < it.m_valid && col < it.n_valid) ? (uint32_t)((row * a.c_ld + col) * 2) : kOOB;
            i32x4 d;
            d[0] = (int)v.x;
            d[1] = (int)v.y;
            d[2] = (int)v.z;
            d[3] = (int)v.w;
            __builtin_amdgcn_raw_buffer_store_b128(d, cr, (int)vo, 0, kPolicyStream);
          }
        }
        lds_sync();   // exchange and staging are free for the next pass
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][2 * h + jj][v] = 0.f;   // ready for the next item
      }
      return;
    }
    uint16_t* stg = reinterpret_cast<uint16_t*>(stg_base) + wave * 32 * SROW;
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(
        reinterpret_cast<uint16_t*>(a.C) + (int64_t)it.g * a.c_gs + it.rowbase * a.c_ld + it.n0, 0x7FFFFFFF);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = e >> 1, h = e & 1;   // 32-row block, 64-column half of the wave's block
      float rs = 1.f;
      if constexpr (SCALED) rs = rcp[wm * 128 + 32 * i + l31];
      const uint32_t pvo = wm * 128 + 32 * i + l31 < it.m_valid ? (uint32_t)(lane * 16) : kOOB;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * h + jj;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cw = 32 * jj + 8 * q + 4 * hi;   // column in the 64-wide staging row
          float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
          float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          if constexpr (PIECES) {
            if (npieces > 0) {
              v0 = v1 = v2 = v3 = 0.f;
              for (int p = 0; p < (DK ? npieces : 0); ++p) {
                const i32x4 pv = __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(slot0 + p), (int)pvo,
                                                                        ((i * 4 + j) * 4 + q) * 1024, kPolicyDevice);
                v0 += __int_as_float(pv[0]);
                v1 += __int_as_float(pv[1]);
                v2 += __int_as_float(pv[2]);
                v3 += __int_as_float(pv[3]);
              }
            }
          }
          if constexpr (SCALED) {
            const f32x4 cs4 = *reinterpret_cast<const f32x4*>(rcp + 256 + wn * 128 + 64 * h + cw);
            v0 = (v0 * cs4[0]) * rs;
            v1 = (v1 * cs4[1]) * rs;
            v2 = (v2 * cs4[2]) * rs;
            v3 = (v3 * cs4[3]) * rs;
          }
          uint2 pk;
          pk.x = pack_bf16x2_hw(v0, v1);
          pk.y = pack_bf16x2_hw(v2, v3);
          *reinterpret_cast<uint2*>(stg + l31 * SROW + cw) = pk;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;   // ready for the next item
      }
      // the wave reads back only what its own lanes wrote
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int qq = lane + k * 64;
        const int rw = qq >> 3, ch = qq & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + rw * SROW + ch * 8);
        const int row = wm * 128 + 32 * i + rw, col = wn * 128 + 64 * h + ch * 8;
        const bool ok = row < it.m_valid && col < it.n_valid && !(TSPLIT && npieces > 0);
        const uint32_t vo = ok ? (uint32_t)((row * a.c_ld + col) * 2) : kOOB;
        i32x4 d;
        d[0] = (int)v.x;
        d[1] = (int)v.y;
        d[2] = (int)v.z;
        d[3] = (int)v.w;
        __builtin_amdgcn_raw_buffer_store_b128(d, cr, (int)vo, 0, kPolicyStream);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      G256_FENCE();   // one pass's values at a time
    }
  };

  // ---- split dynamic-K tiles: partials and the last-arrival combine ----
  // Partial tiles in the MFMA register layout, a 64 KB region per wave: 16
  // bytes per lane and element quad, a 1 KB block per (i, j, q), the block
  // offset in the instruction's scalar offset.  Stores and loads are
  // coherent at device scope (sc1), so no cache-wide writeback is needed: a
  // wait for the stores orders them before the counter update, and loads
  // after it cannot hit stale lines.
  auto part_store = [&](const __amdgpu_buffer_rsrc_t& r, const Item& it) __attribute__((always_inline)) {
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = wm * 128 + 32 * i + (ln & 31) < it.m_valid;
      const uint32_t vo = ok ? (uint32_t)(ln * 16) : kOOB;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          i32x4 v;
          v[0] = __float_as_int(acc[i][j][4 * q]);
          v[1] = __float_as_int(acc[i][j][4 * q + 1]);
          v[2] = __float_as_int(acc[i][j][4 * q + 2]);
          v[3] = __float_as_int(acc[i][j][4 * q + 3]);
          __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)vo, ((i * 4 + j) * 4 + q) * 1024, kPolicyDevice);
        }
    }
  };
  // A piece of a split tile: store the partial, count the arrival; returns
  // true for the last piece to arrive, which then writes the tile from the
  // partials (combine, then the epilogue).  The accumulators are zero
  // afterwards.
  auto dk_arrive = [&](const Item& it) __attribute__((always_inline)) -> bool {
    int32_t* flag = reinterpret_cast<int32_t*>(tab.scratch);
    part_store(slot_rsrc(it.slot() + it.piece()), it);
    zero_acc();
    wait_vm_all();   // this wave's partial has reached the coherence point
    lds_sync();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(a.sk_ctr + it.ctr(), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == it.pieces() - 1;
      if (last) __hip_atomic_store(a.sk_ctr + it.ctr(), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *flag = last;
    }
    lds_sync();
    const bool last = uni(*flag) != 0;
    lds_sync();   // every wave has read the flag before the next use of the word
    return last;
  };

  // A split last-round tile, written by the last of its pieces to arrive
  // (after its item loop: the accumulators are free, no transfer is in
  // flight): every output element is the sum, in piece order, of the
  // pieces' partials in slots slot0 .. slot0 + P - 1, scaled as the
  // epilogue scales, rounded to bf16 and stored 4 columns at a time.  Each
  // wave takes the 128 x 128 region its own partials hold; per round, two
  // 32 x 32 blocks of up to four pieces are in flight (a load past the last
  // piece is out of range and reads zeros, and adding zero to a sum that
  // started at +0 changes no bit).
  auto tail_out = [&](const Item& it) __attribute__((always_inline)) {
    const int P = it.pieces(), slot0 = it.slot();
    uint16_t* C = reinterpret_cast<uint16_t*>(a.C) + (int64_t)it.g * a.c_gs + it.rowbase * a.c_ld + it.n0;
    int ln = threadIdx.x & 63;   // (an opaque copy: nothing lane-derived is held across the k-loop for this)
    asm volatile("" : "+v"(ln));
    const int l31 = ln & 31, hi = ln >> 5;
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + 32 * i + l31;
      const bool rok = row < it.m_valid;
      const uint32_t pvo = rok ? (uint32_t)(ln * 16) : kOOB;
      float rs = 1.f;
      if constexpr (SCALED) {
        const float v = rok ? a.sa[it.rowbase + row] : 0.f;
        rs = v != 0.f ? 1.f / v : 0.f;
      }
#pragma unroll 1
      for (int j = 0; j < 4; j += 2) {
        float sm[2][4][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) sm[jj][q][c] = 0.f;
        for (int p0 = 0; p0 < P; p0 += 4) {
          i32x4 ld[4][2][4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const __amdgpu_buffer_rsrc_t r = slot_rsrc(slot0 + p0 + u);
            const int vo = (int)(p0 + u < P ? pvo : kOOB);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                ld[u][jj][q] = __builtin_amdgcn_raw_buffer_load_b128(r, vo, ((i * 4 + j + jj) * 4 + q) * 1024,
                                                                     kPolicyDevice);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) sm[jj][q][c] += __int_as_float(ld[u][jj][q][c]);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * 128 + 32 * (j + jj) + 8 * q + 4 * hi;
            if (!rok || col >= it.n_valid) continue;   // (column counts are multiples of 8)
            float v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              v[c] = sm[jj][q][c];
              if constexpr (SCALED) {
                const float w = a.sb[(int64_t)it.g * a.Nout + it.n0 + col + c];
                v[c] = (v[c] * (w != 0.f ? 1.f / w : 0.f)) * rs;
              }
            }
            uint2 pk;
            pk.x = pack_bf16x2_hw(v[0], v[1]);
            pk.y = pack_bf16x2_hw(v[2], v[3]);
            *reinterpret_cast<uint2*>(C + (int64_t)row * a.c_ld + col) = pk;
          }
      }
    }
  };

  // ---- main loop ----
  // prologue: the first NS k-steps fill every stage
#pragma unroll
  for (int u = 0; u < NS; ++u) load_step(u);
  wait_vm_sync<(NS - 1) * LPW>();   // B(0)
  int stage = 0;                    // stage of the compute cursor's k-step
  int64_t ck = 0;                   // compute cursor: the workgroup's ck-th item
  int64_t cw = item_of(0);
  Item ci = fetch(cw);
  int cseq = 0;                     // items finished by the compute cursor
  bool tail_last = false;           // the workgroup is the last piece of a split last-round tile
  Frag256<ELEM> F0, F1;
#pragma unroll
  for (int n = 0; n < NREAD; ++n) read_one(F0, 0, 0, n);
  G256_FENCE();
  zero_acc();

  // One k-step on cur (its first sub-step's fragments); the next k-step's
  // first fragments end up in nxt (bf16: back in cur), except after an
  // item's last k-step.
  auto kstep = [&](Frag256<ELEM>& cur, Frag256<ELEM>& nxt, auto last_c, auto live_c) __attribute__((always_inline)) {
    const int st = stage;
    if constexpr (KSUB == 2) {
      inner_sub(cur, nxt, st, live_c);
      boundary_sub(nxt, cur, st, last_c, live_c);
    } else {
      boundary_sub(cur, nxt, st, last_c, live_c);
    }
    stage = st + 1 == NS ? 0 : st + 1;
  };
  // Dynamic-K: a k-step that the group's row range cuts (its first and
  // last) holds bytes of the neighbouring groups in the 16-byte chunks that
  // straddle the range's ends; they are cleared in the fragments before the
  // MFMAs.  A lane's fragment covers contraction bytes 32 (lane / 32) + 0..31
  // of the k-step.
  auto edge_mask = [&](Frag256<ELEM>& f, int s) __attribute__((always_inline)) {
    if constexpr (DK) {
      const int64_t cb = ci.c_begin + (int64_t)s * BK;
      const int64_t lo64 = ci.c_lo - cb, hi64 = ci.c_hi - cb;
      const int mlo = lo64 < 0 ? 0 : (lo64 > BK ? BK : (int)lo64);
      const int mhi = hi64 < 0 ? 0 : (hi64 > BK ? BK : (int)hi64);
      if (mlo > 0 || mhi < BK) {
        int ln = threadIdx.x & 63;
        asm volatile("" : "+v"(ln));
        const int k0 = 32 * (ln >> 5);
        uint32_t m[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) m[d] = byte_range_mask(mlo - k0 - 4 * d, mhi - k0 - 4 * d);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int d = 0; d < 8; ++d) {
            f.a[x][d] = (int)((uint32_t)f.a[x][d] & m[d]);
            f.b[x][d] = (int)((uint32_t)f.b[x][d] & m[d]);
          }
      }
    }
  };
  // every k-step of the item but the last refills the stage it used
  auto item_steps = [&](auto live_c) __attribute__((always_inline)) {
    const int nst = ci.nsteps;
    if constexpr (KSUB == 2) {
      for (int s = 0; s + 1 < nst; ++s) kstep(F0, F1, BoolConst<false>{}, live_c);
    } else {
      // e4m3: one sub-step per k-step, fragments alternate between F0 and F1
      int s = 0;
      for (; s + 2 < nst; s += 2) {
        edge_mask(F0, s);
        kstep(F0, F1, BoolConst<false>{}, live_c);
        edge_mask(F1, s + 1);
        kstep(F1, F0, BoolConst<false>{}, live_c);
      }
      if (s + 1 < nst) {
        edge_mask(F0, s);
        kstep(F0, F1, BoolConst<false>{}, live_c);
        F0 = F1;   // once per item
      }
    }
    const int stl = stage;   // the last k-step's stage
    edge_mask(F0, nst - 1);
    kstep(F0, F1, BoolConst<true>{}, live_c);
    return stl;
  };
  for (;;) {
    // a wave whose quadrant has no valid row or column (the bottom half of a
    // group's last row tile, the right half of a last column tile) skips its
    // MFMAs.  bf16 without the SiLU*mul epilogue only: there a second copy of
    // the k-loop costs registers the epilogue needs (spills), and the e4m3
    // kernels measured slower with it (their registers are laid out anew).
    int st_last;
    if constexpr (SWIGLU || ELEM != EL_BF16) {
      st_last = item_steps(BoolConst<true>{});
    } else {
      const bool live = wm * 128 < ci.m_valid && wn * 128 < ci.n_valid;
      st_last = live ? item_steps(BoolConst<true>{}) : item_steps(BoolConst<false>{});
    }
    // the last k-step's stage holds the epilogue's staging, then its refill
    bool write = true;
    int npieces = 0;
    if constexpr (PIECES) {
      if (ci.pieces() > 1) {
        write = dk_arrive(ci);
        npieces = ci.pieces();
      }
    }
    if constexpr (TSPLIT) tail_last = write && npieces > 0;
    if (write) epilogue(st_last, ci, cseq % NSCB, npieces, ci.slot());   // (leaves the accumulators zeroed)
    if (dyn) grab(ck + 7);
    lds_sync();
    load_step(st_last);
    const int64_t nw = item_of(++ck);
    if (nw < 0) break;
    cw = nw;
    ci = fetch(cw);
    ++cseq;
    // the next item's first fragments (its first k-step's stage landed at
    // the barrier of the last k-step)
#pragma unroll
    for (int n = 0; n < NREAD; ++n) read_one(F0, stage, 0, n);
    G256_FENCE();
  }
  wait_vm_all();   // no LDS-DMA transfer may outlive the workgroup
  if constexpr (TSPLIT) {
    if (tail_last) tail_out(ci);
  }
  // every request of this workgroup precedes its exit count, so the last to
  // count has seen all requests done: the counters start at zero again
  queue_exit();
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
template <bool B_KC, int ELEM, int EPI, int KIND>
static hipError_t launch_256(const GemmArgs& a, hipStream_t stream) {
  const int bne = EPI == EPI_SWIGLU ? 128 : 256;
  const int64_t work = KIND == DYNAMIC_K ? (int64_t)a.E * cdiv(a.Mout, 256) * cdiv(a.Nout, 256)
                                         : fixed_m_capacity(a.total_rows, a.E, 256) * cdiv(a.Nout, bne);
  if (work <= 0) return hipSuccess;
  auto kern = gmm256_kernel<B_KC, ELEM, EPI, KIND>;
  static int configured = 0;
  if (configured == 0) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       table_lds_bytes(kMaxExperts));
    if (e != hipSuccess) return e;
    configured = 1;
  }
  const int64_t slots = device_cu_count();
  const int grid = (int)(work < slots ? work : slots);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), (size_t)table_lds_bytes(a.E), stream, a);
  return hipGetLastError();
}

bool gemm256_eligible(const GemmLaunch& L, const GemmArgs& a) {
  const int64_t cus = device_cu_count();
  if (L.kind == DYNAMIC_K) {
    // e4m3 dW: enough tiles for a few rounds on every CU, and groups of 512
    // rows on average (8 k-steps per tile)
    if (L.elem != EL_FP8 || !L.a_kc || !L.b_kc) return false;
    const int64_t tiles = (int64_t)a.E * cdiv(a.Mout, 256) * cdiv(a.Nout, 256);
    return tiles >= 2 * cus && a.total_rows >= (int64_t)a.E * 512;
  }
  if (L.kind != FIXED_M || !L.a_kc) return false;
  if (L.elem == EL_FP8 && !L.b_kc) return false;
  if (L.elem != EL_BF16 && L.elem != EL_FP8) return false;
  if (L.elem == EL_FP8 && a.gather != nullptr) return false;
  // enough 256 x 256 tiles for a few rounds on every CU, with long enough
  // contractions that a tile's pipeline fill is small beside its k-steps
  const int bne = L.swiglu ? 128 : 256;
  const int64_t tiles = fixed_m_capacity(a.total_rows, a.E, 256) * cdiv(a.Nout, bne);
  if (tiles < 2 * cus) return false;
  if (a.Kc < 1024) return false;
  // rows per group: 256-row tiles of groups under about 192 rows would be
  // mostly empty
  if (a.total_rows < (int64_t)a.E * 192) return false;
  return true;
}

hipError_t launch_gemm256(const GemmLaunch& L, const GemmArgs& a, hipStream_t stream) {
  if (L.elem == EL_BF16) {
    if (L.swiglu) {
      if (L.b_kc) return launch_256<true, EL_BF16, EPI_SWIGLU, FIXED_M>(a, stream);
      return launch_256<false, EL_BF16, EPI_SWIGLU, FIXED_M>(a, stream);
    }
    if (L.b_kc) return launch_256<true, EL_BF16, EPI_NONE, FIXED_M>(a, stream);
    return launch_256<false, EL_BF16, EPI_NONE, FIXED_M>(a, stream);
  }
  if (L.kind == DYNAMIC_K) return launch_256<true, EL_FP8, EPI_GROUP, DYNAMIC_K>(a, stream);
  return launch_256<true, EL_FP8, EPI_ROW_COL, FIXED_M>(a, stream);
}

}  // namespace mg
