// Device helpers shared by the grouped-GEMM kernels (gmm.hip, gmm256.hip):
// buffer resources, LDS-DMA transfers and the explicit waits that order
// them, fp8 fragment byte masks, and the work items of a launch.
#pragma once

#include "kernels.h"
#include "worklist.h"

namespace mg {

// ---------------------------------------------------------------------------
// Buffer resources and LDS DMA.  For every work item and operand the
// workgroup builds a buffer resource (in SGPRs) whose base is the tile origin
// at the current k-step and whose size ends where the operand's valid
// contraction range ends, so rows past a group's end read as zeros with no
// per-load arithmetic.  A lane whose chunk lies outside the tile's valid rows
// or columns gets an offset past any buffer size; the DMA then writes zeros.
// ---------------------------------------------------------------------------
constexpr uint32_t kOOB = 0x80000000u;   // offset no buffer below 2 GiB reaches
constexpr int kBufFlags = 0x00020000;    // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t nr = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nr, kBufFlags);
}

// The same descriptor as four words, for the LDS-DMA asm below: base address
// (48 bits, stride 0), size in bytes, raw-buffer flags.
__device__ inline i32x4 make_rsrc_words(const void* base, int64_t bytes) {
  const int32_t nr = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)p;
  r[1] = (int)((uint32_t)(p >> 32) & 0xFFFFu);
  r[2] = nr;
  r[3] = kBufFlags;
  return r;
}

// Cache policy: operands read exactly once (the weights of a fixed-M bf16
// product whose expert has a single row tile) are loaded non-temporal;
// measured on MI355X, a pure stream runs at ~7.0 TB/s that way against
// ~4.8 TB/s with the default policy.  Operands that other tiles re-read --
// the weights of an expert with several row tiles, which the raster order
// hands to workgroups of one XCD at the same time -- keep the default
// policy so that they are fetched once into L2.
constexpr int kPolicyCached = 0;
constexpr int kPolicyStream = 2;   // nt
constexpr int kPolicyDevice = 16;  // sc1: coherent at device scope (across XCDs)

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ inline uint32_t lds_address(uint8_t* p) { return (uint32_t)(uintptr_t)(lds_void_t*)p; }

// 16 bytes per lane from global memory to LDS: lane l writes lds + 16 l (lds
// is an LDS byte address, the same in all lanes of the wave).  Written as
// asm rather than the compiler builtin: the compiler cannot tell which LDS
// stage a transfer targets, so with the builtin it drains every transfer in
// flight before each LDS read, which would serialise the K pipeline.  The
// waits that order these transfers are all explicit (wait_vm_sync).  M0,
// which supplies the LDS address, is restored before the statement ends.  A
// wait state separates the M0 write from the transfer that reads it (the
// GFX9-family hazard between an SALU write of M0 and an LDS DMA, which the
// compiler cannot see inside the asm).
template <int POL>
__device__ inline void dma16(const i32x4& r, uint32_t lds, uint32_t voff) {
  uint32_t save;
  if constexpr (POL == kPolicyStream) {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "v"(voff), "s"(lds), "s"(r)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(save)
                 : "v"(voff), "s"(lds), "s"(r)
                 : "memory");
  }
}

// A tile whose policy is kPolicyStream streams only when nt (a
// workgroup-uniform choice made per work item); otherwise it is cached.
template <int POL>
__device__ inline void dma_pol(const i32x4& r, uint32_t lds, uint32_t voff, bool nt) {
  if constexpr (POL == kPolicyStream) {
    if (nt) dma16<kPolicyStream>(r, lds, voff);
    else dma16<kPolicyCached>(r, lds, voff);
  } else {
    dma16<POL>(r, lds, voff);
  }
}

// 4 bytes per lane from global memory to LDS: lane l writes lds + 4 l.
__device__ inline void dma4(const i32x4& r, uint32_t lds, uint32_t voff) {
  uint32_t save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %1, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(save)
               : "v"(voff), "s"(lds), "s"(r)
               : "memory");
}

// Wait until at most VM vector-memory operations of this wave are still in
// flight and its LDS operations are done, then meet the other waves.  One asm
// statement, so the compiler moves no memory access across it and adds no
// full drain of the vector-memory counter (a release fence would, for the
// LDS-DMA transfers still in flight).
template <int VM>
__device__ inline void wait_vm_sync() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM) : "memory");
}
__device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ inline void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2_hw(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

template <bool B> struct BoolConst { static constexpr bool value = B; };

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uni64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Bytes [lo, hi) of a 4-byte word kept, the rest cleared (lo, hi relative to
// the word; any values).
__device__ inline uint32_t byte_range_mask(int lo, int hi) {
  const int l = lo < 0 ? 0 : (lo > 4 ? 4 : lo);
  const int h = hi < 0 ? 0 : (hi > 4 ? 4 : hi);
  if (h <= l) return 0u;
  uint32_t m = l >= 4 ? 0u : (0xFFFFFFFFu << (8 * l));
  if (h < 4) m &= (1u << (8 * h)) - 1u;
  return m;
}

// Keep the bytes of a 32-byte fp8 fragment whose contraction index k0 + byte
// lies in [lo, hi).
__device__ inline i32x8 mask_frag8(i32x8 v, int k0, int lo, int hi) {
#pragma unroll
  for (int d = 0; d < 8; ++d) v[d] = (int)((uint32_t)v[d] & byte_range_mask(lo - k0 - 4 * d, hi - k0 - 4 * d));
  return v;
}

// ---------------------------------------------------------------------------
// Work items.
// ---------------------------------------------------------------------------
struct Item {
  int g;            // group (expert)
  int64_t rowbase;  // first output row (token row for FIXED_M, row of C_g for DYNAMIC_K)
  int m_valid;      // rows of the tile that exist
  int n0, n_valid;  // first column, columns that exist
  int64_t c_lo, c_hi, c_begin;
  int nsteps;       // k-steps (>= 1; an empty dW group runs one all-zero step)
  int mt;           // FIXED_M: row tile (work-list entry) of the item
  bool b_stream;    // B is read by this item only (its expert has one row tile)
  // DYNAMIC_K pieces: (pieces the tile's contraction is cut into, 1 when
  // whole) << 16 | this item's piece; and, for a split tile, (its arrival
  // counter) << 16 | (the partial slot of its piece 0)
  int split;
  int sloc;
  __device__ int pieces() const { return split >> 16; }
  __device__ int piece() const { return split & 0xFFFF; }
  __device__ int ctr() const { return sloc >> 16; }
  __device__ int slot() const { return sloc & 0xFFFF; }
};

// Split plan of a dynamic-K launch: the first `groups` entries of the
// size-descending group order are cut into pieces[i] pieces along their
// contraction; items_before[i] counts the items of the split groups before
// order position i (items_before[groups] = all split items).
constexpr int kDkMaxSplitGroups = 16;
struct DkSplit {
  int32_t groups;
  int32_t pieces[kDkMaxSplitGroups];
  int32_t items_before[kDkMaxSplitGroups + 1];
  int32_t slot_before[kDkMaxSplitGroups + 1];
};

// Work item w.  Work-item counts stay below 2^31 (the host bounds every
// operand below 2 GiB), so the index arithmetic is 32-bit.  A fixed-M item
// in the same row tile as `prev` reuses its group lookup.
template <int BM, int BN, int KIND, int ELEM, int BK, bool SPLIT, uint32_t RM = 12>
__device__ inline Item get_item(const GemmArgs& a, const GroupTable& tab, int64_t w64, int n_tiles, int m_tiles_dk,
                                const Item* prev, const DkSplit& sp) {
  Item it;
  it.split = 1 << 16;
  it.sloc = 0;
  const uint32_t w = (uint32_t)w64;
  int nt;
  if (KIND == FIXED_M) {
    // Items run group by group; inside a group, in blocks of up to RM
    // row tiles, column tile outermost: the workgroups of one XCD, which take
    // consecutive items at the same time, then share each weight slice
    // among RM row tiles and each activation slice among the block's
    // column tiles.
    const uint32_t ntu = (uint32_t)n_tiles;
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {   // last group whose first item is <= w
      const int mid = (lo + hi + 1) >> 1;
      if ((uint32_t)tab.tstart[mid] * ntu <= w) lo = mid; else hi = mid - 1;
    }
    const int g = uni(lo);
    const int32_t t0 = uni(tab.tstart[g]);
    const uint32_t mtg = (uint32_t)(uni(tab.tstart[g + 1]) - t0);
    const uint32_t local = w - (uint32_t)t0 * ntu;
    // block height: the group's row tiles cut into the fewest blocks of at
    // most RM, all of one height but the last (with RM = 12, an expert
    // with 9 row tiles runs as one block, so its weights stream once)
    const uint32_t mtg1 = mtg > 0 ? mtg : 1;
    const uint32_t nblk = (mtg1 + RM - 1) / RM;
    const uint32_t rb = (mtg1 + nblk - 1) / nblk;
    const uint32_t blk = local / (rb * ntu);
    const uint32_t rem = local - blk * rb * ntu;
    const uint32_t mb = mtg - blk * rb < rb ? mtg - blk * rb : rb;
    nt = (int)(rem / mb);
    const int ml = (int)(blk * rb + (rem - (uint32_t)nt * mb));
    const int32_t eff = uni(tab.eff[g]);
    it.g = g;
    it.rowbase = (int64_t)uni(tab.off[g]) + (int64_t)ml * BM;
    it.m_valid = eff - ml * BM < BM ? eff - ml * BM : BM;
    it.c_lo = 0;
    it.c_hi = a.Kc;
    it.c_begin = 0;
    it.nsteps = (int)cdiv(a.Kc, BK);
    it.mt = t0 + ml;
    it.b_stream = mtg <= 1;
    (void)prev;
  } else {
    // items: the pieces of the split groups' tiles (piece outermost, so a
    // tile's pieces are dealt to different workgroups), then one item per
    // tile of every other group, in the size-descending group order
    const uint32_t per = (uint32_t)m_tiles_dk * (uint32_t)n_tiles;
    const int ns = SPLIT ? uni(sp.groups) : 0;
    const uint32_t nsplit = SPLIT ? (uint32_t)uni(sp.items_before[ns]) : 0u;
    uint32_t gi, rem;
    if (SPLIT && w < nsplit) {
      int q = 0;
      while (q + 1 < ns && (uint32_t)uni(sp.items_before[q + 1]) <= w) ++q;
      const uint32_t local = w - (uint32_t)uni(sp.items_before[q]);
      const uint32_t j = local / per;
      gi = (uint32_t)q;
      rem = local - j * per;
      const int pc = uni(sp.pieces[q]);
      it.split = (pc << 16) | (int)j;
      it.sloc = ((q * (int)per + (int)rem) << 16) | (uni(sp.slot_before[q]) + (int)rem * pc);
    } else {
      const uint32_t w2 = w - nsplit;
      gi = (uint32_t)ns + w2 / per;
      rem = w2 - (gi - (uint32_t)ns) * per;
    }
    const uint32_t mt = rem / (uint32_t)n_tiles;
    nt = (int)(rem - mt * (uint32_t)n_tiles);
    // every field is the same in all lanes (it comes from LDS reads of the
    // group table, which the compiler cannot see are uniform); say so, so the
    // buffer resources built from them live in SGPRs
    it.g = uni(tab.order[gi]);
    it.rowbase = (int64_t)mt * BM;
    it.m_valid = a.Mout - (int)it.rowbase;
    const int32_t off = uni(tab.off[it.g]), eff = uni(tab.eff[it.g]);
    it.c_lo = off;
    it.c_hi = (int64_t)off + eff;
    // fp8 operands are column-major codes read 16 rows at a time from a
    // 16-aligned row; bf16 operands are read one row at a time
    const int64_t start = (ELEM == EL_FP8) ? (it.c_lo & ~(int64_t)15) : it.c_lo;
    it.c_begin = eff > 0 ? start : it.c_hi;
    const int64_t span = it.c_hi - it.c_begin;
    it.nsteps = span > 0 ? (int)cdiv(span, BK) : 1;
    if (SPLIT && it.pieces() > 1) {   // piece j: k-steps [j n / S, (j + 1) n / S) of the n
      const int s0 = (int)((int64_t)it.piece() * it.nsteps / it.pieces());
      const int s1 = (int)((int64_t)(it.piece() + 1) * it.nsteps / it.pieces());
      it.c_begin += (int64_t)s0 * BK;
      it.nsteps = s1 - s0;
    }
    it.mt = (int)mt;
    it.b_stream = false;
  }
  it.n0 = nt * BN;
  it.n_valid = a.Nout - it.n0;
  return it;
}

}  // namespace mg
