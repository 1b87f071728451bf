// F8I4 grouped GEMM for sparse M (K2, int4 variant), gfx950.
//
// FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse M": fp8 activations
// times int4 weights, launched only over the problems that have rows
// (min(total_M, groups)), so a single routed token among 128 experts costs
// about what one expert costs.  Here the fixed-M work list from the device
// builder (32-row tiles) times 32-column slices of N forms the work items;
// empty experts never appear in it.
//
// The work is bound by streaming the int4 weights.  Each wave moves them
// into its own LDS buffers by LDS-DMA, whole 128-byte lines of a column (two
// K chunks) per lane group, so every load instruction covers 8 full lines,
// not a 32-byte piece of 32 lines; the 16-byte slots of a line are XOR-
// swizzled by the column so that the fragment reads below hit distinct
// banks.  A fragment read gives each lane the layout of
// v_mfma_scale_f32_32x32x64_f8f6f4 (lane l: output column l % 32, a run of
// 32 consecutive k); each nibble becomes the e4m3 code of the same integer
// (exact: -8..7 are e4m3 values) with two byte permutes, and the fp8 MFMA
// runs per 128-long K chunk into a fresh accumulator that is then scaled by
// that chunk's bf16 weight scale (keeping the dequantization exact) and
// added to the running sum.
// The waves of a workgroup (8 for contractions of 64 or more chunks, else 4)
// split K.  When the items are too few to give every slot of the grid one
// (one or two routed rows over a narrow N), K is also split across
// workgroups: each piece stores its fp32 partial tile in the workspace, and
// the last piece to arrive adds them all in piece order (the same bits
// whatever the arrival order) and writes the output.  Each wave requests the
// operands of its next two chunks (a line per column) before it computes the
// current two; the activation and scale loads' offsets are opaque to the
// compiler, which would otherwise branch around the out-of-range loads and
// drain every load in flight.  The partial tiles are summed in LDS (the
// weight buffers, free after the K loop) in wave order, divided by the row
// scale of the activations and rounded to bf16.
#include "gemm_dev.h"

namespace mg {

// e4m3 codes of the integers 0..7 and of -8..-1 (by nibble & 7).
constexpr uint32_t kPosLo = 0x44403800u;   // 0, 1, 2, 3  -> 00 38 40 44
constexpr uint32_t kPosHi = 0x4E4C4A48u;   // 4, 5, 6, 7  -> 48 4A 4C 4E
constexpr uint32_t kNegLo = 0xCACCCED0u;   // -8,-7,-6,-5 -> D0 CE CC CA
constexpr uint32_t kNegHi = 0xB8C0C4C8u;   // -4,-3,-2,-1 -> C8 C4 C0 B8

// Four bytes holding nibble values 0..15 -> their four e4m3 codes: one byte
// permute into the table of 0..7, one into that of -8..-1, and a byte mask
// from bit 3 to choose between them.
__device__ inline uint32_t nibble_bytes_to_e4m3(uint32_t x) {
  const uint32_t idx = x & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(kPosHi, kPosLo, idx);
  const uint32_t neg = __builtin_amdgcn_perm(kNegHi, kNegLo, idx);
  const uint32_t s = (x >> 3) & 0x01010101u;
  const uint32_t m = (s << 8) - s;   // 0xFF in the bytes whose bit 3 is set
  return (pos & ~m) | (neg & m);
}

// 16 bytes = 32 nibbles (k ascending, low nibble first) -> 32 e4m3 codes.
// Per 4-byte word: the low nibbles (even k) and high nibbles (odd k) are
// converted as two words of bytes, then interleaved back into k order.
__device__ inline i32x8 i4x32_to_e4m3(const uint4& w) {
  const uint32_t src[4] = {w.x, w.y, w.z, w.w};
  i32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t even = nibble_bytes_to_e4m3(src[i] & 0x0F0F0F0Fu);
    const uint32_t odd = nibble_bytes_to_e4m3((src[i] >> 4) & 0x0F0F0F0Fu);
    r[2 * i] = (int)__builtin_amdgcn_perm(odd, even, 0x05010400u);       // k = 8i .. 8i+3
    r[2 * i + 1] = (int)__builtin_amdgcn_perm(odd, even, 0x07030602u);   // k = 8i+4 .. 8i+7
  }
  return r;
}

constexpr int F_BM = kF8I4RowTile;
constexpr int F_BN = 32;
constexpr uint32_t F_OOB = 0x80000000u;   // offset past any buffer: the load returns zeros
constexpr int F_DEVICE = 16;              // sc1: coherent at device scope (across XCDs)
constexpr int F_SPLIT_ROUNDS = 1;         // K pieces fill this many waves of the grid's slots

__device__ inline __amdgpu_buffer_rsrc_t f_rsrc(const void* base, int64_t bytes) {
  const int32_t nr = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nr, 0x00020000);
}


// One 128-long K chunk of a wave's work in the register path: the two
// 64-long halves of the weight fragment (int4, 16 bytes each), the chunk's
// bf16 weight scale, and the two matching fp8 activation fragments.
struct F8I4Chunk {
  i32x4 w[2];
  float sc;
  i32x8 x[2];
};

constexpr int F_LINE = 32 * 128;   // a wave's weight buffer: 32 columns x one 128-byte line (two K chunks)

// The register operands of one line step (two 128-long K chunks) of a
// wave's work: each chunk's bf16 weight scale and its two fp8 activation
// fragments (64 k each).  The weights of the step are in LDS.
struct F8I4Step {
  float sc[2];
  i32x8 x[2][2];
};

// The LDS-DMA asm takes its resource in SGPRs; it is workgroup-uniform.
__device__ inline i32x4 f_uni4(i32x4 r) {
  i32x4 u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

// F_WAVES waves per workgroup, each owning a contiguous run of K chunks: 8
// for long contractions (many chunks per wave to keep streaming), 4
// otherwise (less reduction work per tile).  LDSW: the weights go through
// LDS by DMA (4 waves: at 124-149 VGPRs the 8-wave workgroup would lose half
// its occupancy to the extra activation registers, and measured slower),
// else each lane loads its own column's fragments into registers.
template <int F_WAVES, bool LDSW>
__global__ void __launch_bounds__(F_WAVES * 64) f8i4_kernel(GemmArgs a) {
  // LDSW: two weight buffers per wave; after the K loop the same memory
  // holds the cross-wave reduction
  constexpr int WL_BYTES = LDSW ? F_WAVES * 2 * F_LINE : F_WAVES * F_BM * F_BN * 4;
  __shared__ __attribute__((aligned(16))) uint8_t wl[WL_BYTES];
  static_assert(WL_BYTES >= F_WAVES * F_BM * F_BN * 4, "the reduction fits the weight buffers");
  float(*red)[F_BM * F_BN] = reinterpret_cast<float(*)[F_BM * F_BN]>(wl);
  __shared__ int s_last;
  __shared__ float s_rs[F_BM];   // the tile's activation row scales
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int K = a.Kc;
  const int N = a.Nout;
  const int nchunk = K / 128;
  extern __shared__ __attribute__((aligned(16))) uint8_t table_lds[];
  const GroupTable tab = carve_table(table_lds, a.E);
  const int err = build_group_table(a.sizes, a.E, a.total_rows, F_BM, false, tab);
  if (err != 0 && blockIdx.x == 0 && tid == 0 && a.err != nullptr) *a.err = err;
  const int n_tiles = (int)cdiv(N, F_BN);
  const int64_t items = (int64_t)tab.tstart[a.E] * n_tiles;
  // every operand through a buffer descriptor: a lane outside the tile (row
  // past the group, column past N, chunk past the wave's range) reads zeros
  // (X: total_M * K bytes, below 2^31 by the host's checks; the weights and
  // their scales get one descriptor per expert, since all experts' int4
  // weights together may pass 2 GiB)
  const __amdgpu_buffer_rsrc_t xr = f_rsrc(a.A, a.total_rows * (int64_t)K);
  const __amdgpu_buffer_rsrc_t sar = f_rsrc(a.sa, a.total_rows * 4);
  const uint8_t* w4 = reinterpret_cast<const uint8_t*>(a.B);

  // K pieces per item: more than one only while the items leave slots idle,
  // each wave keeps at least two chunks, and every item has an arrival
  // counter of its own in the workspace
  int S = 1;
  if (items > 0 && items <= kSkMaxGrid && items * 2 <= (int64_t)gridDim.x * F_SPLIT_ROUNDS) {
    S = (int)((int64_t)gridDim.x * F_SPLIT_ROUNDS / items);
    const int smax = nchunk / (2 * F_WAVES);
    if (S > smax) S = smax;
    if (S < 1) S = 1;
  }
  const int64_t units = items * S;
  // chunk range of a wave: piece s, wave q -> run s * F_WAVES + q (through
  // LDS: of an even length, so that a wave's runs start on a line)
  int per = (nchunk + S * F_WAVES - 1) / (S * F_WAVES);
  if (LDSW) per = (per + 1) & ~1;
  const uint32_t wlds = lds_address(wl) + (uint32_t)(wave * 2 * F_LINE);
  const __amdgpu_buffer_rsrc_t pr = f_rsrc(a.sk_part, units * (int64_t)(F_BM * F_BN * 4));

  int64_t first = blockIdx.x;
  if ((gridDim.x & 7) == 0) first = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);

  for (int64_t u = first; u < units; u += gridDim.x) {
    const int64_t w = u / S;
    const int piece = (int)(u - w * S);
    const int jr = (piece * F_WAVES + wave) * per;
    const int j0 = jr < nchunk ? jr : nchunk;
    const int j1 = j0 + per < nchunk ? j0 + per : nchunk;
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
    // thread r < F_BM: the activation scale of the tile's row r, requested
    // before the K loop (older than every load the loop's waits count, so it
    // has landed by the first of them) and put in LDS after it, for the
    // output stores
    float rsv;
    {
      uint32_t so = tid < m_valid ? (uint32_t)((row0 + tid) * 4) : F_OOB;
      asm volatile("" : "+v"(so));
      rsv = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(sar, (int)so, 0, 0));
    }
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    if constexpr (LDSW) {
      const i32x4 wrw = f_uni4(make_rsrc_words(w4 + (int64_t)g * N * (K / 2), (int64_t)N * (K / 2)));
      const __amdgpu_buffer_rsrc_t sr = f_rsrc(a.s4 + (int64_t)g * nchunk * N, (int64_t)nchunk * N * 2);
      const uint32_t xrow = (uint32_t)((row0 + col) * (int64_t)K);
      const uint32_t srow = (uint32_t)((n0 + col) * 2);
      // weight transfers: instruction i covers columns 8 i .. 8 i + 7, lane l
      // the 16-byte slot l % 8 of column 8 i + l / 8's line, which holds part
      // (l % 8) ^ (column % 8) of the column's 128 bytes
      uint32_t dvo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dc = 8 * i + (lane >> 3);
        const int part = (lane & 7) ^ (dc & 7);
        dvo[i] = n0 + dc < N ? (uint32_t)((n0 + dc) * (K / 2) + part * 16) : F_OOB;
      }
      // the wave's lines: j0 is even whenever the range is not empty (its
      // length per is even); an empty range -- a wave past the last chunk,
      // whose j0 = j1 = nchunk may be odd -- has no lines
      const int L0 = j0 >> 1, L1 = j1 > j0 ? (j1 + 1) >> 1 : L0;

      // Requests every operand of line L into buffer b (zeros past the wave's
      // range): 4 weight transfers, then per chunk its scale and activations
      // (14 vector-memory operations per lane).  The LDS reads of the line
      // that last used buffer b are complete first.
      auto issue = [&](int L, int b, F8I4Step& st) __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const bool live = L < L1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dma16<kPolicyStream>(wrw, wlds + (uint32_t)(b * F_LINE + i * 1024),
                               live && dvo[i] != F_OOB ? dvo[i] + (uint32_t)L * 128u : F_OOB);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int j = 2 * L + c;
          const bool cl = live && j < j1;
          uint32_t so = (cl && col_ok) ? srow + (uint32_t)j * (uint32_t)N * 2u : F_OOB;
          asm volatile("" : "+v"(so));
          st.sc[c] = bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sr, (int)so, 0, 0));
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            uint32_t xo = (cl && row_ok) ? xrow + j * 128 + sh * 64 + half * 32 : F_OOB;
            asm volatile("" : "+v"(xo));
            const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xo, 0, 0);
            const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xo, 16, 0);
            st.x[c][sh] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      };
      // line L from buffer b: per chunk, the product into a fresh
      // accumulator, scaled by the chunk's weight scale and added to the
      // running sum; a chunk past the wave's range (the second half of its
      // last line) is skipped
      const uint8_t* wbuf = wl + wave * 2 * F_LINE;
      auto compute = [&](int L, int b, const F8I4Step& st) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (2 * L + c >= j1) break;
          f32x16 part;
#pragma unroll
          for (int v = 0; v < 16; ++v) part[v] = 0.f;
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            const int p = c * 4 + sh * 2 + half;
            const i32x4 w = *reinterpret_cast<const i32x4*>(wbuf + b * F_LINE + col * 128 + ((p ^ (col & 7)) << 4));
            const uint4 wq = make_uint4((uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]);
            const i32x8 bf = i4x32_to_e4m3(wq);
            part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(st.x[c][sh], bf, part, 0, 0, 0, 127, 0, 127);
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] += part[v] * st.sc[c];
        }
      };

      // Two lines in flight: line L + 1's operands are requested before line L
      // is computed.  Before a line's fragments are read, only the next line's
      // 14 operations may still be in flight (loads retire in order).
      F8I4Step s0, s1;
      issue(L0, 0, s0);
      for (int L = L0; L < L1; L += 2) {
        issue(L + 1, 1, s1);
        asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
        compute(L, 0, s0);
        issue(L + 2, 0, s0);
        if (L + 1 < L1) {
          asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
          compute(L + 1, 1, s1);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t wr = f_rsrc(w4 + (int64_t)g * N * (K / 2), (int64_t)N * (K / 2));
      const __amdgpu_buffer_rsrc_t sr = f_rsrc(a.s4 + (int64_t)g * nchunk * N, (int64_t)nchunk * N * 2);
      const uint32_t wrow = (uint32_t)((n0 + col) * (K / 2));
      const uint32_t xrow = (uint32_t)((row0 + col) * (int64_t)K);
      const uint32_t srow = (uint32_t)((n0 + col) * 2);

      // Requests every operand of chunk j (zeros past the wave's range).  The
      // weights keep the default cache policy although they are read once: a
      // lane's 16 bytes are a quarter of a 64-byte run whose 128-byte line the
      // next chunk reads too, and non-temporal loads fetched such lines from
      // HBM twice (measured: 1.9 -> 3.0 TB/s at 16 routed rows over 128
      // experts).
      auto load = [&](int j, F8I4Chunk& c) {
        const bool live = j < j1;
        // k = 128 j + 64 s + 32 half .. +32  ->  weight bytes (128 j + 64 s + 32 half) / 2
        uint32_t wo = (live && col_ok) ? wrow + j * 64 + half * 16 : F_OOB;
        asm volatile("" : "+v"(wo));   // opaque: no per-lane branch around the loads
        c.w[0] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)wo, 0, 0);
        c.w[1] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)wo, 32, 0);
        uint32_t so = (live && col_ok) ? srow + (uint32_t)j * (uint32_t)N * 2u : F_OOB;
        asm volatile("" : "+v"(so));
        c.sc = bf16_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sr, (int)so, 0, 0));
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          uint32_t xo = (live && row_ok) ? xrow + j * 128 + sh * 64 + half * 32 : F_OOB;
          asm volatile("" : "+v"(xo));
          const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xo, 0, 0);
          const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xo, 16, 0);
          c.x[sh] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      };
      // chunk product into a fresh accumulator, scaled by the chunk's weight
      // scale and added to the running sum
      auto compute = [&](const F8I4Chunk& c) {
        f32x16 part;
#pragma unroll
        for (int v = 0; v < 16; ++v) part[v] = 0.f;
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          const uint4 wq = make_uint4((uint32_t)c.w[sh][0], (uint32_t)c.w[sh][1], (uint32_t)c.w[sh][2],
                                      (uint32_t)c.w[sh][3]);
          const i32x8 bf = i4x32_to_e4m3(wq);
          part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(c.x[sh], bf, part, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] += part[v] * c.sc;
      };

      // Two chunks in flight: chunk j + 1's operands are requested before
      // chunk j is computed, so each wave keeps its next weight run streaming
      // while the MFMAs of the current one run.
      F8I4Chunk c0, c1;
      load(j0, c0);
      for (int j = j0; j < j1; j += 2) {
        load(j + 1, c1);
        compute(c0);
        load(j + 2, c0);
        if (j + 1 < j1) compute(c1);
      }
    }
    // every transfer of this wave has landed, and every wave is done with
    // its weight buffers, before they hold the reduction
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (tid < F_BM) s_rs[tid] = rsv;
    __syncthreads();

    // cross-wave reduction of the K slices, in a fixed order
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + 4 * half + (v & 3);
      red[wave][r * F_BN + col] = acc[v];
    }
    __syncthreads();
    if (S == 1) {
      for (int idx = tid; idx < F_BM * F_BN; idx += F_WAVES * 64) {
        const int r = idx / F_BN, c = idx % F_BN;
        if (r < m_valid && n0 + c < N) {
          float sum = red[0][idx];
#pragma unroll
          for (int q = 1; q < F_WAVES; ++q) sum += red[q][idx];
          const float y = sum * (1.f / s_rs[r]);
          reinterpret_cast<uint16_t*>(a.C)[(row0 + r) * a.c_ld + n0 + c] = (uint16_t)f32_to_bf16_rne(y);
        }
      }
    } else {
      // this piece's partial tile -> workspace slot u (item w's pieces are
      // slots w * S .. w * S + S - 1)
      for (int idx = tid; idx < F_BM * F_BN; idx += F_WAVES * 64) {
        const int r = idx / F_BN, c = idx % F_BN;
        if (r < m_valid && n0 + c < N) {
          float sum = red[0][idx];
#pragma unroll
          for (int q = 1; q < F_WAVES; ++q) sum += red[q][idx];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(sum), pr, (int)((u * (F_BM * F_BN) + idx) * 4), 0,
                                                F_DEVICE);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the partial has reached the coherence point
      __syncthreads();
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(a.sk_ctr + w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == S - 1;
        if (last) __hip_atomic_store(a.sk_ctr + w, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        for (int idx = tid; idx < F_BM * F_BN; idx += F_WAVES * 64) {
          const int r = idx / F_BN, c = idx % F_BN;
          if (r < m_valid && n0 + c < N) {
            float sum = 0.f;
            for (int q = 0; q < S; ++q) {
              const float v = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                  pr, (int)(((w * S + q) * (F_BM * F_BN) + idx) * 4), 0, F_DEVICE));
              sum = q == 0 ? v : sum + v;
            }
            const float y = sum * (1.f / s_rs[r]);
            reinterpret_cast<uint16_t*>(a.C)[(row0 + r) * a.c_ld + n0 + c] = (uint16_t)f32_to_bf16_rne(y);
          }
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_f8i4(const GemmArgs& a, int64_t cap_entries, hipStream_t stream) {
  const int64_t max_items = cap_entries * cdiv(a.Nout, F_BN);
  if (max_items <= 0) return hipSuccess;
  // the register budget allows 4 waves per SIMD: 2 workgroups of 8 waves or
  // 4 of 4 waves per CU, with as many again queued behind them
  const bool wide = a.Kc / 128 >= 64;
  const int64_t slots = (int64_t)device_cu_count() * (wide ? 4 : 8);
  // The grid follows the host's bound on the items (the capacity of the
  // sorted rows), so K pieces appear where the real items are fewer than
  // half of it: routed decode steps, whose sorted buffer has room for every
  // expert.  A grid widened for pieces beyond that bound measured slower (a
  // routed row over 128 experts, K=5120, N=8192: 19.4 -> 26.8 us).
  const int grid = (int)(max_items < slots ? max_items : slots);
  if (wide)
    hipLaunchKernelGGL((f8i4_kernel<8, false>), dim3(grid), dim3(8 * 64), (size_t)table_lds_bytes(a.E), stream, a);
  else
    hipLaunchKernelGGL((f8i4_kernel<4, true>), dim3(grid), dim3(4 * 64), (size_t)table_lds_bytes(a.E), stream, a);
  return hipGetLastError();
}

}  // namespace mg
