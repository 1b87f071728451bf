// Shared device/host helpers for the gfx950 MoE grouped-GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

// ---------------------------------------------------------------------------
// Vector types used as MFMA operands.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;

// Workspace layout (bytes).  The header holds the sticky error word and
// the counters of a work-queue launch.
constexpr int64_t kWsHeader = 256;
constexpr int kWsErrorWord = 0;   // int32 index into the header
constexpr int kWsQueueWord = 1;   // work-queue counters: words 1 (items handed out), 9 (workgroups finished)
                                  // and 17-24 (items handed out of each XCD's run)
constexpr int kMinTileM = 16;     // smallest row tile any kernel uses

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Fixed-M work-list capacity: sum over groups of ceil(size/bm) is at most
// floor(total/bm) + (number of non-empty groups) <= floor(total/bm) + min(total, E).
__host__ __device__ inline int64_t fixed_m_capacity(int64_t total_M, int32_t E, int32_t bm) {
  return total_M / bm + (total_M < E ? total_M : E);
}

// Workspace layout (bytes):
//   [0, 256)            header: the sticky error word;
//   [256, 1280)         one int32 arrival counter per workgroup of a
//                       stream-K launch (zero between calls: the workgroup
//                       that consumes a counter resets it);
//   [1280, +64 MiB)     two fp32 partial output tiles per workgroup.
// Every work list lives in LDS (each kernel rebuilds it in its prologue), so
// the workspace does not grow with E or total_M.
constexpr int kSkMaxGrid = 256;                       // workgroups of a stream-K launch, at most
constexpr int64_t kSkPartBytes = 128 * 256 * 4;       // one fp32 partial tile (fixed-M tile)
constexpr int64_t kWsCounters = kWsHeader;
constexpr int64_t kWsPartials = kWsHeader + 4 * kSkMaxGrid;
constexpr int kWsZeroWords = (int)(kWsPartials / 4);  // words a fresh workspace must have zeroed

struct WsLayout {
  int64_t total;
};

constexpr int64_t kWsBytes = kWsPartials + 2 * (int64_t)kSkMaxGrid * kSkPartBytes;

__host__ __device__ inline WsLayout ws_layout(int32_t E, int64_t total_M) {
  (void)E;
  (void)total_M;
  WsLayout L;
  L.total = kWsBytes;
  return L;
}

// ---------------------------------------------------------------------------
// Number-format helpers.
// ---------------------------------------------------------------------------
__device__ inline float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------------------
// LDS tile addressing.  Tiles are stored with the contraction index
// contiguous: one 128-byte row per M (or N) index, made of eight 16-byte
// chunks.  The chunk position is XOR-swizzled with bits of the row so that
// both the MFMA fragment reads (32 consecutive rows, one chunk) and the
// transposing writes (rows 8 apart) spread over the banks.
// ---------------------------------------------------------------------------
__device__ inline int swz_chunk(int row, int chunk) { return chunk ^ ((row ^ (row >> 3)) & 7); }
__device__ inline int lds_off(int row, int chunk) { return row * 128 + swz_chunk(row, chunk) * 16; }

}  // namespace mg
