// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include "common.h"

namespace mg {

// ---------------------------------------------------------------------------
// K1: argument builder
// ---------------------------------------------------------------------------
struct BuildArgs {
  const int32_t* sizes;
  int32_t E;
  int64_t total_M;
  int32_t bm;
  int32_t kind;         // 0: fixed-M entries, 1: dynamic-K entries
  int32_t* offs;        // [E+1]
  int32_t* count;       // [1]
  int32_t* entries;     // [cap][4]
};
hipError_t launch_build_worklist(const BuildArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// K2: grouped GEMM
//
// C(m, n) = sum_c A(m, c) * B_g(c, n), computed per work item.
//   FIXED_M   (forward, dX): rows m are token rows of a work-list entry
//             {g, row0, rows}; the contraction length Kc is fixed.
//   DYNAMIC_K (dW): output C_g is [Mout, Nout] per group; the contraction
//             runs over the group's token rows [offs[g], offs[g+1]).
// Operand element addresses (in elements):
//   A k-contiguous: A[m * a_ld + c]     A m-contiguous: A[c * a_ld + m]
//   B k-contiguous: B[g * b_gs + n * b_ld + c]
//   B n-contiguous: B[g * b_gs + c * b_ld + n]
//   C: C[g * c_gs + m * c_ld + n]  (c_gs = 0 for token-stacked outputs)
// ---------------------------------------------------------------------------
enum Kind { FIXED_M = 0, DYNAMIC_K = 1 };
enum Elem { EL_BF16 = 0, EL_FP8 = 1, EL_I4 = 2 };
// EPI_SWIGLU (bf16 fixed-M, B as [K, N]): the tile's 256 columns are 128
// gate columns n0.. and the matching 128 up columns I + n0.. of B, and the
// output is act[r, n] = silu(h[r, n]) * h[r, I + n] with h rounded to bf16
// first (I = the output width, Nout)
enum Epi { EPI_NONE = 0, EPI_ROW_COL = 1, EPI_GROUP = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  const void* A;
  int64_t a_ld;
  const void* B;
  int64_t b_ld;
  int64_t b_gs;
  void* C;
  int64_t c_ld;
  int64_t c_gs;
  // scales (fp8): FIXED_M: sa[row], sb[g * Nout + n]
  //               DYNAMIC_K: sa[g * Mout + m], sb[g * Nout + n]
  const float* sa;
  const float* sb;
  const uint16_t* s4;   // int4 chunk scales, bf16 [E][Kc/128][Nout]
  int32_t Mout;         // DYNAMIC_K: output rows per group
  int32_t Nout;
  int32_t Kc;           // FIXED_M contraction length
  int32_t E;
  int64_t total_rows;       // total_M: rows of the token-stacked operands
  const int32_t* sizes;     // device group sizes [E]
  int32_t* err;             // sticky error word (workspace header)
  // stream-K scratch (workspace): arrival counters [kSkMaxGrid] and two fp32
  // partial tiles per workgroup
  int32_t* sk_ctr;
  float* sk_part;
  // work-queue counters: items handed out (word 1 of the workspace header)
  // and finished workgroups (word 9); zero between calls: the last
  // workgroup of a launch that uses them resets them
  int32_t* wq;
  // FIXED_M, bf16, A contraction-contiguous only: when gather is set, row r
  // of A is row gather[r] / gather_div of the matrix at A (a token row
  // looked up through the token-sorted order), and a zero row when
  // gather[r] >= gather_limit (the padding sentinel)
  const int32_t* gather;
  int32_t gather_div;
  int32_t gather_limit;
};

struct GemmLaunch {
  int kind;      // Kind
  int elem;      // Elem of A (B is the same except EL_I4)
  bool a_kc, b_kc;
  bool swiglu = false;   // EPI_SWIGLU epilogue (bf16 fixed-M, b_kc false)
};

// Output tile of the GEMM kernel for a launch (rows x columns).
int gemm_tile_m(int kind);
int gemm_tile_n(int kind);

hipError_t launch_gemm(const GemmLaunch& L, const GemmArgs& a, hipStream_t stream);
// The 256 x 256-tile kernel (gmm256.hip) for large fixed-M launches;
// launch_gemm hands a launch to it when gemm256_eligible says so.
bool gemm256_eligible(const GemmLaunch& L, const GemmArgs& a);
// row-tile height of this thread's last launch_gemm (0 before the first)
int last_gemm_tile_m();
hipError_t launch_gemm256(const GemmLaunch& L, const GemmArgs& a, hipStream_t stream);
// The GEMM kernels read every operand's tile base unconditionally, so a
// DYNAMIC_K launch needs total_M > 0; with no rows, dW is a plain zero fill.
hipError_t launch_zero_fill(void* p, int64_t bytes, hipStream_t stream);
hipError_t launch_f8i4(const GemmArgs& a, int64_t max_items, hipStream_t stream);
constexpr int kF8I4RowTile = 32;

// ---------------------------------------------------------------------------
// K3/K4: fp8 quantizers, int4 weight quantizer
// ---------------------------------------------------------------------------
// src (optional): output row r quantizes x[src[r] / top_k], or a row of
// zeros where src[r] is not below n_pairs.
hipError_t launch_quant_rowwise(const uint16_t* x, int64_t rows, int32_t cols,
                                int64_t ld, uint8_t* q, float* s, hipStream_t stream,
                                const int32_t* src = nullptr, int32_t top_k = 1, int64_t n_pairs = 0);
// Per-group colwise (single or dual) in two launches.  Its workspace: a
// 256-byte header (word 0: the sticky error word) and 64 partial column
// maxima per (chunk slot, column block) at part_off; nothing in it needs
// initialising.
struct ColwiseLayout {
  int64_t slots;      // chunk slots per column block
  int64_t part_off;   // bytes
  int64_t total;      // bytes
  int64_t items;      // upper bound on a launch's work items
};
ColwiseLayout colwise_layout(int32_t G, int64_t rows, int32_t cols_a, int32_t cols_b);
hipError_t launch_quant_colwise(const uint16_t* a, int32_t cols_a, const uint16_t* b,
                                int32_t cols_b, const int32_t* sizes, int32_t G,
                                int64_t rows, int64_t ld, uint8_t* qa, float* sa, uint8_t* qb,
                                float* sb, void* ws, hipStream_t stream);
hipError_t launch_quant_int4(const uint16_t* w, int32_t E, int32_t K, int32_t N,
                             uint8_t* w4, uint16_t* sw, hipStream_t stream);

// ---------------------------------------------------------------------------
// K5-K7: permutation, activation, combine
// ---------------------------------------------------------------------------
int64_t perm_workspace_bytes(int64_t P, int32_t E);
hipError_t launch_moe_permute_ws(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                                 int32_t block_m, const uint16_t* x, int32_t hidden,
                                 int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp,
                                 int32_t* inv, int32_t* padded, uint16_t* x_sorted,
                                 int64_t cap, int64_t nblk, void* ws, hipStream_t stream);
hipError_t launch_moe_unpermute(const uint16_t* y, const int32_t* inv, const float* w,
                                int64_t T, int32_t k, int32_t hidden, uint16_t* out,
                                hipStream_t stream);
hipError_t launch_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t renorm, int32_t* ids,
                             float* wts, hipStream_t stream);
hipError_t launch_silu_mul(const uint16_t* h, int64_t rows, int32_t inter, uint16_t* act,
                           hipStream_t stream);
// act = silu(h[:, :inter]) * h[:, inter:] (bf16), then rowwise e4m3 of act:
// codes q [rows, inter], scales [rows]; act also written when non-null
hipError_t launch_silu_mul_quant(const uint16_t* h, int64_t rows, int32_t inter, uint16_t* act, uint8_t* q,
                                 float* scales, hipStream_t stream);

int device_cu_count();

}  // namespace mg
