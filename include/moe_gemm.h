/*
 * moe_gemm.h -- C ABI of the MI355X (gfx950) MoE grouped-GEMM library.
 *
 * The library computes one matrix product per expert over a jagged,
 * routing-dependent number of token rows, as stated on the source pages:
 *
 *   [GG]  grouped_gemm PR "Support GPU-resident batch sizes": gmm(x, w,
 *         batch_sizes, trans_b) with the batch sizes resident on the device,
 *         its backward (gradient of out.sum()), and the review thread's
 *         dynamic-k problems (dW) sorted by k, descending, with the outputs of
 *         k = 0 problems zeroed.
 *   [F8I4] FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse M": fp8
 *         activations x int4 weights; kernel arguments cover only
 *         min(total_M, groups) problems so empty groups cost nothing.
 *   [FMOE] applied-ai issue "Column-major fused MoE": moe_align_block_size
 *         (token ids sorted by expert, padded to block_m), fused_moe_kernel
 *         (sorted_token_ids, expert_ids, top-k weights), silu_and_mul and the
 *         top-k weighted sum.
 *   [FP8] torchao commit "Optimize FP8 MoE backward pass: fused colwise kernel
 *         + AMD tuning": fused rowwise absmax + saturated fp8 cast, and the
 *         (dual) per-group colwise scales kernel with column-major output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is caller-owned DEVICE memory.  The library never
 *   allocates, frees or reads device memory on the host; nothing is copied
 *   device -> host and nothing synchronizes.  Work is enqueued on `stream`
 *   (a hipStream_t; NULL is the legacy default stream).
 * - bf16 tensors are IEEE bfloat16 bit patterns; fp8 is OCP E4M3 ("e4m3fn",
 *   max 448, no infinities); int4 is two's-complement nibbles.
 * - Group sizes are device int32 [E]; group g owns the consecutive rows
 *   [offs[g], offs[g+1]) of every token-stacked matrix, offs being the
 *   exclusive prefix sum.  total_M is the host-known row count of those
 *   matrices; the sizes must be >= 0 and sum to at most total_M.  Rows past
 *   the sum belong to no group and are left untouched in outputs.  A device
 *   violation (negative size, sum > total_M) is clamped so nothing is written
 *   out of bounds, and sets a sticky error word in the workspace
 *   (mg_workspace_error reads it back, synchronously; test use only).
 * - FP8 scales are fp32 quantization MULTIPLIERS: value = code / scale.
 * - Return value: MG_OK, or a negative status after which nothing has been
 *   enqueued; mg_last_error() then describes the problem (thread-local).
 *   Host-side checks: null pointers, sizes out of range, unsupported
 *   alignment, E > 1024, workspace too small.
 * - All calls are legal inside hipStreamBeginCapture / hipStreamEndCapture.
 */
#ifndef MOE_GEMM_H
#define MOE_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* mg_stream_t; /* hipStream_t */

enum {
  MG_OK = 0,
  MG_EINVAL = -1,        /* invalid argument */
  MG_EUNSUPPORTED = -2,  /* valid but unsupported shape/alignment */
  MG_EWORKSPACE = -3,    /* workspace missing or too small */
  MG_EHIP = -4           /* a HIP launch failed */
};

/* Largest number of experts/groups (one workgroup scans the sizes; [GG]
 * description: a single thread block, hence at most 1024 experts). */
#define MG_MAX_EXPERTS 1024

/* ------------------------------------------------------------------------ */
/* Workspace                                                                */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace that a grouped-GEMM call with these E and
 * total_M needs: a 256-byte header (the sticky error word, and the
 * counters of the work queue that the 256 x 256-tile dW kernel deals
 * unequal groups' tiles from: one shared, one per XCD, one of finished
 * workgroups), 256 arrival counters (one per split tile or
 * stream-K workgroup) and 64 MiB of fp32 partial output tiles (two
 * 128 x 256 tiles per workgroup of the 8-wave kernel, one 256 x 256 tile
 * per workgroup of the 4-wave kernel), about 64 MiB in all.  The work
 * lists themselves are built in LDS by every kernel's prologue.
 * Depends on host values only; the pointer must be 256-byte aligned.
 * A fresh workspace must be zeroed once before its first use (a
 * zero-filled allocation, or mg_workspace_clear); the GEMM calls (the
 * F8I4 call's K split included) leave the counters at zero again when they
 * finish.  Calls that share a workspace
 * must not overlap in time (enqueue them on one stream): the partial tiles
 * and counters of one call would be taken for another's. */
size_t mg_workspace_bytes(int32_t E, int64_t total_M);

/* Reads the sticky device error word of a workspace (hipMemcpy, blocking):
 * 0 = none, 1 = negative group size, 2 = sizes sum past total_M.  Also
 * reads a colwise quantizer workspace, whose first word is the same. */
int32_t mg_workspace_error(const void* ws);

/* Zeroes the workspace header (error word, work-queue counters) and the
 * arrival counters (enqueued on stream, by a fill kernel). */
int mg_workspace_clear(void* ws, mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Argument builder ([GG] review thread: a single-block scan of the batch    */
/* sizes fills the per-problem arguments on the device; [F8I4]: only         */
/* non-empty groups get work).                                               */
/* ------------------------------------------------------------------------ */

/* Work-list kinds. */
enum { MG_WL_FIXED_M = 0, MG_WL_DYNAMIC_K = 1 };

/* Runs the device builder on group_sizes and writes, to caller buffers:
 *   offs    int32 [E+1]  exclusive prefix sum (offs[E] = clamped total);
 *   count   int32 [1]    number of entries;
 *   entries int32 [cap][4]:
 *     MG_WL_FIXED_M: for each non-empty group g ascending, one entry per
 *       bm-row slice {g, first_row, rows (<= bm), 0};
 *       cap >= total_M / bm + min(total_M, E).
 *     MG_WL_DYNAMIC_K: all E groups ordered by size descending, ties by g
 *       ascending, {g, offs[g], size, 0}; cap >= E.
 * Every grouped-GEMM kernel runs this same builder in its prologue (bm =
 * its row tile: 128, or 32 for gmm_fwd_f8i4), so a call is one launch.
 * Errors: MG_EINVAL for null pointers, E outside [1, 1024], bm < 1, cap too
 * small for the bound above. */
int gmm_build_worklist(int32_t kind, const int32_t* group_sizes, int32_t E,
                       int64_t total_M, int32_t bm, int32_t* offs,
                       int32_t* count, int32_t* entries, int64_t cap,
                       mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* bf16 grouped GEMM ([GG] description: gmm(x, w, batch_sizes, trans_b)).    */
/* ------------------------------------------------------------------------ */

/* Forward: Y[r, :] = X[r, :] . W[g(r)] for every row r of group g.
 *   x  bf16 [total_M, K] row-major
 *   w  bf16 [E, K, N] (trans_b = 0) or [E, N, K] (trans_b = 1), contiguous
 *   y  bf16 [total_M, N] row-major; fp32 accumulation, round-to-nearest-even
 * K and N must be multiples of 8 (16-byte rows).  total_M = 0 is a no-op. */
int gmm_fwd(const void* x, const void* w, const int32_t* group_sizes,
            int32_t E, int64_t total_M, int32_t K, int32_t N, int32_t trans_b,
            void* y, void* ws, size_t ws_bytes, mg_stream_t stream);

/* gmm_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same product and kernels, with the workspace taken from a fixed
 * device array inside the library (64 MiB + 1280 bytes per device, held
 * from the first call on that device until the process ends) instead of a
 * caller's buffer.  The result is bit-identical to gmm_fwd's.
 *   x, w, group_sizes, E, total_M, K, N, trans_b, y: as for gmm_fwd.
 * The array's address on the current device (stream must belong to it) is
 * looked up on the first call there, which also enqueues a fill kernel on
 * `stream` that zeroes its counters; every call leaves them zero again.
 * The call allocates and frees nothing.  Every call on one device shares
 * that device's array: calls that overlap in time on one device (other
 * streams, other threads) race on it and must not be made.  The sticky
 * device error word lives in the array and is not readable through this
 * entry point; violations are still clamped.
 * Errors as gmm_fwd, plus MG_EWORKSPACE should a call need more scratch
 * than the array holds (the need depends on host values only), MG_EHIP if
 * the array's address cannot be found, MG_EUNSUPPORTED for a device index
 * of 64 or more. */
int gmm_fwd_noalloc(const void* x, const void* w, const int32_t* group_sizes,
                    int32_t E, int64_t total_M, int32_t K, int32_t N,
                    int32_t trans_b, void* y, mg_stream_t stream);

/* gmm_fwd over token-sorted rows, with the gather fused into the A-operand
 * load ([FMOE] fused_moe_kernel: the A rows of a block are found through
 * sorted_token_ids // top_k, so no sorted copy of x is made):
 *   y[r, :] = x[sorted_token_ids[r] / top_k, :] . W[g(r)]
 * for the rows r of the groups (group_sizes, normally moe_permute's
 * padded_group_sizes, summing to at most total_M); a row whose id is
 * >= T*top_k (moe_permute's padding sentinel) is a zero row.
 *   x                bf16 [T, K] row-major (the unsorted tokens)
 *   sorted_token_ids int32 [>= total_M], device (moe_permute's output)
 *   w, trans_b, y    as for gmm_fwd; y is bf16 [total_M, N], rows past the
 *                    groups untouched.
 * The result is bit-identical to gmm_fwd over moe_permute's x_sorted.
 * Errors as gmm_fwd, plus MG_EINVAL for T < 0, top_k < 1 or
 * T*top_k > 2^24, and MG_EUNSUPPORTED for T*K*2 bytes past 2 GiB. */
int gmm_fwd_gather(const void* x, int64_t T, const int32_t* sorted_token_ids,
                   int32_t top_k, const void* w, const int32_t* group_sizes,
                   int32_t E, int64_t total_M, int32_t K, int32_t N,
                   int32_t trans_b, void* y, void* ws, size_t ws_bytes,
                   mg_stream_t stream);

/* The expert FFN's first GEMM with SiLU-and-mul in its epilogue ([FMOE]
 * fused_moe: silu_and_mul of the gate and up halves of the first GEMM's
 * output, applied here before that output ever reaches memory):
 *   h[r, :]   = A[r, :] . W1[g(r)]          (fp32 accumulate, rounded to bf16)
 *   act[r, n] = bf16( silu(h[r, n]) * h[r, I + n] ),  silu(v) = v / (1 + e^-v)
 * with A[r, :] = x[sorted_token_ids[r] / top_k, :] (zero row for ids
 * >= T*top_k) when sorted_token_ids is non-NULL, else x[r, :].
 *   x     bf16 [T, K] (gathered) or [total_M, K] row-major
 *   w1    bf16 [E, K, 2I] (gate columns 0..I-1, up columns I..2I-1), or
 *         with trans_b, [E, 2I, K] (gate rows 0..I-1, up rows I..2I-1: the
 *         (E, N, K) weight layout of [FMOE] fused_moe_kernel)
 *   act   bf16 [total_M, I]; rows past the groups untouched
 * The same bits as gmm_fwd (or gmm_fwd_gather) into h followed by silu_mul
 * whenever neither launch splits a tile along K; where the stream-K tail
 * splits tiles, the split points differ (a tile here pairs gate and up
 * columns), so h may differ in its last bit before SiLU*mul.
 * Errors as gmm_fwd_gather; K and I must be multiples of 8. */
int gmm_fwd_silu_mul(const void* x, int64_t T, const int32_t* sorted_token_ids,
                     int32_t top_k, const void* w1, const int32_t* group_sizes,
                     int32_t E, int64_t total_M, int32_t K, int32_t I,
                     int32_t trans_b, void* act, void* ws, size_t ws_bytes,
                     mg_stream_t stream);

/* Backward of gmm_fwd for an upstream gradient dy [total_M, N]:
 *   dx[r, :] = dy[r, :] . W[g(r)]^T          (bf16 [total_M, K]; may be NULL)
 *   dw[g]    = X_g^T . dY_g                   (bf16, laid out like w; may be
 *              NULL).  The contraction runs over the group's own rows (a
 *              "dynamic-k" problem); an empty group's dw is exactly zero.
 * At least one of dx, dw must be non-NULL. */
int gmm_bwd(const void* dy, const void* x, const void* w,
            const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t K,
            int32_t N, int32_t trans_b, void* dx, void* dw, void* ws,
            size_t ws_bytes, mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* FP8 grouped GEMM ([FP8] commit message: rowwise-scaled fp8 operands for   */
/* the forward and dX, per-group colwise scales for dW).  Accumulation is    */
/* fp32 over e4m3 products; the epilogue divides by both scales and rounds   */
/* to bf16.                                                                  */
/* ------------------------------------------------------------------------ */

/* An fp8 stacked weight: code of element (e, c, j) -- c the contraction
 * index, j the output column -- at codes[e * expert_stride + j * ld + c]
 * (contraction index contiguous), with scale scales[e * J + j]. */
typedef struct mg_fp8_weight {
  const uint8_t* codes;
  const float* scales;
  int64_t ld;
  int64_t expert_stride;
} mg_fp8_weight;

/* Forward: Y[r, n] = sum_k (xq[r,k] / sx[r]) * (Wq(g,k,n) / sw[g,n]).
 *   xq  e4m3 [total_M, K] row-major, sx fp32 [total_M] (rowwise quantizer)
 *   w   codes of W(e,k,n) at e*expert_stride + n*ld + k, scales [E][N]
 *       (e.g. the colwise quantizer on W viewed [E*K, N] with E equal groups,
 *       its code rows ld bytes apart, gives that ld and expert_stride = K;
 *       unpadded rows, ld = E*K, read fastest here)
 *   y   bf16 [total_M, N]
 * K must be a multiple of 16 and N a multiple of 8; ld and expert_stride
 * multiples of 16. */
int gmm_fwd_fp8(const uint8_t* xq, const float* sx, const mg_fp8_weight* w,
                const int32_t* group_sizes, int32_t E, int64_t total_M,
                int32_t K, int32_t N, void* y, void* ws, size_t ws_bytes,
                mg_stream_t stream);

/* Backward with fp8 operands (either output may be NULL):
 *   dx[r,k] = sum_n (dyq[r,n]/sdy[r]) * (Wq(g,n,k)/sw[g,k])
 *       dyq e4m3 [total_M, N] rowwise with sdy [total_M]; w codes of W(e,k,n)
 *       at e*expert_stride + k*ld + n (contraction n contiguous), scales
 *       [E][K] (the rowwise quantizer on W viewed [E*K, N] gives ld = N,
 *       expert_stride = K*N);
 *   dw[g,k,n] = sum_{r in g} (xc[k,r]/sxc[g,k]) * (dyc[n,r]/sdyc[g,n])
 *       xc e4m3 column-major, xc[k,r] at xc + k*ldc + r, with sxc [E][K];
 *       dyc column-major, dyc[n,r] at dyc + n*ldc + r, with sdyc [E][N]
 *       (the dual per-group colwise quantizer); dw bf16 [E, K, N]; empty
 *       groups give zero.  Bytes of a row past total_M are never used.
 *   ldc the row stride of xc and dyc in bytes: a multiple of 16, at least
 *       total_M (ignored without dw or without rows).  A stride that is a multiple of a
 *       large power of two (98304 = 3 * 2^15 bytes, say) puts the 256 rows
 *       a tile reads on the same few HBM channels: an odd multiple of 256
 *       avoids that.
 * total_M must be a multiple of 16 when dw is requested. */
int gmm_bwd_fp8(const uint8_t* dyq, const float* sdy, const mg_fp8_weight* w,
                const uint8_t* xc, const float* sxc, const uint8_t* dyc,
                const float* sdyc, int64_t ldc, const int32_t* group_sizes, int32_t E,
                int64_t total_M, int32_t K, int32_t N, void* dx, void* dw,
                void* ws, size_t ws_bytes, mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* F8I4 grouped GEMM ([F8I4]: fp8 activations x int4 weights, sparse M).     */
/* ------------------------------------------------------------------------ */

/* Y[r,n] = (1/sx[r]) * sum_j sw[g,j,n] * sum_{k in chunk j} xq[r,k] * q(g,n,k)
 *   xq  e4m3 [total_M, K] row-major, sx fp32 [total_M]
 *   w4  int4 packed [E][N][K/2]; byte (e,n,i) holds k = 2i in its low
 *       nibble and k = 2i+1 in its high nibble
 *   sw  bf16 [E][K/128][N], one scale per 128-long chunk of K
 *   y   bf16 [total_M, N]
 * K must be a multiple of 128 and N a multiple of 8; K*N and
 * total_M*max(K, N) must stay below 2^31 (MG_EUNSUPPORTED otherwise).  Only
 * non-empty groups are visited.  When the (row tile, 32-column) items are
 * at most 256 and fill at most half the grid, K is split across workgroups:
 * fp32 partial tiles go to the workspace and one arrival counter per item
 * is used and left at zero, so the workspace rules above apply here too.
 * The last piece to arrive adds the partials in piece order, so results do
 * not depend on the arrival order. */
int gmm_fwd_f8i4(const uint8_t* xq, const float* sx, const uint8_t* w4,
                 const void* sw, const int32_t* group_sizes, int32_t E,
                 int64_t total_M, int32_t K, int32_t N, void* y, void* ws,
                 size_t ws_bytes, mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* FP8 quantizers ([FP8] commit message and colwise kernel).                 */
/* Per scaled block: amax = max |x|; t = fp32(448 / max(amax, 1e-12)) (the   */
/* division in fp64); scale s = 2^floor(log2 t) (t's mantissa cleared);      */
/* code = e4m3_rne(clamp(x * s, -448, 448)).                                 */
/* ------------------------------------------------------------------------ */

/* Rowwise: x bf16 [rows, cols] with row stride ld (elements, >= cols) ->
 * q e4m3 [rows, cols] contiguous, scales fp32 [rows].  cols % 8 == 0 and
 * ld % 8 == 0. */
int quantize_rowwise_fp8(const void* x, int64_t rows, int32_t cols, int64_t ld,
                         uint8_t* q, float* scales, mg_stream_t stream);

/* Rowwise of token rows in sorted order ([FMOE] docstring: fused_moe reads A
 * row sorted_id / top_k and masks the padding sentinel): output row r
 * quantizes x[sorted_token_ids[r] / top_k], and an entry that is not below
 * T * top_k (the sentinel) gives a row of zeros (codes 0, the scale of
 * amax 0), bit for bit what quantize_rowwise_fp8 gives for the rows
 * moe_permute gathers.
 *   x                 bf16 [T, cols] contiguous (may be NULL when T == 0)
 *   sorted_token_ids  int32 [rows] (moe_permute's sorted_token_ids)
 *   q                 e4m3 [rows, cols] contiguous, scales fp32 [rows]
 * cols % 8 == 0, top_k >= 1; MG_EINVAL for negative sizes or NULL
 * pointers, MG_EUNSUPPORTED for misaligned tensors (x 16-byte, q 8-byte). */
int quantize_rowwise_fp8_gather(const void* x, int64_t T, const int32_t* sorted_token_ids,
                                int32_t top_k, int64_t rows, int32_t cols, uint8_t* q,
                                float* scales, mg_stream_t stream);

/* Per-group colwise, single or dual: for each group g and column c of a
 * (and of b, if non-NULL), one scale over the group's rows.  Codes are
 * written column-major: qa[c * ld + r]; scales sa[g * cols_a + c].  b,
 * qb, sb are either all NULL (single tensor) or all set (both tensors share
 * the group sizes and row count).  Rows beyond the sizes' sum are not
 * written, nor are the bytes r in [rows, ld) of a code row; an empty group
 * gets the scales of amax 0.  cols % 8 == 0, cols <= 2^20;
 * 1 <= G <= MG_MAX_EXPERTS; rows < 2^31; rows <= ld < 2^32 (ld, the code
 * rows' stride in bytes, shared by qa and qb: see gmm_bwd_fp8's ldc for
 * the choice that keeps the fp8 dW off a few HBM channels).
 *
 * Two kernel launches.  Work is cut into (tensor, group, 64-column
 * block) sets.  A group of at most 256 rows is one chunk; a longer group's
 * chunks are its pieces of the global 256-row blocks (a group touching more
 * than 128 blocks gives each chunk several).  The first launch holds a
 * chunk in registers: a set of one chunk is quantized there from a single
 * read of its input, a chunk of a larger set leaves its partial column
 * maxima in the workspace.  The second launch reads those chunks again
 * (most recently read first, so partly from cache), takes the set's
 * maximum from the partials and writes their codes.
 *
 *   ws        device workspace of at least
 *             quantize_colwise_workspace_bytes(G, rows, cols_a, cols_b)
 *             bytes (cols_b = 0 for a single tensor), 256-byte aligned,
 *             caller-owned.  Its first word is a sticky error word
 *             (mg_workspace_error): 1 for a negative group size, 2 for
 *             sizes that sum past rows, as for the GEMMs (meaningful when
 *             it started at zero); the rest needs no initialising.  Calls
 *             that share a workspace must not overlap in time (enqueue them
 *             on one stream).
 * Errors: MG_EINVAL for the ranges above and NULL pointers,
 * MG_EUNSUPPORTED for misaligned inputs (16-byte) or cols above 2^20,
 * MG_EWORKSPACE for a missing, misaligned or small workspace. */
size_t quantize_colwise_workspace_bytes(int32_t G, int64_t rows, int32_t cols_a,
                                        int32_t cols_b);
int quantize_colwise_per_group_fp8(const void* a, int32_t cols_a,
                                   const void* b, int32_t cols_b,
                                   const int32_t* group_sizes, int32_t G,
                                   int64_t rows, int64_t ld, uint8_t* qa,
                                   float* sa, uint8_t* qb, float* sb, void* ws,
                                   size_t ws_bytes, mg_stream_t stream);

/* int4 weight quantizer for gmm_fwd_f8i4: w bf16 [E, K, N] -> w4 packed
 * [E][N][K/2] and sw bf16 [E][K/128][N]; per (e, n, 128-chunk j):
 * s = bf16_rne(max|w| / 7), q = clamp(rne(w / s), -8, 7) (q = 0 if s = 0).
 * K % 128 == 0, N % 8 == 0. */
int quantize_int4_weights(const void* w, int32_t E, int32_t K, int32_t N,
                          uint8_t* w4, void* sw, mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Token permutation for the token-sorted fused path ([FMOE]).               */
/* ------------------------------------------------------------------------ */

/* Router ([FMOE] fused_moe: softmax of the gating output in fp32, topk,
 * then, with renormalize, division by the sum of the chosen weights).  Per
 * token t:
 *   p = softmax(logits[t, :]) in fp32
 *   topk_ids[t, j]     = the j-th largest expert by probability (j ascending
 *                        = descending probability; ties to the lower index)
 *   topk_weights[t, j] = p[topk_ids[t, j]] (divided by the sum over j of
 *                        those when renormalize != 0)
 * logits fp32 [T, E] row-major; topk_ids int32 [T, top_k]; topk_weights
 * fp32 [T, top_k]; all device memory, caller-owned.  The choice is made on
 * the logits themselves (softmax is increasing), so ids are exactly those
 * of the fp32 logits.  One wave per token, no workspace.  Errors: T < 0,
 * E outside [1, MG_MAX_EXPERTS], top_k outside [1, min(E, 64)], NULL
 * pointers with T > 0 -> MG_EINVAL. */
int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t top_k,
                   int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                   mg_stream_t stream);

/* Capacity helpers: sorted_token_ids holds T*k + E*(block_m-1) entries;
 * expert_ids holds ceil(that / block_m). */
int64_t moe_sorted_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m);
int64_t moe_block_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m);

/* moe_align_block_size + gather.  For the flattened pair f = t*top_k + j
 * with expert topk_ids[f] (int32 [T, top_k], values in [0, E)):
 *   sorted_token_ids int32 [cap]: pairs grouped by expert ascending, f
 *       ascending within an expert, each expert's run padded to a multiple of
 *       block_m with the sentinel T*top_k; entries past the padded length are
 *       the sentinel.  An expert with no pairs has no block.
 *   expert_ids int32 [nblk]: expert of each block_m block (tail unspecified)
 *   num_tokens_post_padded int32 [1]: padded length
 *   inv_pos int32 [T*top_k]: position of pair f in sorted_token_ids
 *   padded_group_sizes int32 [E]: padded run length per expert (the group
 *       sizes for gmm_fwd over x_sorted)
 *   x_sorted bf16 [cap, hidden] (optional, with x bf16 [T, hidden]):
 *       row i = x[sorted_token_ids[i] / top_k], zeros for the sentinel.
 * A pair with an out-of-range expert id is dropped: it gets no position
 * and inv_pos = -1 (moe_unpermute skips it).  T*top_k must be <= 2^24;
 * hidden % 8 == 0. */
int moe_permute(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
                int32_t block_m, const void* x, int32_t hidden,
                int32_t* sorted_token_ids, int32_t* expert_ids,
                int32_t* num_tokens_post_padded, int32_t* inv_pos,
                int32_t* padded_group_sizes, void* x_sorted, void* ws,
                size_t ws_bytes, mg_stream_t stream);

/* Device workspace moe_permute needs (per-chunk counts and ranks). */
size_t moe_permute_workspace_bytes(int64_t T, int32_t top_k, int32_t E);

/* Top-k weighted combine: out[t, :] = bf16( sum_{j<top_k} w[t,j] *
 * y_sorted[inv_pos[t*top_k + j], :] ), summed in fp32 with j ascending
 * (deterministic, no atomics).  topk_weights fp32 [T, top_k] or NULL
 * (weights 1).  hidden % 8 == 0. */
int moe_unpermute(const void* y_sorted, const int32_t* inv_pos,
                  const float* topk_weights, int64_t T, int32_t top_k,
                  int32_t hidden, void* out, mg_stream_t stream);

/* act[r, i] = bf16( silu(h[r, i]) * h[r, inter + i] ), silu(x) = x/(1+e^-x),
 * computed in fp32 from bf16 h [rows, 2*inter]; act bf16 [rows, inter].
 * inter % 8 == 0. */
int silu_mul(const void* h, int64_t rows, int32_t inter, void* act,
             mg_stream_t stream);

/* SiLU*mul then rowwise e4m3 ([FMOE] fused_moe: silu_and_mul between the
 * two expert GEMMs; [FP8] commit message: the rowwise scale and cast as one
 * fused kernel), for the e4m3 operand of the second expert GEMM:
 * act = silu_mul(h) exactly as silu_mul computes it (bf16), then codes
 * q e4m3 [rows, inter] and scales fp32 [rows] exactly as
 * quantize_rowwise_fp8 computes them from act -- the same bits as the two
 * calls, in one pass over h.  act (bf16 [rows, inter]) may be NULL; when
 * given it receives act as well.  h bf16 [rows, 2*inter] contiguous,
 * 16-byte aligned (act too), q 8-byte aligned; inter % 8 == 0;
 * rows < 2^31. */
int silu_mul_quantize_rowwise_fp8(const void* h, int64_t rows, int32_t inter,
                                  void* act, uint8_t* q, float* scales,
                                  mg_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                              */
/* ------------------------------------------------------------------------ */

/* Message for the last failing call on this thread ("" if none). */
const char* mg_last_error(void);

/* Library version string. */
const char* mg_version(void);

/* Row-tile height (128 or 256) of the most recent grouped-GEMM launch this
 * thread enqueued through gmm_fwd, gmm_fwd_gather, gmm_fwd_silu_mul,
 * gmm_bwd, gmm_fwd_fp8 or gmm_bwd_fp8 (the last kernel of a call that
 * enqueues several), or 0 before the first.  Large fixed-M launches -- at
 * least two rounds of 256 x 256 tiles on every compute unit, contractions
 * of 1024 or more, 192 or more rows per group on average -- run on
 * 256 x 256 tiles with four waves; the rest on 128 x 256 tiles (dW: 128 or
 * 256 rows) with eight.  The result does not depend on the choice beyond
 * rounding order.  For diagnostics and tests; reads no device state. */
int32_t mg_last_gemm_tile_m(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GEMM_H */
