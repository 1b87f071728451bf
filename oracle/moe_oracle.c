/*
 * moe_oracle.c -- plain, slow, fp64 CPU oracle for the MoE grouped GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header or constant table with the HIP
 * library: every definition below is written out from the source pages.
 *
 * Sources (cited by page title and section):
 *  [P1] FBGEMM PR "F8I4 Grouped Gemm Optimization for Sparse M" -- summary:
 *       grouped GEMM over min(total_M, groups), empty groups are skipped.
 *  [P2] grouped_gemm PR "Support GPU-resident batch sizes" -- description
 *       (gmm(x, w, batch_sizes), grad of out.sum()) and review thread
 *       (single-block scan of the batch sizes; kDynamicK sorts problems by k
 *       in descending order; K=0 problems have their outputs zeroed).
 *  [P3] applied-ai issue "Column-major fused MoE" -- fused_moe_kernel,
 *       moe_align_block_size docstring (worked example), fused_moe
 *       (silu_and_mul between the two GEMMs, top-k weighted sum).
 *  [P4] torchao commit "Optimize FP8 MoE backward pass: fused colwise kernel"
 *       -- commit message (rowwise absmax + saturated cast) and the
 *       standalone colwise kernel in bench_colwise_block_configs.py
 *       (per-group column amax, EPS clamp in fp64, power-of-2 floor,
 *       column-major fp8 output, scales at group*N + col).
 *
 * Every GEMM is an unblocked triple loop accumulating in double.  The only
 * parallelism is an optional OpenMP split over independent output rows; it
 * does not change any result (each output element is summed in a fixed
 * order by one thread).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Threading control (for timing the oracle as a CPU baseline).             */
/* ------------------------------------------------------------------------ */

int or_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Number formats.                                                          */
/* ------------------------------------------------------------------------ */

/* bfloat16 -> double: bf16 is the upper half of an IEEE binary32. */
static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void or_bf16_to_f64(const uint16_t* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = bf16_value(src[i]);
}

/* double -> bfloat16, round to nearest, ties to even, directly from the
 * double (no intermediate float rounding).  Finite inputs only. */
static uint16_t bf16_from_double(double x) {
  if (x == 0.0) return signbit(x) ? 0x8000u : 0x0000u;
  int neg = x < 0;
  double a = fabs(x);
  int e;
  frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) */
  int unit_exp = e - 8;       /* bf16 keeps 8 significant bits */
  if (unit_exp < -133) unit_exp = -133; /* subnormal spacing 2^-133 */
  double m = ldexp(a, -unit_exp);
  double r = nearbyint(m);    /* default rounding mode: ties to even */
  double v = ldexp(r, unit_exp);
  float f = (float)v;         /* exact: v has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint16_t h = (uint16_t)(u >> 16);
  return neg ? (uint16_t)(h | 0x8000u) : h;
}

void or_f64_to_bf16(const double* src, int64_t n, uint16_t* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = bf16_from_double(src[i]);
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448.
 * Value of a non-negative code c (0..0x7E): */
static double e4m3_magnitude(int c) {
  int e = (c >> 3) & 0xF;
  int m = c & 0x7;
  if (e == 0) return ldexp((double)m, -9);         /* subnormal: m/8 * 2^-6 */
  return ldexp(1.0 + m / 8.0, e - 7);
}

double or_e4m3_value(uint8_t code) {
  int c = code & 0x7F;
  if (c == 0x7F) return NAN;
  double v = e4m3_magnitude(c);
  return (code & 0x80) ? -v : v;
}

void or_e4m3_to_f64(const uint8_t* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = or_e4m3_value(src[i]);
}

/* Encode a finite value already clamped to [-448, 448]: the nearest finite
 * magnitude found by brute force over the 127 non-negative finite codes;
 * an exact tie goes to the code whose mantissa LSB is 0 (round half to
 * even).  The sign bit is copied, so -0 and tiny negatives give 0x80. */
uint8_t or_e4m3_encode(float v) {
  if (isnan(v)) return (uint8_t)(0x7F | (signbit(v) ? 0x80 : 0));
  double a = fabs((double)v);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double err = fabs(e4m3_magnitude(c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

void or_e4m3_encode_array(const float* src, int64_t n, uint8_t* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = or_e4m3_encode(src[i]);
}

/* ------------------------------------------------------------------------ */
/* Group offsets and work lists ([P1] summary, [P2] review thread).          */
/* ------------------------------------------------------------------------ */

/* Exclusive prefix sum: offs[0] = 0, offs[g+1] = offs[g] + sizes[g].
 * Group g owns rows [offs[g], offs[g+1]). */
void or_offsets(const int32_t* sizes, int32_t E, int64_t* offs) {
  offs[0] = 0;
  for (int32_t g = 0; g < E; ++g) offs[g + 1] = offs[g] + sizes[g];
}

/* Fixed-M work list (forward, dX): for every non-empty group in ascending
 * order, one entry per BM-row slice: {g, first row, rows in slice, 0}.
 * Empty groups produce nothing ([P1]: only min(total_M, groups) problems).
 * Returns the number of entries; writes at most cap of them. */
int64_t or_worklist_fixed_m(const int32_t* sizes, int32_t E, int32_t BM,
                            int32_t* entries, int64_t cap) {
  int64_t count = 0, row = 0;
  for (int32_t g = 0; g < E; ++g) {
    for (int64_t r = 0; r < sizes[g]; r += BM) {
      if (count < cap) {
        entries[4 * count + 0] = g;
        entries[4 * count + 1] = (int32_t)(row + r);
        entries[4 * count + 2] = (int32_t)((sizes[g] - r) < BM ? (sizes[g] - r) : BM);
        entries[4 * count + 3] = 0;
      }
      ++count;
    }
    row += sizes[g];
  }
  return count;
}

/* Dynamic-K work list (dW): all E groups, ordered by size descending, ties
 * by group index ascending ([P2]: problems sorted by k, descending).  An
 * entry with size 0 stands for a group whose dW is all zeros. */
void or_worklist_dynamic_k(const int32_t* sizes, int32_t E, int32_t* entries) {
  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E + 1));
  or_offsets(sizes, E, offs);
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int32_t i = 0; i < E; ++i) order[i] = i;
  /* insertion sort: stable, obviously correct */
  for (int32_t i = 1; i < E; ++i) {
    int32_t g = order[i];
    int32_t j = i - 1;
    while (j >= 0 && sizes[order[j]] < sizes[g]) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = g;
  }
  for (int32_t i = 0; i < E; ++i) {
    int32_t g = order[i];
    entries[4 * i + 0] = g;
    entries[4 * i + 1] = (int32_t)offs[g];
    entries[4 * i + 2] = sizes[g];
    entries[4 * i + 3] = 0;
  }
  free(order);
  free(offs);
}

/* ------------------------------------------------------------------------ */
/* Grouped GEMMs in fp64 ([P2] description: gmm forward and the gradients   */
/* of out.sum()).  W is [E][K][N] (N fastest).  Rows r of X belong to the    */
/* group g with offs[g] <= r < offs[g+1].                                    */
/* ------------------------------------------------------------------------ */

/* Y[r,n] = sum_k X[r,k] * W[g,k,n] */
void or_gmm_fwd(const double* X, const double* W, const int32_t* sizes,
                int32_t E, int64_t M, int64_t K, int64_t N, double* Y) {
  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E + 1));
  or_offsets(sizes, E, offs);
  for (int64_t i = 0; i < M * N; ++i) Y[i] = 0.0;
  for (int32_t g = 0; g < E; ++g) {
    const double* Wg = W + (int64_t)g * K * N;
#pragma omp parallel for schedule(static)
    for (int64_t r = offs[g]; r < offs[g + 1]; ++r) {
      for (int64_t k = 0; k < K; ++k) {
        double a = X[r * K + k];
        for (int64_t n = 0; n < N; ++n) Y[r * N + n] += a * Wg[k * N + n];
      }
    }
  }
  free(offs);
}

/* dX[r,k] = sum_n dY[r,n] * W[g,k,n] */
void or_gmm_dx(const double* dY, const double* W, const int32_t* sizes,
               int32_t E, int64_t M, int64_t K, int64_t N, double* dX) {
  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E + 1));
  or_offsets(sizes, E, offs);
  for (int64_t i = 0; i < M * K; ++i) dX[i] = 0.0;
  for (int32_t g = 0; g < E; ++g) {
    const double* Wg = W + (int64_t)g * K * N;
#pragma omp parallel for schedule(static)
    for (int64_t r = offs[g]; r < offs[g + 1]; ++r) {
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += dY[r * N + n] * Wg[k * N + n];
        dX[r * K + k] = acc;
      }
    }
  }
  free(offs);
}

/* dW[g,k,n] = sum_{r in g} X[r,k] * dY[r,n]; an empty group gives exactly 0
 * ([P2] review thread: outputs of K=0 problems are zeroed). */
void or_gmm_dw(const double* X, const double* dY, const int32_t* sizes,
               int32_t E, int64_t M, int64_t K, int64_t N, double* dW) {
  (void)M;
  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E + 1));
  or_offsets(sizes, E, offs);
  for (int64_t i = 0; i < (int64_t)E * K * N; ++i) dW[i] = 0.0;
  for (int32_t g = 0; g < E; ++g) {
    double* dWg = dW + (int64_t)g * K * N;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
      for (int64_t r = offs[g]; r < offs[g + 1]; ++r) {
        double a = X[r * K + k];
        for (int64_t n = 0; n < N; ++n) dWg[k * N + n] += a * dY[r * N + n];
      }
    }
  }
  free(offs);
}

/* ------------------------------------------------------------------------ */
/* FP8 quantizers ([P4] commit message and colwise kernel).                 */
/* Scale recipe: t = fp32(448 / max(amax, 1e-12)) computed in double, then  */
/* s = 2^floor(log2 t), taken exactly by clearing t's mantissa bits.  Code  */
/* = e4m3(clamp(x * s, -448, 448)).  Dequantization is code / s.            */
/* ------------------------------------------------------------------------ */

#define OR_FP8_MAX 448.0
#define OR_EPS 1e-12

static float pow2_floor_scale(double amax) {
  double clamped = amax > OR_EPS ? amax : OR_EPS;
  float t = (float)(OR_FP8_MAX / clamped);   /* round to nearest fp32 */
  uint32_t u;
  memcpy(&u, &t, sizeof u);
  u &= 0xFF800000u;                           /* keep sign and exponent */
  float s;
  memcpy(&s, &u, sizeof s);
  return s;
}

float or_fp8_scale_from_amax(double amax) { return pow2_floor_scale(amax); }

static uint8_t quant_one(uint16_t xb, float s) {
  float x = (float)bf16_value(xb);
  float v = x * s;
  if (v > (float)OR_FP8_MAX) v = (float)OR_FP8_MAX;
  if (v < -(float)OR_FP8_MAX) v = -(float)OR_FP8_MAX;
  return or_e4m3_encode(v);
}

/* Rowwise: one scale per row of a row-major [rows, cols] bf16 matrix. */
void or_quant_rowwise(const uint16_t* x, int64_t rows, int64_t cols,
                      uint8_t* q, float* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double amax = 0.0;
    for (int64_t c = 0; c < cols; ++c) {
      double a = fabs(bf16_value(x[r * cols + c]));
      if (a > amax) amax = a;
    }
    float s = pow2_floor_scale(amax);
    scales[r] = s;
    for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = quant_one(x[r * cols + c], s);
  }
}

/* Per-group colwise: for each group g (rows [offs[g], offs[g+1])) and each
 * column c, one scale over the group's rows.  Codes are written
 * column-major, q[c * rows + r]; scales at s[g * cols + c].  An empty group
 * gets amax 0 and writes no codes. */
void or_quant_colwise(const uint16_t* x, int64_t rows, int64_t cols,
                      const int32_t* sizes, int32_t G, uint8_t* q, float* scales) {
  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
  or_offsets(sizes, G, offs);
  for (int32_t g = 0; g < G; ++g) {
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
      double amax = 0.0;
      for (int64_t r = offs[g]; r < offs[g + 1]; ++r) {
        double a = fabs(bf16_value(x[r * cols + c]));
        if (a > amax) amax = a;
      }
      float s = pow2_floor_scale(amax);
      scales[(int64_t)g * cols + c] = s;
      for (int64_t r = offs[g]; r < offs[g + 1]; ++r)
        q[c * rows + r] = quant_one(x[r * cols + c], s);
    }
  }
  free(offs);
}

/* Dequantize rowwise codes: out[r,c] = e4m3(q[r,c]) / s[r]. */
void or_dequant_rowwise(const uint8_t* q, const float* s, int64_t rows,
                        int64_t cols, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      out[r * cols + c] = or_e4m3_value(q[r * cols + c]) / (double)s[r];
}

/* Dequantize per-group colwise codes (column-major) into row-major. */
void or_dequant_colwise(const uint8_t* q, const float* s, int64_t rows,
                        int64_t cols, const int32_t* sizes, int32_t G,
                        double* out) {
  int64_t* offs = (int64_t*)malloc(sizeof(int64_t) * (size_t)(G + 1));
  or_offsets(sizes, G, offs);
  for (int32_t g = 0; g < G; ++g)
    for (int64_t r = offs[g]; r < offs[g + 1]; ++r)
      for (int64_t c = 0; c < cols; ++c)
        out[r * cols + c] = or_e4m3_value(q[c * rows + r]) / (double)s[(int64_t)g * cols + c];
  free(offs);
}

/* ------------------------------------------------------------------------ */
/* int4 weights ([P1] F8I4: fp8 activations x int4 weights).  Symmetric,     */
/* one bf16 scale per (expert, column n, 128-long chunk of K).               */
/*   s = bf16(max|w| / 7),  q = clamp(round_half_even(w / s), -8, 7)        */
/* Packed [E][N][K/2]: byte = (q[2i] & 0xF) | (q[2i+1] << 4).  Scales are    */
/* [E][K/group][N].  W is given as fp64 [E][K][N].                           */
/* ------------------------------------------------------------------------ */

void or_quant_int4(const double* W, int32_t E, int64_t K, int64_t N,
                   int32_t group, uint8_t* packed, uint16_t* scales) {
  int64_t nchunks = K / group;
  for (int32_t e = 0; e < E; ++e) {
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t j = 0; j < nchunks; ++j) {
        double amax = 0.0;
        for (int64_t k = j * group; k < (j + 1) * group; ++k) {
          double a = fabs(W[((int64_t)e * K + k) * N + n]);
          if (a > amax) amax = a;
        }
        uint16_t sb = bf16_from_double(amax / 7.0);
        scales[((int64_t)e * nchunks + j) * N + n] = sb;
        double s = bf16_value(sb);
        for (int64_t k = j * group; k < (j + 1) * group; ++k) {
          int q = 0;
          if (s != 0.0) {
            double t = nearbyint(W[((int64_t)e * K + k) * N + n] / s);
            if (t > 7) t = 7;
            if (t < -8) t = -8;
            q = (int)t;
          }
          uint8_t* byte = &packed[((int64_t)e * N + n) * (K / 2) + k / 2];
          if ((k & 1) == 0)
            *byte = (uint8_t)((*byte & 0xF0) | (q & 0xF));
          else
            *byte = (uint8_t)((*byte & 0x0F) | ((q & 0xF) << 4));
        }
      }
    }
  }
}

/* Signed value of nibble k of row (e, n). */
static int int4_at(const uint8_t* packed, int64_t K, int64_t N, int32_t e,
                   int64_t n, int64_t k) {
  uint8_t byte = packed[((int64_t)e * N + n) * (K / 2) + k / 2];
  int v = (k & 1) ? (byte >> 4) : (byte & 0xF);
  return v >= 8 ? v - 16 : v;
}

/* Dequantize to fp64 [E][K][N]: w = q * s (exact in double). */
void or_dequant_int4(const uint8_t* packed, const uint16_t* scales, int32_t E,
                     int64_t K, int64_t N, int32_t group, double* W) {
  int64_t nchunks = K / group;
  for (int32_t e = 0; e < E; ++e)
    for (int64_t k = 0; k < K; ++k)
      for (int64_t n = 0; n < N; ++n)
        W[((int64_t)e * K + k) * N + n] =
            (double)int4_at(packed, K, N, e, n, k) *
            bf16_value(scales[((int64_t)e * nchunks + k / group) * N + n]);
}

/* ------------------------------------------------------------------------ */
/* Token permutation for the fused path ([P3] moe_align_block_size and       */
/* fused_moe).                                                               */
/* ------------------------------------------------------------------------ */

/* topk_ids [T][k] (0-based experts).  Flattened pair f = t*k + j.  Pairs are
 * grouped by expert in ascending order, keeping f ascending inside an
 * expert; each expert's run is padded up to a multiple of block_m with the
 * sentinel T*k; an expert with no pairs gets no block.  Outputs:
 *   sorted_ids[cap]      (cap = T*k + E*(block_m-1); tail = sentinel)
 *   expert_ids[nblk_cap] (one expert per block; unused tail = -1)
 *   *num_post_padded     (padded length)
 *   inv[T*k]             (position of pair f in sorted_ids)
 *   padded_sizes[E]      (padded run length per expert)
 * Returns 0, or -1 if an expert id is out of range. */
int or_moe_align(const int32_t* topk_ids, int64_t T, int32_t k, int32_t E,
                 int32_t block_m, int32_t* sorted_ids, int64_t cap,
                 int32_t* expert_ids, int64_t nblk_cap,
                 int32_t* num_post_padded, int32_t* inv, int32_t* padded_sizes) {
  int64_t P = T * k;
  for (int64_t i = 0; i < P; ++i)
    if (topk_ids[i] < 0 || topk_ids[i] >= E) return -1;
  for (int64_t i = 0; i < cap; ++i) sorted_ids[i] = (int32_t)P;
  for (int64_t i = 0; i < nblk_cap; ++i) expert_ids[i] = -1;
  int64_t pos = 0, blk = 0;
  for (int32_t e = 0; e < E; ++e) {
    int64_t cnt = 0;
    for (int64_t f = 0; f < P; ++f) {
      if (topk_ids[f] == e) {
        sorted_ids[pos + cnt] = (int32_t)f;
        inv[f] = (int32_t)(pos + cnt);
        ++cnt;
      }
    }
    int64_t padded = (cnt + block_m - 1) / block_m * block_m;
    padded_sizes[e] = (int32_t)padded;
    for (int64_t b = 0; b < padded / block_m; ++b) expert_ids[blk++] = e;
    pos += padded;
  }
  *num_post_padded = (int32_t)pos;
  return 0;
}

/* x_sorted[i] = X[sorted_ids[i] / k], zeros for the sentinel (bf16 bits). */
void or_gather_rows(const uint16_t* X, int64_t T, int32_t k, int64_t H,
                    const int32_t* sorted_ids, int64_t rows, uint16_t* out) {
  for (int64_t i = 0; i < rows; ++i) {
    int64_t f = sorted_ids[i];
    for (int64_t h = 0; h < H; ++h)
      out[i * H + h] = (f < T * k) ? X[(f / k) * H + h] : (uint16_t)0;
  }
}

/* act[r,i] = silu(h[r,i]) * h[r,I+i], silu(x) = x / (1 + exp(-x)); the
 * first half of each row is the gate, the second half the up projection
 * ([P3] fused_moe: silu_and_mul of the first GEMM's output). */
void or_silu_mul(const double* h, int64_t rows, int64_t I, double* act) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < I; ++i) {
      double g = h[r * 2 * I + i];
      double u = h[r * 2 * I + I + i];
      act[r * I + i] = g / (1.0 + exp(-g)) * u;
    }
}

/* out[t,:] = sum_{j<k} w[t,j] * Y[inv[t*k+j], :], j ascending ([P3]
 * fused_moe: the top-k weighted sum over each token's expert outputs). */
void or_unpermute(const double* Y, const int32_t* inv, const float* w,
                  int64_t T, int32_t k, int64_t H, double* out) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        double wt = w ? (double)w[t * k + j] : 1.0;
        acc += wt * Y[(int64_t)inv[t * k + j] * H + h];
      }
      out[t * H + h] = acc;
    }
}

/* Router: probabilities p = softmax(logits) in fp64 over each token's E
 * logits; the token's experts are the top_k largest, in descending order
 * ([P3] fused_moe: softmax of the gating output in fp32, then topk, then an
 * optional division by the sum of the chosen weights).  The integer decision
 * is taken on the fp32 logits themselves (softmax is increasing, so the
 * order is the same), ties to the lower expert index; weights are
 * p[id] (divided by their sum when renormalize). */
void or_route_topk(const float* logits, int64_t T, int32_t E, int32_t top_k,
                   int32_t renormalize, int32_t* ids, double* weights) {
  for (int64_t t = 0; t < T; ++t) {
    const float* z = logits + t * E;
    double mx = -INFINITY;
    for (int32_t e = 0; e < E; ++e)
      if ((double)z[e] > mx) mx = (double)z[e];
    double sum = 0.0;
    for (int32_t e = 0; e < E; ++e) sum += exp((double)z[e] - mx);
    double chosen = 0.0;
    for (int32_t j = 0; j < top_k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        int taken = 0;
        for (int32_t i = 0; i < j; ++i)
          if (ids[t * top_k + i] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || z[e] > z[best]) best = e;
      }
      ids[t * top_k + j] = best;
      weights[t * top_k + j] = exp((double)z[best] - mx) / sum;
      chosen += weights[t * top_k + j];
    }
    if (renormalize)
      for (int32_t j = 0; j < top_k; ++j) weights[t * top_k + j] /= chosen;
  }
}
