// C ABI of the library: host-side argument checks, workspace carving and
// kernel launches.  Nothing here reads device memory or synchronizes, except
// mg_workspace_error, which exists for tests.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe_gemm.h"
#include "kernels.h"

using namespace mg;

// Scratch of gmm_fwd_noalloc: one GEMM workspace (error word, stream-K
// arrival counters, partial tiles: 64 MiB + 1280 bytes) as a file-scope
// device array, so that entry point allocates nothing.  Each device the
// library runs on holds its own copy until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only stands for
// the symbol): the device's address of its copy comes from
// hipGetSymbolAddress, once per device, and is kept in noalloc_ptr.
static constexpr size_t kNoAllocBytes = (size_t)kWsBytes;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MG_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MG_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

hipStream_t S(mg_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxRows = (int64_t)1 << 31;

int check_common(const int32_t* sizes, int32_t E, int64_t total_M, const void* ws, size_t ws_bytes) {
  if (E < 1 || E > MG_MAX_EXPERTS) return fail(MG_EINVAL, "E=%d outside [1, %d]", E, MG_MAX_EXPERTS);
  if (total_M < 0 || total_M >= kMaxRows) return fail(MG_EINVAL, "total_M=%lld outside [0, 2^31)", (long long)total_M);
  if (sizes == nullptr) return fail(MG_EINVAL, "group_sizes is NULL");
  if (ws == nullptr) return fail(MG_EWORKSPACE, "workspace is NULL");
  const size_t need = (size_t)ws_layout(E, total_M).total;
  if (ws_bytes < need) return fail(MG_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return fail(MG_EINVAL, "workspace must be 256-byte aligned");
  return MG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The GEMM kernels address each operand tile through a buffer resource that
// reaches at most 2 GiB from the tile origin: one expert's weight slice and
// the token rows of one operand must stay below that.
int check_extents(int64_t total_M, int32_t K, int32_t N, int esz) {
  const int64_t lim = ((int64_t)1 << 31) - 1;
  const int64_t mx = K > N ? K : N;
  if ((int64_t)K * N * esz > lim || total_M * mx * esz > lim)
    return fail(MG_EUNSUPPORTED, "operand larger than 2 GiB (K*N or total_M*max(K,N) bytes)");
  return MG_OK;
}

int32_t* err_word(void* ws) { return reinterpret_cast<int32_t*>(ws) + kWsErrorWord; }

// Workspace pointers every GEMM launch carries.
void attach_ws(GemmArgs& a, void* ws) {
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  a.err = err_word(ws);
  a.sk_ctr = reinterpret_cast<int32_t*>(p + kWsCounters);
  a.wq = reinterpret_cast<int32_t*>(ws) + kWsQueueWord;
  a.sk_part = reinterpret_cast<float*>(p + kWsPartials);
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

__global__ void set_word_kernel(int32_t* p, int32_t v) {
  if (threadIdx.x == 0) p[0] = v;
}

GemmArgs blank_args() {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  return a;
}

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices] = {};

// The current device's scratch address.  On the first call on a device the
// header and counters are cleared by a fill kernel enqueued on `stream`
// (a kernel, not a memset, so a capturing stream records a kernel node).
int noalloc_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "gmm_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MG_EUNSUPPORTED, "device %d past the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                           "gmm_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if ((reinterpret_cast<uintptr_t>(p) & 255) != 0) return fail(MG_EHIP, "gmm_fwd_noalloc: scratch not 256-byte aligned");
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, stream, reinterpret_cast<int32_t*>(p), kWsZeroWords);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "gmm_fwd_noalloc: clearing the scratch");
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return MG_OK;
}

}  // namespace

extern "C" {

const char* mg_last_error(void) { return g_err; }

const char* mg_version(void) { return "moe-gemm-gfx950 0.1"; }

int32_t mg_last_gemm_tile_m(void) { return last_gemm_tile_m(); }

size_t mg_workspace_bytes(int32_t E, int64_t total_M) {
  if (E < 1 || E > MG_MAX_EXPERTS || total_M < 0) return 0;
  return (size_t)ws_layout(E, total_M).total;
}

int32_t mg_workspace_error(const void* ws) {
  if (ws == nullptr) return -1;
  int32_t v = 0;
  if (hipMemcpy(&v, reinterpret_cast<const int32_t*>(ws) + kWsErrorWord, sizeof v, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return -1;
  return v;
}

int mg_workspace_clear(void* ws, mg_stream_t stream) {
  if (ws == nullptr) return fail(MG_EINVAL, "workspace is NULL");
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, S(stream), reinterpret_cast<int32_t*>(ws),
                     kWsZeroWords);
  return hip_status(hipGetLastError(), "mg_workspace_clear");
}

int gmm_build_worklist(int32_t kind, const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t bm,
                       int32_t* offs, int32_t* count, int32_t* entries, int64_t cap, mg_stream_t stream) {
  if (E < 1 || E > MG_MAX_EXPERTS) return fail(MG_EINVAL, "E=%d outside [1, %d]", E, MG_MAX_EXPERTS);
  if (total_M < 0 || total_M >= kMaxRows) return fail(MG_EINVAL, "total_M out of range");
  if (bm < 1) return fail(MG_EINVAL, "bm must be >= 1");
  if (!group_sizes || !offs || !count || !entries) return fail(MG_EINVAL, "NULL pointer argument");
  if (kind != MG_WL_FIXED_M && kind != MG_WL_DYNAMIC_K) return fail(MG_EINVAL, "unknown work-list kind %d", kind);
  const int64_t need = kind == MG_WL_FIXED_M ? fixed_m_capacity(total_M, E, bm) : E;
  if (cap < need) return fail(MG_EINVAL, "cap %lld < %lld", (long long)cap, (long long)need);
  BuildArgs b;
  b.sizes = group_sizes;
  b.E = E;
  b.total_M = total_M;
  b.bm = bm;
  b.kind = kind;
  b.offs = offs;
  b.count = count;
  b.entries = entries;
  hipError_t e = launch_build_worklist(b, S(stream));
  return hip_status(e, "gmm_build_worklist");
}

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

static int gmm_fwd_with(const void* x, const void* w, const int32_t* group_sizes, int32_t E, int64_t total_M,
                        int32_t K, int32_t N, int32_t trans_b, void* y, void* ws, size_t ws_bytes, mg_stream_t stream,
                        const char* name) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if (K < 1 || N < 1) return fail(MG_EINVAL, "K and N must be positive");
  if (K % 8 || N % 8) return fail(MG_EUNSUPPORTED, "K and N must be multiples of 8");
  if ((rc = check_extents(total_M, K, N, 2))) return rc;
  if (total_M == 0) return ok();
  if (!x || !w || !y) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  GemmArgs a = blank_args();
  a.A = x;
  a.a_ld = K;
  a.B = w;
  if (trans_b) {
    a.b_ld = K;                 // W[g, n, k]
  } else {
    a.b_ld = N;                 // W[g, k, n]
  }
  a.b_gs = (int64_t)K * N;
  a.C = y;
  a.c_ld = N;
  a.c_gs = 0;
  a.Nout = N;
  a.Kc = K;
  a.E = E;
  a.total_rows = total_M;
  a.sizes = group_sizes;
  attach_ws(a, ws);
  GemmLaunch L;
  L.kind = FIXED_M;
  L.elem = EL_BF16;
  L.a_kc = true;
  L.b_kc = trans_b != 0;
  return hip_status(launch_gemm(L, a, S(stream)), name);
}

int gmm_fwd(const void* x, const void* w, const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t K,
            int32_t N, int32_t trans_b, void* y, void* ws, size_t ws_bytes, mg_stream_t stream) {
  return gmm_fwd_with(x, w, group_sizes, E, total_M, K, N, trans_b, y, ws, ws_bytes, stream, "gmm_fwd");
}

int gmm_fwd_noalloc(const void* x, const void* w, const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t K,
                    int32_t N, int32_t trans_b, void* y, mg_stream_t stream) {
  // the scratch a call needs depends on host values only; refuse what the
  // fixed array cannot hold before touching the device
  if (E < 1 || E > MG_MAX_EXPERTS) return fail(MG_EINVAL, "E=%d outside [1, %d]", E, MG_MAX_EXPERTS);
  if (total_M < 0 || total_M >= kMaxRows) return fail(MG_EINVAL, "total_M=%lld outside [0, 2^31)", (long long)total_M);
  const size_t need = (size_t)ws_layout(E, total_M).total;
  if (need > kNoAllocBytes)
    return fail(MG_EWORKSPACE, "gmm_fwd_noalloc: needs %zu bytes of scratch, the fixed array holds %zu", need,
                kNoAllocBytes);
  void* ws = nullptr;
  int rc = noalloc_scratch(&ws, S(stream));
  if (rc) return rc;
  return gmm_fwd_with(x, w, group_sizes, E, total_M, K, N, trans_b, y, ws, kNoAllocBytes, stream, "gmm_fwd_noalloc");
}

int gmm_fwd_gather(const void* x, int64_t T, const int32_t* sorted_token_ids, int32_t top_k, const void* w,
                   const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t K, int32_t N, int32_t trans_b,
                   void* y, void* ws, size_t ws_bytes, mg_stream_t stream) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if (K < 1 || N < 1) return fail(MG_EINVAL, "K and N must be positive");
  if (K % 8 || N % 8) return fail(MG_EUNSUPPORTED, "K and N must be multiples of 8");
  if (T < 0 || top_k < 1 || T * (int64_t)top_k > ((int64_t)1 << 24))
    return fail(MG_EINVAL, "T=%lld, top_k=%d: need T >= 0, top_k >= 1, T*top_k <= 2^24", (long long)T, top_k);
  if ((rc = check_extents(total_M, K, N, 2))) return rc;
  if ((rc = check_extents(T, K, N, 2))) return rc;
  if (total_M == 0) return ok();
  if (!x || !w || !y || !sorted_token_ids) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  GemmArgs a = blank_args();
  a.A = x;
  a.a_ld = K;
  a.gather = sorted_token_ids;
  a.gather_div = top_k;
  a.gather_limit = (int32_t)(T * top_k);
  a.B = w;
  a.b_ld = trans_b ? K : N;
  a.b_gs = (int64_t)K * N;
  a.C = y;
  a.c_ld = N;
  a.c_gs = 0;
  a.Nout = N;
  a.Kc = K;
  a.E = E;
  a.total_rows = total_M;
  a.sizes = group_sizes;
  attach_ws(a, ws);
  GemmLaunch L;
  L.kind = FIXED_M;
  L.elem = EL_BF16;
  L.a_kc = true;
  L.b_kc = trans_b != 0;
  return hip_status(launch_gemm(L, a, S(stream)), "gmm_fwd_gather");
}

int gmm_fwd_silu_mul(const void* x, int64_t T, const int32_t* sorted_token_ids, int32_t top_k, const void* w1,
                     const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t K, int32_t I, int32_t trans_b,
                     void* act, void* ws, size_t ws_bytes, mg_stream_t stream) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if (K < 1 || I < 1) return fail(MG_EINVAL, "K and I must be positive");
  if (K % 8 || I % 8) return fail(MG_EUNSUPPORTED, "K and I must be multiples of 8");
  if (I > (1 << 30)) return fail(MG_EUNSUPPORTED, "I too large");
  if ((rc = check_extents(total_M, K, 2 * I, 2))) return rc;
  if (sorted_token_ids) {
    if (T < 0 || top_k < 1 || T * (int64_t)top_k > ((int64_t)1 << 24))
      return fail(MG_EINVAL, "T=%lld, top_k=%d: need T >= 0, top_k >= 1, T*top_k <= 2^24", (long long)T, top_k);
    if ((rc = check_extents(T, K, 2 * I, 2))) return rc;
  }
  if (total_M == 0) return ok();
  if (!x || !w1 || !act) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || !aligned16(w1) || !aligned16(act)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  GemmArgs a = blank_args();
  a.A = x;
  a.a_ld = K;
  if (sorted_token_ids) {
    a.gather = sorted_token_ids;
    a.gather_div = top_k;
    a.gather_limit = (int32_t)(T * top_k);
  }
  a.B = w1;
  // W1[g, k, n]: gate columns 0..I-1, up columns I..2I-1; with trans_b,
  // W1[g, n, k]: gate rows 0..I-1, up rows I..2I-1
  a.b_ld = trans_b ? (int64_t)K : 2 * (int64_t)I;
  a.b_gs = (int64_t)K * 2 * I;
  a.C = act;
  a.c_ld = I;
  a.c_gs = 0;
  a.Nout = I;
  a.Kc = K;
  a.E = E;
  a.total_rows = total_M;
  a.sizes = group_sizes;
  attach_ws(a, ws);
  GemmLaunch L;
  L.kind = FIXED_M;
  L.elem = EL_BF16;
  L.a_kc = true;
  L.b_kc = trans_b != 0;
  L.swiglu = true;
  return hip_status(launch_gemm(L, a, S(stream)), "gmm_fwd_silu_mul");
}

int gmm_bwd(const void* dy, const void* x, const void* w, const int32_t* group_sizes, int32_t E,
            int64_t total_M, int32_t K, int32_t N, int32_t trans_b, void* dx, void* dw, void* ws,
            size_t ws_bytes, mg_stream_t stream) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if (!dx && !dw) return fail(MG_EINVAL, "dx and dw are both NULL");
  if (total_M > 0 && (!dy || (dx && !w) || (dw && !x))) return fail(MG_EINVAL, "NULL tensor argument");
  if (K < 1 || N < 1) return fail(MG_EINVAL, "K and N must be positive");
  if (K % 8 || N % 8) return fail(MG_EUNSUPPORTED, "K and N must be multiples of 8");
  if ((rc = check_extents(total_M, K, N, 2))) return rc;
  if (!aligned16(dy) || (x && !aligned16(x)) || (w && !aligned16(w)) || (dx && !aligned16(dx)) ||
      (dw && !aligned16(dw)))
    return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  if (total_M == 0 && !dw) return ok();
  hipError_t e = hipSuccess;
  if (dx && total_M > 0) {
    GemmArgs a = blank_args();
    a.A = dy;
    a.a_ld = N;
    a.B = w;
    a.b_ld = trans_b ? K : N;   // [E,K,N]: W[g,k,n], contraction n contiguous; [E,N,K]: k contiguous
    a.b_gs = (int64_t)K * N;
    a.C = dx;
    a.c_ld = K;
    a.Nout = K;
    a.Kc = N;
    a.E = E;
    a.total_rows = total_M;
    a.sizes = group_sizes;
    attach_ws(a, ws);
    GemmLaunch L;
    L.kind = FIXED_M;
    L.elem = EL_BF16;
    L.a_kc = true;
    L.b_kc = trans_b == 0;
    e = launch_gemm(L, a, S(stream));
    if (e != hipSuccess) return hip_status(e, "gmm_bwd dx");
  }
  if (dw && total_M == 0) {
    e = launch_zero_fill(dw, (int64_t)E * K * N * 2, S(stream));
    if (e != hipSuccess) return hip_status(e, "gmm_bwd dw zero fill");
  } else if (dw) {
    GemmArgs a = blank_args();
    if (!trans_b) {   // dW[g, k, n] = sum_r X[r, k] dY[r, n]
      a.A = x;
      a.a_ld = K;
      a.B = dy;
      a.b_ld = N;
      a.Mout = K;
      a.Nout = N;
      a.c_ld = N;
    } else {          // dW[g, n, k] = sum_r dY[r, n] X[r, k]
      a.A = dy;
      a.a_ld = N;
      a.B = x;
      a.b_ld = K;
      a.Mout = N;
      a.Nout = K;
      a.c_ld = K;
    }
    a.b_gs = 0;
    a.C = dw;
    a.c_gs = (int64_t)K * N;
    a.E = E;
    a.total_rows = total_M;
    a.sizes = group_sizes;
    attach_ws(a, ws);
    GemmLaunch L;
    L.kind = DYNAMIC_K;
    L.elem = EL_BF16;
    L.a_kc = false;
    L.b_kc = false;
    e = launch_gemm(L, a, S(stream));
    if (e != hipSuccess) return hip_status(e, "gmm_bwd dw");
  }
  return ok();
}

// ---------------------------------------------------------------------------
// fp8
// ---------------------------------------------------------------------------

static int check_fp8_weight(const mg_fp8_weight* w) {
  if (!w || !w->codes || !w->scales) return fail(MG_EINVAL, "fp8 weight descriptor incomplete");
  if (w->ld < 1 || w->expert_stride < 0) return fail(MG_EINVAL, "fp8 weight strides invalid");
  if (w->ld % 16 || w->expert_stride % 16 || !aligned16(w->codes))
    return fail(MG_EUNSUPPORTED, "fp8 weight strides and base must be multiples of 16 bytes");
  return MG_OK;
}

int gmm_fwd_fp8(const uint8_t* xq, const float* sx, const mg_fp8_weight* w, const int32_t* group_sizes,
                int32_t E, int64_t total_M, int32_t K, int32_t N, void* y, void* ws, size_t ws_bytes,
                mg_stream_t stream) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_fp8_weight(w))) return rc;
  if (K < 1 || N < 1) return fail(MG_EINVAL, "K and N must be positive");
  if (K % 16 || N % 8) return fail(MG_EUNSUPPORTED, "K must be a multiple of 16 and N of 8");
  if (w->ld < K) return fail(MG_EINVAL, "weight ld < K");
  if ((rc = check_extents(total_M, K, N, 1))) return rc;
  if (total_M == 0) return ok();
  if (!xq || !sx || !y) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(xq) || !aligned16(y)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  GemmArgs a = blank_args();
  a.A = xq;
  a.a_ld = K;
  a.B = w->codes;
  a.b_ld = w->ld;
  a.b_gs = w->expert_stride;
  a.C = y;
  a.c_ld = N;
  a.sa = sx;
  a.sb = w->scales;
  a.Nout = N;
  a.Kc = K;
  a.E = E;
  a.total_rows = total_M;
  a.sizes = group_sizes;
  attach_ws(a, ws);
  GemmLaunch L;
  L.kind = FIXED_M;
  L.elem = EL_FP8;
  L.a_kc = L.b_kc = true;
  return hip_status(launch_gemm(L, a, S(stream)), "gmm_fwd_fp8");
}

int gmm_bwd_fp8(const uint8_t* dyq, const float* sdy, const mg_fp8_weight* w, const uint8_t* xc,
                const float* sxc, const uint8_t* dyc, const float* sdyc, int64_t ldc, const int32_t* group_sizes,
                int32_t E, int64_t total_M, int32_t K, int32_t N, void* dx, void* dw, void* ws, size_t ws_bytes,
                mg_stream_t stream) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if (!dx && !dw) return fail(MG_EINVAL, "dx and dw are both NULL");
  if (K < 1 || N < 1) return fail(MG_EINVAL, "K and N must be positive");
  if ((rc = check_extents(total_M, K, N, 1))) return rc;
  if (dx) {
    if ((rc = check_fp8_weight(w))) return rc;
    if (total_M > 0 && (!dyq || !sdy)) return fail(MG_EINVAL, "NULL dx operand");
    if (N % 16 || K % 8) return fail(MG_EUNSUPPORTED, "dx needs N % 16 == 0 and K % 8 == 0");
    if (w->ld < N) return fail(MG_EINVAL, "weight ld < N");
    if (!aligned16(dyq) || !aligned16(dx)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  }
  if (dw) {
    if (!sxc || !sdyc || (total_M > 0 && (!xc || !dyc))) return fail(MG_EINVAL, "NULL dw operand");
    if (total_M % 16) return fail(MG_EUNSUPPORTED, "dw needs total_M % 16 == 0");
    if (total_M > 0 && (ldc < total_M || ldc % 16))
      return fail(MG_EINVAL, "ldc must be a multiple of 16 and at least total_M");
    if (total_M > 0 && (rc = check_extents(ldc, K, N, 1))) return rc;
    if (K % 8 || N % 8) return fail(MG_EUNSUPPORTED, "dw needs K and N multiples of 8");
    if (!aligned16(xc) || !aligned16(dyc) || !aligned16(dw)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  }
  if (total_M == 0 && !dw) return ok();
  hipError_t e = hipSuccess;
  if (dx && total_M > 0) {
    GemmArgs a = blank_args();
    a.A = dyq;
    a.a_ld = N;
    a.B = w->codes;
    a.b_ld = w->ld;
    a.b_gs = w->expert_stride;
    a.C = dx;
    a.c_ld = K;
    a.sa = sdy;
    a.sb = w->scales;
    a.Nout = K;
    a.Kc = N;
    a.E = E;
    a.total_rows = total_M;
    a.sizes = group_sizes;
    attach_ws(a, ws);
    GemmLaunch L;
    L.kind = FIXED_M;
    L.elem = EL_FP8;
    L.a_kc = L.b_kc = true;
    e = launch_gemm(L, a, S(stream));
    if (e != hipSuccess) return hip_status(e, "gmm_bwd_fp8 dx");
  }
  if (dw && total_M == 0) {
    e = launch_zero_fill(dw, (int64_t)E * K * N * 2, S(stream));
    if (e != hipSuccess) return hip_status(e, "gmm_bwd_fp8 dw zero fill");
  } else if (dw) {
    GemmArgs a = blank_args();
    a.A = xc;
    a.a_ld = ldc;
    a.B = dyc;
    a.b_ld = ldc;
    a.b_gs = 0;
    a.C = dw;
    a.c_ld = N;
    a.c_gs = (int64_t)K * N;
    a.sa = sxc;
    a.sb = sdyc;
    a.Mout = K;
    a.Nout = N;
    a.E = E;
    a.total_rows = total_M;
    a.sizes = group_sizes;
    attach_ws(a, ws);
    GemmLaunch L;
    L.kind = DYNAMIC_K;
    L.elem = EL_FP8;
    L.a_kc = L.b_kc = true;
    e = launch_gemm(L, a, S(stream));
    if (e != hipSuccess) return hip_status(e, "gmm_bwd_fp8 dw");
  }
  return ok();
}

int gmm_fwd_f8i4(const uint8_t* xq, const float* sx, const uint8_t* w4, const void* sw,
                 const int32_t* group_sizes, int32_t E, int64_t total_M, int32_t K, int32_t N, void* y, void* ws,
                 size_t ws_bytes, mg_stream_t stream) {
  int rc = check_common(group_sizes, E, total_M, ws, ws_bytes);
  if (rc) return rc;
  if (K < 1 || N < 1) return fail(MG_EINVAL, "K and N must be positive");
  if (K % 128 || N % 8) return fail(MG_EUNSUPPORTED, "K must be a multiple of 128 and N of 8");
  if ((rc = check_extents(total_M, K, N, 1))) return rc;   // 32-bit offsets into X and one expert's weights
  if (total_M == 0) return ok();
  if (!xq || !sx || !w4 || !sw || !y) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(xq) || !aligned16(w4)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  const int bm = 32;
  GemmArgs a = blank_args();
  a.A = xq;
  a.a_ld = K;
  a.B = w4;
  a.s4 = reinterpret_cast<const uint16_t*>(sw);
  a.sa = sx;
  a.C = y;
  a.c_ld = N;
  a.Nout = N;
  a.Kc = K;
  a.E = E;
  a.total_rows = total_M;
  a.sizes = group_sizes;
  attach_ws(a, ws);
  return hip_status(launch_f8i4(a, fixed_m_capacity(total_M, E, bm), S(stream)), "gmm_fwd_f8i4");
}

// ---------------------------------------------------------------------------
// quantizers
// ---------------------------------------------------------------------------

int quantize_rowwise_fp8(const void* x, int64_t rows, int32_t cols, int64_t ld, uint8_t* q, float* scales,
                         mg_stream_t stream) {
  if (rows < 0 || cols < 1) return fail(MG_EINVAL, "rows must be >= 0 and cols >= 1");
  if (ld < cols) return fail(MG_EINVAL, "ld < cols");
  if (cols % 8 || ld % 8) return fail(MG_EUNSUPPORTED, "cols and ld must be multiples of 8");
  if (rows == 0) return ok();
  if (!x || !q || !scales) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7)) return fail(MG_EUNSUPPORTED, "x must be 16-byte and q 8-byte aligned");
  return hip_status(launch_quant_rowwise(reinterpret_cast<const uint16_t*>(x), rows, cols, ld, q, scales, S(stream)),
                    "quantize_rowwise_fp8");
}

int quantize_rowwise_fp8_gather(const void* x, int64_t T, const int32_t* sorted_token_ids, int32_t top_k,
                                int64_t rows, int32_t cols, uint8_t* q, float* scales, mg_stream_t stream) {
  if (rows < 0 || T < 0 || cols < 1) return fail(MG_EINVAL, "rows and T must be >= 0 and cols >= 1");
  if (top_k < 1) return fail(MG_EINVAL, "top_k must be >= 1");
  if (cols % 8) return fail(MG_EUNSUPPORTED, "cols must be a multiple of 8");
  if (rows == 0) return ok();
  if (!sorted_token_ids || !q || !scales || (T > 0 && !x)) return fail(MG_EINVAL, "NULL tensor argument");
  if ((x && !aligned16(x)) || (reinterpret_cast<uintptr_t>(q) & 7))
    return fail(MG_EUNSUPPORTED, "x must be 16-byte and q 8-byte aligned");
  return hip_status(launch_quant_rowwise(reinterpret_cast<const uint16_t*>(x), rows, cols, cols, q, scales,
                                         S(stream), sorted_token_ids, top_k, T * (int64_t)top_k),
                    "quantize_rowwise_fp8_gather");
}

// Largest column count of a colwise operand: a 1024-row block's byte
// offsets (row * cols * 2) stay below 2^31.
constexpr int32_t kColwiseMaxCols = 1 << 20;

size_t quantize_colwise_workspace_bytes(int32_t G, int64_t rows, int32_t cols_a, int32_t cols_b) {
  const int32_t g = G < 1 ? 1 : (G > MG_MAX_EXPERTS ? MG_MAX_EXPERTS : G);
  const int64_t r = rows < 0 ? 0 : (rows >= kMaxRows ? kMaxRows - 1 : rows);
  const int32_t ca = cols_a < 1 ? 1 : (cols_a > kColwiseMaxCols ? kColwiseMaxCols : cols_a);
  const int32_t cb = cols_b < 1 ? 0 : (cols_b > kColwiseMaxCols ? kColwiseMaxCols : cols_b);
  return (size_t)colwise_layout(g, r, ca, cb).total;
}

int quantize_colwise_per_group_fp8(const void* a, int32_t cols_a, const void* b, int32_t cols_b,
                                   const int32_t* group_sizes, int32_t G, int64_t rows, int64_t ld, uint8_t* qa,
                                   float* sa, uint8_t* qb, float* sb, void* ws, size_t ws_bytes,
                                   mg_stream_t stream) {
  if (G < 1 || G > MG_MAX_EXPERTS) return fail(MG_EINVAL, "G=%d outside [1, %d]", G, MG_MAX_EXPERTS);
  if (rows < 0 || rows >= kMaxRows) return fail(MG_EINVAL, "rows out of range");
  if (ld < rows || ld >= 2 * kMaxRows) return fail(MG_EINVAL, "ld=%lld below rows or out of range", (long long)ld);
  if (!a || !qa || !sa || !group_sizes) return fail(MG_EINVAL, "NULL tensor argument");
  const bool dual = b != nullptr;
  if (dual != (qb != nullptr) || dual != (sb != nullptr)) return fail(MG_EINVAL, "b, qb, sb must be all set or all NULL");
  if (cols_a < 1 || (dual && cols_b < 1)) return fail(MG_EINVAL, "cols must be positive");
  if (cols_a % 8 || (dual && cols_b % 8)) return fail(MG_EUNSUPPORTED, "cols must be multiples of 8");
  if (cols_a > kColwiseMaxCols || (dual && cols_b > kColwiseMaxCols))
    return fail(MG_EUNSUPPORTED, "cols above 2^20");
  if (!aligned16(a) || (dual && !aligned16(b))) return fail(MG_EUNSUPPORTED, "inputs must be 16-byte aligned");
  const ColwiseLayout L = colwise_layout(G, rows, cols_a, dual ? cols_b : 0);
  if (L.items + 65536 >= kMaxRows) return fail(MG_EUNSUPPORTED, "too many (row block, column block) pairs");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) || ws_bytes < (size_t)L.total)
    return fail(MG_EWORKSPACE, "colwise workspace missing, not 256-byte aligned or below %lld bytes",
                (long long)L.total);
  return hip_status(launch_quant_colwise(reinterpret_cast<const uint16_t*>(a), cols_a,
                                         reinterpret_cast<const uint16_t*>(b), dual ? cols_b : 0, group_sizes, G,
                                         rows, ld, qa, sa, qb, sb, ws, S(stream)),
                    "quantize_colwise_per_group_fp8");
}

int quantize_int4_weights(const void* w, int32_t E, int32_t K, int32_t N, uint8_t* w4, void* sw,
                          mg_stream_t stream) {
  if (E < 1 || E > 65535 || K < 1 || N < 1) return fail(MG_EINVAL, "E, K, N out of range");
  if (K % 128 || N % 8) return fail(MG_EUNSUPPORTED, "K % 128 == 0 and N % 8 == 0 required");
  if (!w || !w4 || !sw) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(w4)) return fail(MG_EUNSUPPORTED, "w4 must be 16-byte aligned");
  return hip_status(launch_quant_int4(reinterpret_cast<const uint16_t*>(w), E, K, N, w4,
                                      reinterpret_cast<uint16_t*>(sw), S(stream)),
                    "quantize_int4_weights");
}

// ---------------------------------------------------------------------------
// permutation
// ---------------------------------------------------------------------------

int64_t moe_sorted_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m) {
  if (T < 0 || top_k < 1 || E < 1 || block_m < 1) return 0;
  return T * top_k + (int64_t)E * (block_m - 1);
}

int64_t moe_block_capacity(int64_t T, int32_t top_k, int32_t E, int32_t block_m) {
  if (T < 0 || top_k < 1 || E < 1 || block_m < 1) return 0;
  return cdiv(moe_sorted_capacity(T, top_k, E, block_m), block_m);
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t top_k, int32_t E) {
  if (T < 0 || top_k < 1 || E < 1 || E > MG_MAX_EXPERTS) return 0;
  return (size_t)perm_workspace_bytes(T * top_k, E);
}

int moe_permute(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E, int32_t block_m, const void* x,
                int32_t hidden, int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                int32_t* inv_pos, int32_t* padded_group_sizes, void* x_sorted, void* ws, size_t ws_bytes,
                mg_stream_t stream) {
  if (E < 1 || E > MG_MAX_EXPERTS) return fail(MG_EINVAL, "E=%d outside [1, %d]", E, MG_MAX_EXPERTS);
  if (T < 0 || top_k < 1 || block_m < 1) return fail(MG_EINVAL, "T >= 0, top_k >= 1, block_m >= 1 required");
  if (T * top_k > (1 << 24)) return fail(MG_EUNSUPPORTED, "T * top_k must be <= 2^24");
  const int64_t cap = moe_sorted_capacity(T, top_k, E, block_m);
  if (cap >= kMaxRows) return fail(MG_EUNSUPPORTED, "sorted capacity exceeds int32");
  if (!sorted_token_ids || !expert_ids || !num_tokens_post_padded || !inv_pos || !padded_group_sizes)
    return fail(MG_EINVAL, "NULL output argument");
  if (T > 0 && !topk_ids) return fail(MG_EINVAL, "topk_ids is NULL");
  if ((x == nullptr) != (x_sorted == nullptr)) return fail(MG_EINVAL, "x and x_sorted must both be set or NULL");
  if (x && (hidden < 1 || hidden % 8)) return fail(MG_EUNSUPPORTED, "hidden must be a positive multiple of 8");
  if (x && (!aligned16(x) || !aligned16(x_sorted))) return fail(MG_EUNSUPPORTED, "x, x_sorted must be 16-byte aligned");
  const size_t need = moe_permute_workspace_bytes(T, top_k, E);
  if (!ws || ws_bytes < need) return fail(MG_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return hip_status(launch_moe_permute_ws(topk_ids, T, top_k, E, block_m, reinterpret_cast<const uint16_t*>(x),
                                          hidden, sorted_token_ids, expert_ids, num_tokens_post_padded, inv_pos,
                                          padded_group_sizes, reinterpret_cast<uint16_t*>(x_sorted), cap,
                                          moe_block_capacity(T, top_k, E, block_m), ws, S(stream)),
                    "moe_permute");
}

int moe_unpermute(const void* y_sorted, const int32_t* inv_pos, const float* topk_weights, int64_t T,
                  int32_t top_k, int32_t hidden, void* out, mg_stream_t stream) {
  if (T < 0 || top_k < 1 || hidden < 1) return fail(MG_EINVAL, "T >= 0, top_k >= 1, hidden >= 1 required");
  if (hidden % 8) return fail(MG_EUNSUPPORTED, "hidden must be a multiple of 8");
  if (T == 0) return ok();
  if (!y_sorted || !inv_pos || !out) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(y_sorted) || !aligned16(out)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  return hip_status(launch_moe_unpermute(reinterpret_cast<const uint16_t*>(y_sorted), inv_pos, topk_weights, T,
                                         top_k, hidden, reinterpret_cast<uint16_t*>(out), S(stream)),
                    "moe_unpermute");
}

int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t top_k, int32_t renormalize,
                   int32_t* topk_ids, float* topk_weights, mg_stream_t stream) {
  if (T < 0) return fail(MG_EINVAL, "T=%lld must be >= 0", (long long)T);
  if (E < 1 || E > MG_MAX_EXPERTS) return fail(MG_EINVAL, "E=%d outside [1, %d]", E, MG_MAX_EXPERTS);
  if (top_k < 1 || top_k > E || top_k > 64) return fail(MG_EINVAL, "top_k=%d outside [1, min(E, 64)]", top_k);
  if (T == 0) return ok();
  if (!logits || !topk_ids || !topk_weights) return fail(MG_EINVAL, "NULL tensor argument");
  return hip_status(launch_route_topk(logits, T, E, top_k, renormalize != 0, topk_ids, topk_weights, S(stream)),
                    "moe_route_topk");
}

int silu_mul(const void* h, int64_t rows, int32_t inter, void* act, mg_stream_t stream) {
  if (rows < 0 || inter < 1) return fail(MG_EINVAL, "rows >= 0 and inter >= 1 required");
  if (inter % 8) return fail(MG_EUNSUPPORTED, "inter must be a multiple of 8");
  if (rows == 0) return ok();
  if (!h || !act) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(h) || !aligned16(act)) return fail(MG_EUNSUPPORTED, "tensors must be 16-byte aligned");
  return hip_status(launch_silu_mul(reinterpret_cast<const uint16_t*>(h), rows, inter,
                                    reinterpret_cast<uint16_t*>(act), S(stream)),
                    "silu_mul");
}

int silu_mul_quantize_rowwise_fp8(const void* h, int64_t rows, int32_t inter, void* act, uint8_t* q, float* scales,
                                  mg_stream_t stream) {
  if (rows < 0 || inter < 1) return fail(MG_EINVAL, "rows >= 0 and inter >= 1 required");
  if (inter % 8) return fail(MG_EUNSUPPORTED, "inter must be a multiple of 8");
  if (rows >= kMaxRows) return fail(MG_EINVAL, "rows must be below 2^31");
  if (rows == 0) return ok();
  if (!h || !q || !scales) return fail(MG_EINVAL, "NULL tensor argument");
  if (!aligned16(h) || (act && !aligned16(act)) || (reinterpret_cast<uintptr_t>(q) & 7))
    return fail(MG_EUNSUPPORTED, "h and act must be 16-byte and q 8-byte aligned");
  return hip_status(launch_silu_mul_quant(reinterpret_cast<const uint16_t*>(h), rows, inter,
                                          reinterpret_cast<uint16_t*>(act), q, scales, S(stream)),
                    "silu_mul_quantize_rowwise_fp8");
}

}  // extern "C"
