"""fp64 CPU oracle for the MoE grouped-GEMM path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library; the C source (``moe_oracle.c``) writes every definition out from
the source pages:

* grouped GEMM forward / dX / dW -- grouped_gemm PR "Support GPU-resident
  batch sizes" (description: gmm(x, w, batch_sizes) and the gradient of
  out.sum(); review thread: dynamic-k problems sorted by k descending,
  outputs of K=0 problems zeroed);
* work lists skipping empty groups -- FBGEMM PR "F8I4 Grouped Gemm
  Optimization for Sparse M" (summary: grouped gemm over min(total_M, groups));
* FP8 rowwise and per-group colwise quantizers -- torchao commit "Optimize
  FP8 MoE backward pass" (commit message; colwise kernel in
  bench_colwise_block_configs.py);
* router (softmax, top-k, optional renormalization), token permutation,
  SiLU-and-mul and the top-k weighted sum -- applied-ai issue "Column-major
  fused MoE" (moe_align_block_size docstring and example, fused_moe).

Pins: every function here is checked by the ``-m "not gpu"`` tests against
closed forms, library routines, brute force and the pages' worked example.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = ctypes.CDLL(_build.LIB)
        _declare(_LIB)
    return _LIB


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def _declare(lib):
    sig = {
        "or_set_threads": (ctypes.c_int, [ctypes.c_int]),
        "or_bf16_to_f64": (None, [_P, _I64, _P]),
        "or_f64_to_bf16": (None, [_P, _I64, _P]),
        "or_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
        "or_e4m3_to_f64": (None, [_P, _I64, _P]),
        "or_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "or_e4m3_encode_array": (None, [_P, _I64, _P]),
        "or_offsets": (None, [_P, _I32, _P]),
        "or_worklist_fixed_m": (_I64, [_P, _I32, _I32, _P, _I64]),
        "or_worklist_dynamic_k": (None, [_P, _I32, _P]),
        "or_gmm_fwd": (None, [_P, _P, _P, _I32, _I64, _I64, _I64, _P]),
        "or_gmm_dx": (None, [_P, _P, _P, _I32, _I64, _I64, _I64, _P]),
        "or_gmm_dw": (None, [_P, _P, _P, _I32, _I64, _I64, _I64, _P]),
        "or_fp8_scale_from_amax": (ctypes.c_float, [ctypes.c_double]),
        "or_quant_rowwise": (None, [_P, _I64, _I64, _P, _P]),
        "or_quant_colwise": (None, [_P, _I64, _I64, _P, _I32, _P, _P]),
        "or_dequant_rowwise": (None, [_P, _P, _I64, _I64, _P]),
        "or_dequant_colwise": (None, [_P, _P, _I64, _I64, _P, _I32, _P]),
        "or_quant_int4": (None, [_P, _I32, _I64, _I64, _I32, _P, _P]),
        "or_dequant_int4": (None, [_P, _P, _I32, _I64, _I64, _I32, _P]),
        "or_moe_align": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _I64, _P, _I64, _P, _P, _P]),
        "or_gather_rows": (None, [_P, _I64, _I32, _I64, _P, _I64, _P]),
        "or_silu_mul": (None, [_P, _I64, _I64, _P]),
        "or_unpermute": (None, [_P, _P, _P, _I64, _I32, _I64, _P]),
        "or_route_topk": (None, [_P, _I64, _I32, _I32, _I32, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def _c(a, dtype):
    """Contiguous array of the given dtype (no copy if already right)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def set_threads(n: int) -> int:
    """Set the OpenMP thread count used by the GEMM loops; returns it."""
    return _lib().or_set_threads(int(n))


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _lib().or_bf16_to_f64(_ptr(bits), bits.size, _ptr(out))
    return out


def f64_to_bf16(x):
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _lib().or_f64_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_to_f64(codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _lib().or_e4m3_to_f64(_ptr(codes), codes.size, _ptr(out))
    return out


def e4m3_encode(x):
    """Encode float32 values (already within [-448, 448]) to e4m3fn codes."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _lib().or_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def fp8_scale_from_amax(amax: float) -> float:
    return float(_lib().or_fp8_scale_from_amax(float(amax)))


# --------------------------------------------------------------------------
# Offsets and work lists
# --------------------------------------------------------------------------

def offsets(sizes):
    sizes = _c(sizes, np.int32)
    out = np.empty(sizes.size + 1, np.int64)
    _lib().or_offsets(_ptr(sizes), sizes.size, _ptr(out))
    return out


def worklist_fixed_m(sizes, bm: int):
    """(count, entries[count, 4]) of the fixed-M work list."""
    sizes = _c(sizes, np.int32)
    total = int(sizes.astype(np.int64).sum())
    cap = total // bm + min(total, sizes.size) + 1
    ent = np.zeros((cap, 4), np.int32)
    n = _lib().or_worklist_fixed_m(_ptr(sizes), sizes.size, int(bm), _ptr(ent), cap)
    return int(n), ent[: min(n, cap)].copy()


def worklist_dynamic_k(sizes):
    sizes = _c(sizes, np.int32)
    ent = np.zeros((sizes.size, 4), np.int32)
    _lib().or_worklist_dynamic_k(_ptr(sizes), sizes.size, _ptr(ent))
    return ent


# --------------------------------------------------------------------------
# Grouped GEMMs in fp64 (operands given as fp64; W as [E, K, N])
# --------------------------------------------------------------------------

def _check_sizes(sizes, M):
    sizes = _c(sizes, np.int32)
    if (sizes < 0).any() or int(sizes.astype(np.int64).sum()) > M:
        raise ValueError("group sizes must be >= 0 and sum to at most M")
    return sizes


def gmm_fwd(X, W, sizes):
    X = _c(X, np.float64)
    W = _c(W, np.float64)
    E, K, N = W.shape
    M = X.shape[0]
    sizes = _check_sizes(sizes, M)
    Y = np.empty((M, N), np.float64)
    _lib().or_gmm_fwd(_ptr(X), _ptr(W), _ptr(sizes), E, M, K, N, _ptr(Y))
    return Y


def gmm_dx(dY, W, sizes):
    dY = _c(dY, np.float64)
    W = _c(W, np.float64)
    E, K, N = W.shape
    M = dY.shape[0]
    sizes = _check_sizes(sizes, M)
    dX = np.empty((M, K), np.float64)
    _lib().or_gmm_dx(_ptr(dY), _ptr(W), _ptr(sizes), E, M, K, N, _ptr(dX))
    return dX


def gmm_dw(X, dY, sizes):
    X = _c(X, np.float64)
    dY = _c(dY, np.float64)
    M, K = X.shape
    N = dY.shape[1]
    sizes = _check_sizes(sizes, M)
    E = sizes.size
    dW = np.empty((E, K, N), np.float64)
    _lib().or_gmm_dw(_ptr(X), _ptr(dY), _ptr(sizes), E, M, K, N, _ptr(dW))
    return dW


def gmm_fwd_bf16(x_bits, w_bits, sizes, trans_b=False):
    """Forward from bf16 bit patterns; W is [E,K,N], or [E,N,K] if trans_b."""
    W = bf16_to_f64(w_bits)
    if trans_b:
        W = np.ascontiguousarray(W.transpose(0, 2, 1))
    return gmm_fwd(bf16_to_f64(x_bits), W, sizes)


def gmm_dx_bf16(dy_bits, w_bits, sizes, trans_b=False):
    W = bf16_to_f64(w_bits)
    if trans_b:
        W = np.ascontiguousarray(W.transpose(0, 2, 1))
    return gmm_dx(bf16_to_f64(dy_bits), W, sizes)


def gmm_dw_bf16(x_bits, dy_bits, sizes):
    return gmm_dw(bf16_to_f64(x_bits), bf16_to_f64(dy_bits), sizes)


# --------------------------------------------------------------------------
# FP8 quantizers
# --------------------------------------------------------------------------

def quant_rowwise(x_bits):
    """bf16 [R, C] -> (e4m3 codes [R, C], fp32 scales [R])."""
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    q = np.empty((R, C), np.uint8)
    s = np.empty(R, np.float32)
    _lib().or_quant_rowwise(_ptr(x), R, C, _ptr(q), _ptr(s))
    return q, s


def quant_colwise(x_bits, sizes):
    """bf16 [R, C] + group sizes [G] -> (codes column-major [C, R], scales [G, C]).

    Codes of rows that belong to no group (beyond the sum of the sizes) are
    left as 0 here; they are not part of the result.
    """
    x = _c(x_bits, np.uint16)
    R, C = x.shape
    sizes = _check_sizes(sizes, R)
    G = sizes.size
    q = np.zeros((C, R), np.uint8)
    s = np.empty((G, C), np.float32)
    _lib().or_quant_colwise(_ptr(x), R, C, _ptr(sizes), G, _ptr(q), _ptr(s))
    return q, s


def dequant_rowwise(q, s):
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    R, C = q.shape
    out = np.empty((R, C), np.float64)
    _lib().or_dequant_rowwise(_ptr(q), _ptr(s), R, C, _ptr(out))
    return out


def dequant_colwise(q_colmajor, s, sizes):
    q = _c(q_colmajor, np.uint8)
    s = _c(s, np.float32)
    C, R = q.shape
    sizes = _check_sizes(sizes, R)
    out = np.zeros((R, C), np.float64)
    _lib().or_dequant_colwise(_ptr(q), _ptr(s), R, C, _ptr(sizes), sizes.size, _ptr(out))
    return out


# --------------------------------------------------------------------------
# int4 weights
# --------------------------------------------------------------------------

def quant_int4(W, group=128):
    """fp64 W [E, K, N] -> (packed uint8 [E, N, K/2], bf16 scale bits [E, K/group, N])."""
    W = _c(W, np.float64)
    E, K, N = W.shape
    if K % group or K % 2:
        raise ValueError("K must be a multiple of the group size and even")
    packed = np.zeros((E, N, K // 2), np.uint8)
    scales = np.empty((E, K // group, N), np.uint16)
    _lib().or_quant_int4(_ptr(W), E, K, N, group, _ptr(packed), _ptr(scales))
    return packed, scales


def dequant_int4(packed, scales, group=128):
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    E, N, K2 = packed.shape
    K = 2 * K2
    W = np.empty((E, K, N), np.float64)
    _lib().or_dequant_int4(_ptr(packed), _ptr(scales), E, K, N, group, _ptr(W))
    return W


# --------------------------------------------------------------------------
# Token permutation for the fused path
# --------------------------------------------------------------------------

def sorted_capacity(T, k, E, block_m):
    return T * k + E * (block_m - 1)


def block_capacity(T, k, E, block_m):
    return (sorted_capacity(T, k, E, block_m) + block_m - 1) // block_m


def moe_align(topk_ids, E, block_m):
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    cap = sorted_capacity(T, k, E, block_m)
    nblk = block_capacity(T, k, E, block_m)
    sorted_ids = np.empty(cap, np.int32)
    expert_ids = np.empty(nblk, np.int32)
    ntpp = np.zeros(1, np.int32)
    inv = np.empty(T * k, np.int32)
    padded = np.empty(E, np.int32)
    rc = _lib().or_moe_align(_ptr(ids), T, k, E, block_m, _ptr(sorted_ids), cap,
                             _ptr(expert_ids), nblk, _ptr(ntpp), _ptr(inv), _ptr(padded))
    if rc != 0:
        raise ValueError("expert id out of range")
    return dict(sorted_token_ids=sorted_ids, expert_ids=expert_ids,
                num_tokens_post_padded=int(ntpp[0]), inv=inv, padded_sizes=padded)


def gather_rows(x_bits, topk_k, sorted_ids):
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    ids = _c(sorted_ids, np.int32)
    out = np.empty((ids.size, H), np.uint16)
    _lib().or_gather_rows(_ptr(x), T, topk_k, H, _ptr(ids), ids.size, _ptr(out))
    return out


def silu_mul(h):
    h = _c(h, np.float64)
    R, I2 = h.shape
    act = np.empty((R, I2 // 2), np.float64)
    _lib().or_silu_mul(_ptr(h), R, I2 // 2, _ptr(act))
    return act


def route_topk(logits, top_k, renormalize=False):
    """fp32 logits [T, E] -> (ids int32 [T, top_k], weights fp64 [T, top_k]):
    the top_k experts by probability, descending, ties to the lower index;
    weights softmax probabilities (divided by their sum if renormalize)."""
    z = _c(logits, np.float32)
    T, E = z.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float64)
    _lib().or_route_topk(_ptr(z), T, E, top_k, int(bool(renormalize)), _ptr(ids), _ptr(w))
    return ids, w


def unpermute(Y, inv, weights, T, k):
    Y = _c(Y, np.float64)
    inv = _c(inv, np.int32)
    w = None if weights is None else _c(weights, np.float32)
    H = Y.shape[1]
    out = np.empty((T, H), np.float64)
    _lib().or_unpermute(_ptr(Y), _ptr(inv), _ptr(w), T, k, H, _ptr(out))
    return out


def fused_moe(x_bits, w1_bits, w2_bits, topk_ids, topk_weights, block_m):
    """Token-sorted fused MoE, rounding to bf16 only where the pages keep a
    bf16 intermediate (the first GEMM's output, the activation, the second
    GEMM's output).  The top-k weighted sum is returned in fp64, unrounded:
    callers compare it with the library's bf16 output, whose own final
    rounding the tolerance covers.  W1 is [E, H, 2I], W2 is [E, I, H]."""
    E = w1_bits.shape[0]
    T, k = topk_ids.shape
    al = moe_align(topk_ids, E, block_m)
    xs = gather_rows(x_bits, k, al["sorted_token_ids"])
    sizes = al["padded_sizes"]
    h1 = f64_to_bf16(gmm_fwd_bf16(xs, w1_bits, sizes))
    act = f64_to_bf16(silu_mul(bf16_to_f64(h1)))
    y2 = f64_to_bf16(gmm_fwd_bf16(act, w2_bits, sizes))
    out = unpermute(bf16_to_f64(y2), al["inv"], topk_weights, T, k)
    return out, al
