"""MI355X (gfx950) MoE grouped GEMM: thin Python binding over libmoegemm.so.

Every function here only marshals arguments (torch tensors -> device
pointers, the current HIP stream) and calls the C ABI declared in
``include/moe_gemm.h``; every step of the computation runs in the library's
HIP kernels.  PyTorch provides device memory and streams.  There is no CPU
fallback: if the library is missing or a call fails, an exception is raised.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoegemm.so")

MG_OK, MG_EINVAL, MG_EUNSUPPORTED, MG_EWORKSPACE, MG_EHIP = 0, -1, -2, -3, -4
MG_WL_FIXED_M, MG_WL_DYNAMIC_K = 0, 1
MAX_EXPERTS = 1024

_lib = None


class MoeGemmError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class FP8Weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("ld", ctypes.c_int64), ("expert_stride", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_SIGS = {
    "mg_workspace_bytes": (_SZ, [_I32, _I64]),
    "mg_workspace_error": (_I32, [_P]),
    "mg_workspace_clear": (ctypes.c_int, [_P, _P]),
    "gmm_build_worklist": (ctypes.c_int, [_I32, _P, _I32, _I64, _I32, _P, _P, _P, _I64, _P]),
    "gmm_fwd": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "gmm_fwd_noalloc": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I32, _I32, _I32, _P, _P]),
    "gmm_fwd_gather": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, _I32, _I64, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "gmm_fwd_silu_mul": (ctypes.c_int, [_P, _I64, _P, _I32, _P, _P, _I32, _I64, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "gmm_bwd": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "gmm_fwd_fp8": (ctypes.c_int, [_P, _P, ctypes.POINTER(FP8Weight), _P, _I32, _I64, _I32, _I32, _P, _P, _SZ, _P]),
    "gmm_bwd_fp8": (ctypes.c_int, [_P, _P, ctypes.POINTER(FP8Weight), _P, _P, _P, _P, _I64, _P, _I32, _I64, _I32,
                                   _I32, _P, _P, _P, _SZ, _P]),
    "gmm_fwd_f8i4": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _P, _SZ, _P]),
    "quantize_rowwise_fp8": (ctypes.c_int, [_P, _I64, _I32, _I64, _P, _P, _P]),
    "quantize_rowwise_fp8_gather": (ctypes.c_int, [_P, _I64, _P, _I32, _I64, _I32, _P, _P, _P]),
    "quantize_colwise_workspace_bytes": (_SZ, [_I32, _I64, _I32, _I32]),
    "quantize_colwise_per_group_fp8": (ctypes.c_int, [_P, _I32, _P, _I32, _P, _I32, _I64, _I64, _P, _P, _P, _P,
                                                      _P, _SZ, _P]),
    "quantize_int4_weights": (ctypes.c_int, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_sorted_capacity": (_I64, [_I64, _I32, _I32, _I32]),
    "moe_block_capacity": (_I64, [_I64, _I32, _I32, _I32]),
    "moe_permute_workspace_bytes": (_SZ, [_I64, _I32, _I32]),
    "moe_permute": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_unpermute": (ctypes.c_int, [_P, _P, _P, _I64, _I32, _I32, _P, _P]),
    "silu_mul": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    "silu_mul_quantize_rowwise_fp8": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P, _P]),
    "moe_route_topk": (ctypes.c_int, [_P, _I64, _I32, _I32, _I32, _P, _P, _P]),
    "mg_last_error": (ctypes.c_char_p, []),
    "mg_version": (ctypes.c_char_p, []),
    "mg_last_gemm_tile_m": (_I32, []),
}

EXPORTS = tuple(_SIGS)


def lib():
    """Load libmoegemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python moe_grouped_gemm_device_amd/build.py")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != MG_OK:
        raise MoeGemmError(name, rc, lib().mg_last_error().decode())
    return rc


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, ndim=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def last_gemm_tile_m():
    """Row-tile height (128 or 256) of this thread's most recent grouped-GEMM
    launch (0 before the first); diagnostics."""
    return int(lib().mg_last_gemm_tile_m())


def workspace_bytes(E, total_M):
    return int(lib().mg_workspace_bytes(int(E), int(total_M)))


def workspace(E, total_M, device="cuda"):
    """A fresh, zeroed device workspace big enough for any grouped-GEMM call
    with E, total_M (its size does not depend on them)."""
    return torch.zeros(max(workspace_bytes(E, total_M), 256), dtype=torch.uint8, device=device)


_WS_CACHE = {}


def default_workspace(device=None, stream=None):
    """The workspace a call made without ``ws`` uses: one per (device,
    stream), zeroed once when first needed and kept.  Its arrival counters
    return to zero after every call, so it never needs clearing again, and
    calls on one stream never overlap, so they may share it.  It cannot be
    created during graph capture: make one eager call on the stream first,
    or pass ``ws``."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    s = torch.cuda.current_stream(idx) if stream is None else stream
    key = (idx, s.cuda_stream)
    ws = _WS_CACHE.get(key)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("no workspace for this stream yet and the stream is capturing: "
                               "make one eager call on it first, or pass ws")
        with torch.cuda.device(idx), torch.cuda.stream(s):
            ws = torch.zeros(max(workspace_bytes(1, 0), 256), dtype=torch.uint8, device=torch.device("cuda", idx))
        _WS_CACHE[key] = ws
    return ws


def workspace_error(ws):
    return int(lib().mg_workspace_error(_ptr(ws)))


def workspace_clear(ws, stream=None):
    _call("mg_workspace_clear", _ptr(ws), _stream(stream))


# --------------------------------------------------------------------------
# argument builder
# --------------------------------------------------------------------------

def build_worklist(kind, group_sizes, total_M, bm, stream=None):
    """Run the device builder; returns (offs int32[E+1], count int32[1], entries int32[cap,4])."""
    _need(group_sizes, torch.int32, "group_sizes", 1)
    E = group_sizes.numel()
    cap = (total_M // bm + min(total_M, E)) if kind == MG_WL_FIXED_M else E
    cap = max(cap, 1)
    dev = group_sizes.device
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    entries = torch.empty(cap, 4, dtype=torch.int32, device=dev)
    _call("gmm_build_worklist", int(kind), _ptr(group_sizes), E, int(total_M), int(bm), _ptr(offs),
          _ptr(count), _ptr(entries), cap, _stream(stream))
    return offs, count, entries


# --------------------------------------------------------------------------
# bf16 grouped GEMM
# --------------------------------------------------------------------------

def gmm_fwd(x, w, group_sizes, trans_b=False, out=None, ws=None, stream=None):
    """y[r] = x[r] @ w[g(r)] (w [E,K,N], or [E,N,K] with trans_b)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w, torch.bfloat16, "w", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = x.shape
    E = w.shape[0]
    N = w.shape[1] if trans_b else w.shape[2]
    if (w.shape[2] if trans_b else w.shape[1]) != K or group_sizes.numel() != E:
        raise ValueError("shape mismatch between x, w and group_sizes")
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, torch.bfloat16, "out", 2)
    ws = default_workspace(x.device, stream) if ws is None else ws
    _call("gmm_fwd", _ptr(x), _ptr(w), _ptr(group_sizes), E, M, K, N, int(bool(trans_b)), _ptr(y),
          _ptr(ws), ws.numel(), _stream(stream))
    return y


def gmm_fwd_noalloc(x, w, group_sizes, out, trans_b=False, stream=None):
    """gmm_fwd with the library's own fixed scratch instead of a workspace:
    the call allocates nothing (out is required).  Calls on one device must
    not overlap in time."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w, torch.bfloat16, "w", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    _need(out, torch.bfloat16, "out", 2)
    M, K = x.shape
    E = w.shape[0]
    N = w.shape[1] if trans_b else w.shape[2]
    if (w.shape[2] if trans_b else w.shape[1]) != K or group_sizes.numel() != E or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch between x, w, group_sizes and out")
    _call("gmm_fwd_noalloc", _ptr(x), _ptr(w), _ptr(group_sizes), E, M, K, N, int(bool(trans_b)), _ptr(out),
          _stream(stream))
    return out


def gmm_fwd_gather(x, sorted_token_ids, top_k, w, group_sizes, trans_b=False, out=None, ws=None, stream=None):
    """y[r] = x[sorted_token_ids[r] // top_k] @ w[g(r)] over the token-sorted
    rows (zero rows for the padding sentinel); y has one row per entry of
    sorted_token_ids.  The same result as gmm_fwd over moe_permute's
    x_sorted, without that copy."""
    _need(x, torch.bfloat16, "x", 2)
    _need(sorted_token_ids, torch.int32, "sorted_token_ids", 1)
    _need(w, torch.bfloat16, "w", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    T, K = x.shape
    M = sorted_token_ids.numel()
    E = w.shape[0]
    N = w.shape[1] if trans_b else w.shape[2]
    if (w.shape[2] if trans_b else w.shape[1]) != K or group_sizes.numel() != E:
        raise ValueError("shape mismatch between x, w and group_sizes")
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, torch.bfloat16, "out", 2)
    if y.shape[0] < M:
        raise ValueError("out has fewer rows than sorted_token_ids")
    ws = default_workspace(x.device, stream) if ws is None else ws
    _call("gmm_fwd_gather", _ptr(x), T, _ptr(sorted_token_ids), int(top_k), _ptr(w), _ptr(group_sizes), E, M, K,
          N, int(bool(trans_b)), _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    return y


def gmm_fwd_silu_mul(x, w1, group_sizes, sorted_token_ids=None, top_k=1, trans_b=False, out=None, ws=None,
                     stream=None):
    """act = silu(h[:, :I]) * h[:, I:] with h = A @ w1[g] rounded to bf16,
    in one kernel (w1 [E, K, 2I], or [E, 2I, K] with trans_b).  A is x (one
    row per output row) or, with sorted_token_ids, x[sorted_token_ids //
    top_k] with zero padding rows."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w1, torch.bfloat16, "w1", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    T, K = x.shape
    if trans_b:
        E, N2, K2 = w1.shape
    else:
        E, K2, N2 = w1.shape
    if K2 != K or N2 % 2 or group_sizes.numel() != E:
        raise ValueError("shape mismatch between x, w1 and group_sizes")
    I = N2 // 2
    if sorted_token_ids is not None:
        _need(sorted_token_ids, torch.int32, "sorted_token_ids", 1)
        M = sorted_token_ids.numel()
    else:
        M = T
    y = torch.empty(M, I, dtype=torch.bfloat16, device=x.device) if out is None else out
    _need(y, torch.bfloat16, "out", 2)
    if y.shape[0] < M or y.shape[1] != I:
        raise ValueError("out must be [rows, I]")
    ws = default_workspace(x.device, stream) if ws is None else ws
    _call("gmm_fwd_silu_mul", _ptr(x), T, _ptr(sorted_token_ids), int(top_k), _ptr(w1), _ptr(group_sizes), E, M,
          K, I, int(bool(trans_b)), _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    return y


def gmm_bwd(dy, x, w, group_sizes, trans_b=False, need_dx=True, need_dw=True, dx=None, dw=None, ws=None,
            stream=None):
    """Returns (dx, dw): dx = dy @ w[g]^T, dw[g] = x_g^T @ dy_g (laid out like w)."""
    _need(dy, torch.bfloat16, "dy", 2)
    _need(x, torch.bfloat16, "x", 2)
    _need(w, torch.bfloat16, "w", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = x.shape
    E = w.shape[0]
    N = dy.shape[1]
    if need_dx and dx is None:
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=x.device)
    if need_dw and dw is None:
        dw = torch.empty_like(w)
    ws = default_workspace(x.device, stream) if ws is None else ws
    _call("gmm_bwd", _ptr(dy), _ptr(x), _ptr(w), _ptr(group_sizes), E, M, K, N, int(bool(trans_b)),
          _ptr(dx if need_dx else None), _ptr(dw if need_dw else None), _ptr(ws), ws.numel(), _stream(stream))
    return (dx if need_dx else None), (dw if need_dw else None)


# --------------------------------------------------------------------------
# fp8 / f8i4 grouped GEMM
# --------------------------------------------------------------------------

def _fp8w(codes, scales, ld, expert_stride):
    """The weight descriptor; ld (the bytes between output columns' code
    runs) defaults to the codes tensor's row stride, and an explicit ld must
    equal it (a colwise-quantized weight is a view of padded rows)."""
    if codes.dim() < 2 or codes.stride(-1) != 1:
        raise ValueError("fp8 weight codes need at least 2 dimensions and a unit last stride")
    row = codes.stride(-2)
    if ld is None:
        ld = row
    elif int(ld) != row:
        raise ValueError(f"w_ld={ld} differs from the codes' row stride {row}")
    return FP8Weight(codes.data_ptr(), scales.data_ptr(), int(ld), int(expert_stride))


def gmm_fwd_fp8(xq, sx, wq, sw, w_ld, w_expert_stride, group_sizes, N, out=None, ws=None, stream=None):
    """y[r,n] = sum_k (xq[r,k]/sx[r]) (Wq(g,k,n)/sw[g,n]); Wq(e,k,n) at e*w_expert_stride + n*w_ld + k.
    w_ld None: the row stride of wq."""
    _need(xq, torch.uint8, "xq", 2)
    _need(sx, torch.float32, "sx", 1)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = xq.shape
    E = group_sizes.numel()
    y = torch.empty(M, N, dtype=torch.bfloat16, device=xq.device) if out is None else out
    ws = default_workspace(xq.device, stream) if ws is None else ws
    wd = _fp8w(wq, sw, w_ld, w_expert_stride)
    _call("gmm_fwd_fp8", _ptr(xq), _ptr(sx), ctypes.byref(wd), _ptr(group_sizes), E, M, K, int(N), _ptr(y),
          _ptr(ws), ws.numel(), _stream(stream))
    return y


def gmm_bwd_fp8(group_sizes, K, N, dyq=None, sdy=None, wq=None, sw=None, w_ld=None, w_expert_stride=0,
                xc=None, sxc=None, dyc=None, sdyc=None, need_dx=True, need_dw=True, dx=None, dw=None,
                ws=None, stream=None):
    """fp8 backward; see gmm_bwd_fp8 in include/moe_gemm.h for operand layouts."""
    _need(group_sizes, torch.int32, "group_sizes", 1)
    E = group_sizes.numel()
    dev = group_sizes.device
    M = dyq.shape[0] if dyq is not None else xc.shape[1]
    ldc = 0
    if need_dw:
        for t, name in ((xc, "xc"), (dyc, "dyc")):
            if t is None or t.dtype != torch.uint8 or t.dim() != 2 or t.device.type != "cuda" or t.stride(1) != 1:
                raise ValueError(f"{name} must be a 2-D uint8 device tensor with unit column stride")
        ldc = xc.stride(0)
        if dyc.stride(0) != ldc or xc.shape[1] != M or dyc.shape[1] != M:
            raise ValueError("xc and dyc must be [K, M] and [N, M] views with one row stride")
    if need_dx and dx is None:
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    if need_dw and dw is None:
        dw = torch.empty(E, K, N, dtype=torch.bfloat16, device=dev)
    ws = default_workspace(dev, stream) if ws is None else ws
    wd = _fp8w(wq, sw, w_ld, w_expert_stride) if need_dx else None
    _call("gmm_bwd_fp8", _ptr(dyq), _ptr(sdy), ctypes.byref(wd) if wd is not None else None, _ptr(xc),
          _ptr(sxc), _ptr(dyc), _ptr(sdyc), ldc, _ptr(group_sizes), E, M, int(K), int(N),
          _ptr(dx if need_dx else None), _ptr(dw if need_dw else None), _ptr(ws), ws.numel(), _stream(stream))
    return (dx if need_dx else None), (dw if need_dw else None)


def gmm_fwd_f8i4(xq, sx, w4, sw, group_sizes, out=None, ws=None, stream=None):
    """y = (xq/sx) @ dequant(w4, sw) per group; w4 [E,N,K/2] uint8, sw bf16 [E,K/128,N]."""
    _need(xq, torch.uint8, "xq", 2)
    _need(sx, torch.float32, "sx", 1)
    _need(w4, torch.uint8, "w4", 3)
    _need(sw, torch.bfloat16, "sw", 3)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, K = xq.shape
    E, N, K2 = w4.shape
    if K2 * 2 != K or group_sizes.numel() != E:
        raise ValueError("shape mismatch between xq, w4 and group_sizes")
    y = torch.empty(M, N, dtype=torch.bfloat16, device=xq.device) if out is None else out
    ws = default_workspace(xq.device, stream) if ws is None else ws
    _call("gmm_fwd_f8i4", _ptr(xq), _ptr(sx), _ptr(w4), _ptr(sw), _ptr(group_sizes), E, M, K, N, _ptr(y),
          _ptr(ws), ws.numel(), _stream(stream))
    return y


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def _rowwise_outputs(q, scales, R, C, device):
    """Fresh (codes, scales) for R rows of C values, or the caller's buffers
    checked for dtype, shape, contiguity and device (the kernels write R * C
    codes and R scales through them)."""
    q = torch.empty(R, C, dtype=torch.uint8, device=device) if q is None else q
    scales = torch.empty(R, dtype=torch.float32, device=device) if scales is None else scales
    _need(q, torch.uint8, "q", 2)
    _need(scales, torch.float32, "scales", 1)
    if tuple(q.shape) != (R, C) or scales.numel() != R:
        raise ValueError(f"q must be [{R}, {C}] and scales [{R}]")
    if q.device != device or scales.device != device:
        raise ValueError("q and scales must be on the input's device")
    return q, scales


def quantize_rowwise_fp8(x, q=None, scales=None, stream=None):
    """bf16 [R, C] -> (e4m3 codes uint8 [R, C], fp32 scales [R])."""
    if x.device.type != "cuda" or x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a device bf16 matrix with unit column stride")
    R, C = x.shape
    q, scales = _rowwise_outputs(q, scales, R, C, x.device)
    _call("quantize_rowwise_fp8", _ptr(x), R, C, x.stride(0), _ptr(q), _ptr(scales), _stream(stream))
    return q, scales


def quantize_rowwise_fp8_gather(x, sorted_token_ids, top_k, q=None, scales=None, stream=None):
    """Rowwise e4m3 of the token rows in sorted order: row r quantizes
    x[sorted_token_ids[r] // top_k]; the padding sentinel (>= T * top_k)
    gives a row of zeros.  x bf16 [T, C] contiguous.  Returns (codes uint8
    [rows, C], fp32 scales [rows]), rows = sorted_token_ids.numel()."""
    _need(x, torch.bfloat16, "x", 2)
    _need(sorted_token_ids, torch.int32, "sorted_token_ids", 1)
    T, C = x.shape
    R = sorted_token_ids.numel()
    q, scales = _rowwise_outputs(q, scales, R, C, x.device)
    _call("quantize_rowwise_fp8_gather", _ptr(x), T, _ptr(sorted_token_ids), int(top_k), R, C, _ptr(q),
          _ptr(scales), _stream(stream))
    return q, scales


def colwise_workspace_bytes(G, rows, cols_a, cols_b=0):
    return int(lib().quantize_colwise_workspace_bytes(int(G), int(rows), int(cols_a), int(cols_b)))


_CW_CACHE = {}


def default_colwise_workspace(nbytes, device=None, stream=None):
    """The colwise quantizer's workspace for a call made without ``ws``: one
    per (device, stream), zero-filled when created (its first word is the
    sticky error word) and replaced by a larger one when a call needs more.
    It carries partial maxima from the quantizer's first launch to its
    second and nothing between calls; calls on one stream never overlap, so
    they may share it.  It cannot be created or grown during graph capture:
    make one eager call of the largest shape first, or pass ``ws``."""
    dev = torch.device("cuda") if device is None else torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    s = torch.cuda.current_stream(idx) if stream is None else stream
    key = (idx, s.cuda_stream)
    ws = _CW_CACHE.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("no colwise workspace of this size for this stream yet and the stream is capturing: "
                               "make one eager call of this shape on it first, or pass ws")
        with torch.cuda.device(idx), torch.cuda.stream(s):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=torch.device("cuda", idx))
        _CW_CACHE[key] = ws
    return ws


def colwise_ld(M):
    """Row stride (bytes) the colwise quantizer's fresh outputs get for M
    rows: M rounded up to an odd multiple of 256.  The fp8 dW reads 256 such
    rows per tile at once; with a stride that is a multiple of a large power
    of two (98304 rows = 3 * 2^15, say) they share a few HBM channels."""
    ld = (int(M) + 255) // 256 * 256
    return ld + 256 if (ld // 256) % 2 == 0 else ld


def quantize_colwise_per_group_fp8(a, group_sizes, b=None, stream=None, out=None, ws=None):
    """Per-group colwise quantization of a (and b).  Returns
    (qa [Ca, M] column-major codes, sa [G, Ca]) or, with b,
    (qa, sa, qb, sb).  Fresh code tensors are [C, M] views of [C,
    colwise_ld(M)] buffers.  Codes of rows past the groups, and the bytes
    past M of a code row, are not written (a fresh output holds whatever
    its allocation held there); out=(qa, sa[, qb, sb]) reuses buffers,
    checked for dtype, shape and device (code tensors: unit column stride,
    row stride at least M, the same for qa and qb).  ws: a
    uint8 device tensor of at least colwise_workspace_bytes(G, M, Ca, Cb)
    bytes whose first word (the sticky error word) starts at zero (default:
    the cached one of the device and stream)."""
    _need(a, torch.bfloat16, "a", 2)
    _need(group_sizes, torch.int32, "group_sizes", 1)
    M, Ca = a.shape
    G = group_sizes.numel()
    def check(q, sc, C, name):
        if q.device.type != "cuda" or q.dtype != torch.uint8 or q.dim() != 2:
            raise ValueError(f"q{name} must be a 2-D uint8 device tensor")
        if q.stride(1) != 1 or q.stride(0) < M:
            raise ValueError(f"q{name} needs a unit column stride and a row stride of at least {M}")
        _need(sc, torch.float32, "s" + name, 2)
        if tuple(q.shape) != (C, M) or tuple(sc.shape) != (G, C) or q.device != a.device or sc.device != a.device:
            raise ValueError(f"q{name} must be [{C}, {M}] and s{name} [{G}, {C}] on the input's device")

    ld = colwise_ld(M)
    if out is not None:
        qa, sa = out[0], out[1]
        check(qa, sa, Ca, "a")
        ld = qa.stride(0)
    else:
        qa = torch.empty(Ca, ld, dtype=torch.uint8, device=a.device)[:, :M]
        sa = torch.empty(G, Ca, dtype=torch.float32, device=a.device)
    qb = sb = None
    Cb = 0
    if b is not None:
        _need(b, torch.bfloat16, "b", 2)
        if b.shape[0] != M:
            raise ValueError("a and b must have the same number of rows")
        Cb = b.shape[1]
        if out is not None:
            qb, sb = out[2], out[3]
            check(qb, sb, Cb, "b")
            if qb.stride(0) != ld:
                raise ValueError("qa and qb must have the same row stride")
        else:
            qb = torch.empty(Cb, ld, dtype=torch.uint8, device=a.device)[:, :M]
            sb = torch.empty(G, Cb, dtype=torch.float32, device=a.device)
    need = colwise_workspace_bytes(G, M, Ca, Cb)
    if ws is None:
        ws = default_colwise_workspace(need, a.device, stream)
    else:
        _need(ws, torch.uint8, "ws", 1)
        if ws.device != a.device:
            raise ValueError("ws must be on the input's device")
    _call("quantize_colwise_per_group_fp8", _ptr(a), Ca, _ptr(b), Cb, _ptr(group_sizes), G, M, ld, _ptr(qa),
          _ptr(sa), _ptr(qb), _ptr(sb), _ptr(ws), ws.numel(), _stream(stream))
    return (qa, sa) if b is None else (qa, sa, qb, sb)


def quantize_int4_weights(w, stream=None):
    """bf16 [E, K, N] -> (int4 packed uint8 [E, N, K/2], bf16 scales [E, K/128, N])."""
    _need(w, torch.bfloat16, "w", 3)
    E, K, N = w.shape
    w4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=w.device)
    sw = torch.empty(E, K // 128, N, dtype=torch.bfloat16, device=w.device)
    _call("quantize_int4_weights", _ptr(w), E, K, N, _ptr(w4), _ptr(sw), _stream(stream))
    return w4, sw


# --------------------------------------------------------------------------
# token permutation for the fused path
# --------------------------------------------------------------------------

def sorted_capacity(T, k, E, block_m):
    return int(lib().moe_sorted_capacity(int(T), int(k), int(E), int(block_m)))


def block_capacity(T, k, E, block_m):
    return int(lib().moe_block_capacity(int(T), int(k), int(E), int(block_m)))


def moe_permute(topk_ids, E, block_m, x=None, ws=None, stream=None):
    """moe_align_block_size (+ gather of x rows).  Returns a dict with
    sorted_token_ids, expert_ids, num_tokens_post_padded, inv, padded_sizes
    and x_sorted (or None)."""
    _need(topk_ids, torch.int32, "topk_ids", 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    cap = sorted_capacity(T, k, E, block_m)
    nblk = block_capacity(T, k, E, block_m)
    sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    expert_ids = torch.empty(max(nblk, 1), dtype=torch.int32, device=dev)
    ntpp = torch.empty(1, dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    padded = torch.empty(E, dtype=torch.int32, device=dev)
    hidden = 0
    xs = None
    if x is not None:
        _need(x, torch.bfloat16, "x", 2)
        hidden = x.shape[1]
        xs = torch.empty(max(cap, 1), hidden, dtype=torch.bfloat16, device=dev)
    need = int(lib().moe_permute_workspace_bytes(T, k, E))
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _call("moe_permute", _ptr(topk_ids), T, k, int(E), int(block_m), _ptr(x), hidden, _ptr(sorted_ids),
          _ptr(expert_ids), _ptr(ntpp), _ptr(inv), _ptr(padded), _ptr(xs), _ptr(ws), ws.numel(),
          _stream(stream))
    return dict(sorted_token_ids=sorted_ids[:cap], expert_ids=expert_ids[:nblk], num_tokens_post_padded=ntpp,
                inv=inv[:T * k], padded_sizes=padded, x_sorted=None if xs is None else xs[:cap])


def fused_moe_f8i4(x, w1_4, s1, w2_4, s2, topk_ids, topk_weights, block_m=16, ws=None, stream=None,
                   keep_act=False):
    """Token-sorted MoE expert FFN with int4 expert weights and fp8
    activations, for decode-sized token counts: align -> rowwise e4m3
    quantization of the token rows in sorted order -> F8I4 GEMM1 -> SiLU*mul
    and rowwise e4m3 quantization in one pass -> F8I4 GEMM2 -> top-k
    weighted combine.  Weights as quantize_int4_weights returns them: w1_4
    uint8 [E, 2I, H/2] with s1 bf16 [E, H/128, 2I] (from W1 [E, H, 2I]),
    w2_4 uint8 [E, H, I/2] with s2 bf16 [E, I/128, H] (from W2 [E, I, H]).
    Every weight tile is streamed once per 32 sorted rows, so this path
    suits small T; large T belongs on the bf16 or fp8 kernels.  Returns
    (out bf16 [T, H], dict of the intermediates); the bf16 activations are
    written and returned only with keep_act."""
    T, k = topk_ids.shape
    E = w1_4.shape[0]
    inter = w1_4.shape[1] // 2
    p = moe_permute(topk_ids, E, block_m, stream=stream)
    ids, sizes = p["sorted_token_ids"], p["padded_sizes"]
    ws = default_workspace(x.device, stream) if ws is None else ws
    # the token rows are read through the sorted order by the quantizer
    xq, sx = quantize_rowwise_fp8_gather(x, ids, k, stream=stream)
    h1 = gmm_fwd_f8i4(xq, sx, w1_4, s1, sizes, ws=ws, stream=stream)
    act = torch.empty(h1.shape[0], inter, dtype=torch.bfloat16, device=x.device) if keep_act else None
    aq, sa = silu_mul_quantize_rowwise_fp8(h1, act=act, stream=stream)
    y2 = gmm_fwd_f8i4(aq, sa, w2_4, s2, sizes, ws=ws, stream=stream)
    out = moe_unpermute(y2, p["inv"], topk_weights, T, k, stream=stream)
    return out, dict(permute=p, xq=xq, sx=sx, h1=h1, act=act, aq=aq, sa=sa, y2=y2)


def quantize_fp8_expert_weights(w, stream=None):
    """Expert weights w bf16 [E, K, N] -> (wq uint8 [N, E*K], sw fp32 [E, N]):
    column-major e4m3 codes with one power-of-two scale per (expert, output
    column) over its K weights.  This is the per-group colwise quantizer on w
    viewed as [E*K, N] with E groups of K rows, into contiguous codes (the
    forward reads weight rows E*K bytes apart faster than the padded rows
    the quantizer gives activations); gmm_fwd_fp8 takes them with w_ld =
    E*K (or None) and w_expert_stride = K."""
    _need(w, torch.bfloat16, "w", 3)
    E, K, N = w.shape
    sizes = torch.full((E,), K, dtype=torch.int32, device=w.device)
    out = (torch.empty(N, E * K, dtype=torch.uint8, device=w.device),
           torch.empty(E, N, dtype=torch.float32, device=w.device))
    return quantize_colwise_per_group_fp8(w.reshape(E * K, N), sizes, stream=stream, out=out)


def fused_moe_fp8(x, w1q, s1, w2q, s2, topk_ids, topk_weights, block_m=None, ws=None, stream=None,
                  keep_act=False):
    """Token-sorted MoE expert FFN with e4m3 expert weights and
    activations: align -> rowwise e4m3 of the token rows in sorted order ->
    fp8 GEMM1 (row scales x per-(expert, column) weight scales) -> SiLU*mul
    and rowwise e4m3 of the activations in one pass -> fp8 GEMM2 -> top-k
    weighted combine.  Weights as quantize_fp8_expert_weights returns them:
    w1q uint8 [2I, E*H] with s1 fp32 [E, 2I] (from W1 [E, H, 2I]), w2q
    uint8 [H, E*I] with s2 fp32 [E, H] (from W2 [E, I, H]).  Returns (out
    bf16 [T, H], dict of the intermediates); the bf16 activations are
    written and returned only with keep_act."""
    T, k = topk_ids.shape
    E, two_i = s1.shape
    H = x.shape[1]
    inter = two_i // 2
    if s2.shape != (E, H) or w1q.shape != (two_i, E * H) or w2q.shape != (H, E * inter):
        raise ValueError("fp8 expert weights do not match x and each other")
    if block_m is None:
        block_m = 16 if T * k <= 64 * E else 128
    p = moe_permute(topk_ids, E, block_m, stream=stream)
    ids, sizes = p["sorted_token_ids"], p["padded_sizes"]
    ws = default_workspace(x.device, stream) if ws is None else ws
    # the token rows are read through the sorted order by the quantizer
    xq, sx = quantize_rowwise_fp8_gather(x, ids, k, stream=stream)
    h1 = gmm_fwd_fp8(xq, sx, w1q, s1, None, H, sizes, two_i, ws=ws, stream=stream)
    act = torch.empty(h1.shape[0], inter, dtype=torch.bfloat16, device=x.device) if keep_act else None
    aq, sa = silu_mul_quantize_rowwise_fp8(h1, act=act, stream=stream)
    y2 = gmm_fwd_fp8(aq, sa, w2q, s2, None, inter, sizes, H, ws=ws, stream=stream)
    out = moe_unpermute(y2, p["inv"], topk_weights, T, k, stream=stream)
    return out, dict(permute=p, xq=xq, sx=sx, h1=h1, act=act, aq=aq, sa=sa, y2=y2)


def route_topk(logits, top_k, renormalize=False, stream=None):
    """Router: fp32 softmax of each token's logits, its top_k experts in
    descending order (ties to the lower index) and their probabilities
    (divided by their sum with renormalize).  Returns (topk_ids int32 [T, k],
    topk_weights fp32 [T, k])."""
    _need(logits, torch.float32, "logits", 2)
    T, E = logits.shape
    ids = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, top_k, dtype=torch.float32, device=logits.device)
    _call("moe_route_topk", _ptr(logits), T, E, int(top_k), int(bool(renormalize)), _ptr(ids), _ptr(w),
          _stream(stream))
    return ids, w


def moe_unpermute(y_sorted, inv, topk_weights, T, k, out=None, stream=None):
    """out[t] = sum_j w[t,j] * y_sorted[inv[t*k+j]] (fp32 sum, bf16 out)."""
    _need(y_sorted, torch.bfloat16, "y_sorted", 2)
    _need(inv, torch.int32, "inv")
    if topk_weights is not None:
        _need(topk_weights, torch.float32, "topk_weights")
    H = y_sorted.shape[1]
    out = torch.empty(T, H, dtype=torch.bfloat16, device=y_sorted.device) if out is None else out
    _call("moe_unpermute", _ptr(y_sorted), _ptr(inv), _ptr(topk_weights), int(T), int(k), H, _ptr(out),
          _stream(stream))
    return out


def silu_mul(h, out=None, stream=None):
    """act = silu(h[:, :I]) * h[:, I:] in bf16."""
    _need(h, torch.bfloat16, "h", 2)
    R, I2 = h.shape
    out = torch.empty(R, I2 // 2, dtype=torch.bfloat16, device=h.device) if out is None else out
    _call("silu_mul", _ptr(h), R, I2 // 2, _ptr(out), _stream(stream))
    return out


def silu_mul_quantize_rowwise_fp8(h, q=None, scales=None, act=None, stream=None):
    """silu(h[:, :I]) * h[:, I:] in bf16, then rowwise e4m3 of it, in one
    pass: returns (codes uint8 [R, I], fp32 scales [R]), the same bits as
    quantize_rowwise_fp8(silu_mul(h)).  act, a bf16 [R, I] buffer, also
    receives the bf16 activations when given."""
    _need(h, torch.bfloat16, "h", 2)
    R, I2 = h.shape
    q, scales = _rowwise_outputs(q, scales, R, I2 // 2, h.device)
    if act is not None:
        _need(act, torch.bfloat16, "act", 2)
        if tuple(act.shape) != (R, I2 // 2) or act.device != h.device:
            raise ValueError(f"act must be [{R}, {I2 // 2}] on h's device")
    _call("silu_mul_quantize_rowwise_fp8", _ptr(h), R, I2 // 2, _ptr(act), _ptr(q), _ptr(scales), _stream(stream))
    return q, scales


def fused_moe(x, w1, w2, topk_ids, topk_weights, block_m=None, ws=None, stream=None, trans_b=False):
    """Token-sorted MoE expert FFN: align -> gmm(W1) over the token rows
    looked up through the sorted order, with SiLU*mul in its epilogue ->
    gmm(W2) -> top-k weighted combine.  w1 [E, H, 2I], w2 [E, I, H] bf16,
    or with trans_b w1 [E, 2I, H], w2 [E, H, I] (the (E, N, K) layout)."""
    T, k = topk_ids.shape
    E = w1.shape[0]
    if block_m is None:
        block_m = 16 if T * k <= 64 * E else 128
    p = moe_permute(topk_ids, E, block_m, stream=stream)
    ids = p["sorted_token_ids"]
    sizes = p["padded_sizes"]
    ws = default_workspace(x.device, stream) if ws is None else ws
    # GEMM1 reads the token rows through the sorted order (no sorted copy)
    # and applies SiLU-and-mul in its epilogue (no [rows, 2I] intermediate)
    act = gmm_fwd_silu_mul(x, w1, sizes, sorted_token_ids=ids, top_k=k, trans_b=trans_b, ws=ws, stream=stream)
    y2 = gmm_fwd(act, w2, sizes, trans_b=trans_b, ws=ws, stream=stream)
    return moe_unpermute(y2, p["inv"], topk_weights, T, k, stream=stream), p
