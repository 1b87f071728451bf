"""Host-side checks of the C-ABI library: it loads, exports every function the
header declares, and rejects bad arguments before touching the GPU.  CPU only:
every call below fails validation, so no HIP API is reached."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_grouped_gemm_device_amd as mg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_gemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mg.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return mg.lib()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ["gmm_fwd", "gmm_bwd", "quantize_rowwise_fp8", "quantize_colwise_per_group_fp8",
                     "quantize_colwise_workspace_bytes",
                     "moe_permute", "moe_unpermute", "gmm_fwd_fp8", "gmm_bwd_fp8", "gmm_fwd_f8i4",
                     "gmm_build_worklist", "silu_mul", "quantize_int4_weights"]:
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", mg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    # and the binding wraps each of them
    assert set(_declared_functions()) <= set(mg.EXPORTS)


def test_version(lib):
    assert lib.mg_version().decode().startswith("moe-gemm-gfx950")


def _p(v):
    return ctypes.c_void_p(v)


FAKE = 0x1000  # never dereferenced: every call below fails host validation first


def test_workspace_size_is_host_only(lib):
    a = lib.mg_workspace_bytes(8, 1024)
    b = lib.mg_workspace_bytes(8, 1 << 30)
    c = lib.mg_workspace_bytes(1024, 1)
    assert 0 < a <= b and c > 0 and a % 256 == 0
    assert lib.mg_workspace_bytes(0, 10) == 0 and lib.mg_workspace_bytes(1025, 10) == 0


@pytest.mark.parametrize("E,total_M,K,N,code", [
    (0, 16, 64, 64, mg.MG_EINVAL),           # no experts
    (1025, 16, 64, 64, mg.MG_EINVAL),        # above the single-workgroup scan limit
    (4, -1, 64, 64, mg.MG_EINVAL),           # negative rows
    (4, 16, 0, 64, mg.MG_EINVAL),            # empty K
    (4, 16, 60, 64, mg.MG_EUNSUPPORTED),     # K not a multiple of 8
    (4, 16, 64, 36, mg.MG_EUNSUPPORTED),     # N not a multiple of 8
])
def test_gmm_fwd_rejects_bad_shapes(lib, E, total_M, K, N, code):
    ws_bytes = max(lib.mg_workspace_bytes(max(1, min(E, 1024)), max(total_M, 0)), 256)
    rc = lib.gmm_fwd(_p(FAKE), _p(FAKE), _p(FAKE), E, total_M, K, N, 0, _p(FAKE), _p(0x10000), ws_bytes, None)
    assert rc == code, lib.mg_last_error()
    assert lib.mg_last_error()


def test_gmm_fwd_rejects_null_and_small_workspace(lib):
    need = lib.mg_workspace_bytes(4, 64)
    assert lib.gmm_fwd(None, _p(FAKE), _p(FAKE), 4, 64, 64, 64, 0, _p(FAKE), _p(0x10000), need, None) == mg.MG_EINVAL
    assert lib.gmm_fwd(_p(FAKE), _p(FAKE), None, 4, 64, 64, 64, 0, _p(FAKE), _p(0x10000), need, None) == mg.MG_EINVAL
    assert lib.gmm_fwd(_p(FAKE), _p(FAKE), _p(FAKE), 4, 64, 64, 64, 0, _p(FAKE), _p(0x10000), need - 1,
                       None) == mg.MG_EWORKSPACE
    assert lib.gmm_fwd(_p(FAKE), _p(FAKE), _p(FAKE), 4, 64, 64, 64, 0, _p(FAKE), None, need, None) == mg.MG_EWORKSPACE
    assert lib.gmm_fwd(_p(FAKE), _p(FAKE), _p(FAKE), 4, 64, 64, 64, 0, _p(FAKE), _p(0x10008), need,
                       None) == mg.MG_EINVAL  # misaligned workspace


@pytest.mark.parametrize("E,total_M", [(0, 16), (1025, 16), (4, -1), (4, 1 << 31)])
def test_gmm_fwd_noalloc_rejects_before_any_device_call(lib, E, total_M):
    """The allocation-free forward refuses out-of-range sizes on the host,
    before it looks up its scratch array on the device."""
    rc = lib.gmm_fwd_noalloc(_p(FAKE), _p(FAKE), _p(FAKE), E, total_M, 64, 64, 0, _p(FAKE), None)
    assert rc == mg.MG_EINVAL and lib.mg_last_error()


def test_gmm_bwd_rejects_no_outputs(lib):
    need = lib.mg_workspace_bytes(4, 64)
    rc = lib.gmm_bwd(_p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 4, 64, 64, 64, 0, None, None, _p(0x10000), need, None)
    assert rc == mg.MG_EINVAL


def test_fp8_and_f8i4_reject_unsupported_alignment(lib):
    need = lib.mg_workspace_bytes(4, 64)
    w = mg.FP8Weight(FAKE, FAKE, 64, 64 * 64)
    assert lib.gmm_fwd_fp8(_p(FAKE), _p(FAKE), ctypes.byref(w), _p(FAKE), 4, 64, 40, 64, _p(FAKE), _p(0x10000),
                           need, None) == mg.MG_EUNSUPPORTED          # K % 16
    wbad = mg.FP8Weight(FAKE, FAKE, 72, 64 * 64)
    assert lib.gmm_fwd_fp8(_p(FAKE), _p(FAKE), ctypes.byref(wbad), _p(FAKE), 4, 64, 64, 64, _p(FAKE),
                           _p(0x10000), need, None) == mg.MG_EUNSUPPORTED   # ld % 16
    assert lib.gmm_fwd_f8i4(_p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 4, 64, 192, 64, _p(FAKE),
                            _p(0x10000), need, None) == mg.MG_EUNSUPPORTED  # K % 128
    assert lib.gmm_fwd_f8i4(_p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 4, 64, 65536, 65536, _p(FAKE),
                            _p(0x10000), need, None) == mg.MG_EUNSUPPORTED  # one expert's weights past 2 GiB
    assert lib.gmm_bwd_fp8(None, None, None, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), 48, _p(FAKE), 4, 40, 64, 64,
                           None, _p(FAKE), _p(0x10000), lib.mg_workspace_bytes(4, 40),
                           None) == mg.MG_EUNSUPPORTED                   # dw needs total_M % 16


def test_fp8_dw_rejects_bad_row_stride(lib):
    need = lib.mg_workspace_bytes(4, 64)
    dw = lambda ldc: lib.gmm_bwd_fp8(None, None, None, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE), ldc, _p(FAKE), 4, 64,
                                     64, 64, None, _p(FAKE), _p(0x10000), need, None)
    assert dw(48) == mg.MG_EINVAL         # below total_M
    assert dw(72) == mg.MG_EINVAL         # not a multiple of 16
    assert dw(1 << 30) == mg.MG_EUNSUPPORTED   # K rows of that stride past 2 GiB


def test_colwise_workspace_size(lib):
    # a 256-byte header and 64 partial maxima per (chunk slot, column block),
    # with rows / 256 + 2 G chunk slots
    f = lib.quantize_colwise_workspace_bytes
    ncb = 22 + 32
    assert f(64, 98304, 1408, 2048) == 256 + 4 * (384 + 128) * ncb * 64
    assert f(64, 98304, 1408, 0) < f(64, 98304, 1408, 2048)
    assert f(64, 98304, 1408, 2048) < f(64, 98305, 1408, 2048) < f(65, 98305, 1408, 2048)
    assert f(1, 0, 8, 0) == 256 + 4 * 2 * 64


def test_quantizers_reject_bad_arguments(lib):
    assert lib.quantize_rowwise_fp8(_p(FAKE), 4, 12, 12, _p(FAKE), _p(FAKE), None) == mg.MG_EUNSUPPORTED
    assert lib.quantize_rowwise_fp8(_p(FAKE), 4, 16, 8, _p(FAKE), _p(FAKE), None) == mg.MG_EINVAL
    cw = lib.quantize_colwise_per_group_fp8
    need = lib.quantize_colwise_workspace_bytes(4, 64, 16, 16)
    assert cw(_p(FAKE), 16, _p(FAKE), 16, _p(FAKE), 4, 64, 64, _p(FAKE), _p(FAKE), None, _p(FAKE),
              _p(0x10000), need, None) == mg.MG_EINVAL        # b without qb
    assert cw(_p(FAKE), 16, None, 0, _p(FAKE), 0, 64, 64, _p(FAKE), _p(FAKE), None, None,
              _p(0x10000), need, None) == mg.MG_EINVAL        # G = 0
    assert cw(_p(FAKE), (1 << 20) + 8, None, 0, _p(FAKE), 4, 64, 64, _p(FAKE), _p(FAKE), None, None,
              _p(0x10000), 1 << 40, None) == mg.MG_EUNSUPPORTED   # cols above 2^20
    assert cw(_p(FAKE), 16, None, 0, _p(FAKE), 4, 64, 64, _p(FAKE), _p(FAKE), None, None,
              None, need, None) == mg.MG_EWORKSPACE           # no workspace
    assert cw(_p(FAKE), 16, None, 0, _p(FAKE), 4, 64, 64, _p(FAKE), _p(FAKE), None, None,
              _p(0x10080), need, None) == mg.MG_EWORKSPACE    # not 256-byte aligned
    assert cw(_p(FAKE), 16, None, 0, _p(FAKE), 4, 64, 63, _p(FAKE), _p(FAKE), None, None,
              _p(0x10000), need, None) == mg.MG_EINVAL        # code rows closer than the row count
    single = lib.quantize_colwise_workspace_bytes(4, 64, 16, 0)
    assert cw(_p(FAKE), 16, None, 0, _p(FAKE), 4, 64, 64, _p(FAKE), _p(FAKE), None, None,
              _p(0x10000), single - 4, None) == mg.MG_EWORKSPACE   # too small
    assert lib.quantize_int4_weights(_p(FAKE), 2, 100, 16, _p(FAKE), _p(FAKE), None) == mg.MG_EUNSUPPORTED
    g = lib.quantize_rowwise_fp8_gather
    assert g(_p(FAKE), 4, _p(FAKE), 2, 8, 12, _p(FAKE), _p(FAKE), None) == mg.MG_EUNSUPPORTED   # cols % 8
    assert g(_p(FAKE), 4, _p(FAKE), 0, 8, 16, _p(FAKE), _p(FAKE), None) == mg.MG_EINVAL        # top_k 0
    assert g(_p(FAKE), -1, _p(FAKE), 2, 8, 16, _p(FAKE), _p(FAKE), None) == mg.MG_EINVAL       # T < 0
    assert g(_p(FAKE), 4, None, 2, 8, 16, _p(FAKE), _p(FAKE), None) == mg.MG_EINVAL            # no ids
    assert g(None, 4, _p(FAKE), 2, 8, 16, _p(FAKE), _p(FAKE), None) == mg.MG_EINVAL            # no x, T > 0
    assert g(_p(FAKE), 4, _p(FAKE), 2, 0, 16, None, None, None) == mg.MG_OK                    # no rows


def test_permute_rejects_bad_arguments(lib):
    need = lib.moe_permute_workspace_bytes(4, 2, 8)
    args = lambda E, bm, ws_bytes: (_p(FAKE), 4, 2, E, bm, None, 0, _p(FAKE), _p(FAKE), _p(FAKE), _p(FAKE),
                                    _p(FAKE), None, _p(FAKE), ws_bytes, None)
    assert lib.moe_permute(*args(0, 16, need)) == mg.MG_EINVAL
    assert lib.moe_permute(*args(8, 0, need)) == mg.MG_EINVAL
    assert lib.moe_permute(*args(8, 16, need - 1)) == mg.MG_EWORKSPACE
    assert lib.moe_sorted_capacity(4096, 2, 8, 128) == 4096 * 2 + 8 * 127
    assert lib.moe_block_capacity(4, 3, 4, 4) == 6
    assert lib.moe_unpermute(_p(FAKE), _p(FAKE), None, 4, 2, 12, _p(FAKE), None) == mg.MG_EUNSUPPORTED
    assert lib.silu_mul(_p(FAKE), 4, 12, _p(FAKE), None) == mg.MG_EUNSUPPORTED


def test_gathered_and_silu_gemms_reject_bad_arguments(lib):
    need = lib.mg_workspace_bytes(4, 64)
    ws = _p(0x10000)
    # gmm_fwd_gather(x, T, ids, top_k, w, sizes, E, total_M, K, N, trans_b, y, ws, ws_bytes, stream)
    g = lambda T, k, ids, K, N, wsb: lib.gmm_fwd_gather(_p(FAKE), T, ids, k, _p(FAKE), _p(FAKE), 4, 64, K, N, 0,
                                                       _p(FAKE), ws, wsb, None)
    assert g(32, 0, _p(FAKE), 64, 64, need) == mg.MG_EINVAL               # top_k < 1
    assert g(-1, 2, _p(FAKE), 64, 64, need) == mg.MG_EINVAL               # T < 0
    assert g(1 << 23, 4, _p(FAKE), 64, 64, need) == mg.MG_EINVAL          # T*top_k past 2^24
    assert g(32, 2, None, 64, 64, need) == mg.MG_EINVAL                   # no sorted ids
    assert g(32, 2, _p(FAKE), 60, 64, need) == mg.MG_EUNSUPPORTED         # K % 8
    assert g(32, 2, _p(FAKE), 64, 64, need - 1) == mg.MG_EWORKSPACE
    assert g(1 << 20, 2, _p(FAKE), 4096, 64, need) == mg.MG_EUNSUPPORTED  # x past 2 GiB
    # gmm_fwd_silu_mul(x, T, ids, top_k, w1, sizes, E, total_M, K, I, trans_b, act, ws, ws_bytes, stream)
    s = lambda ids, k, K, I, wsb: lib.gmm_fwd_silu_mul(_p(FAKE), 32, ids, k, _p(FAKE), _p(FAKE), 4, 64, K, I, 0,
                                                      _p(FAKE), ws, wsb, None)
    assert s(None, 1, 64, 36, need) == mg.MG_EUNSUPPORTED                 # I % 8
    assert s(None, 1, 0, 64, need) == mg.MG_EINVAL                        # K = 0
    assert s(_p(FAKE), 0, 64, 64, need) == mg.MG_EINVAL                   # gathered, top_k < 1
    assert s(None, 1, 64, 64, need - 1) == mg.MG_EWORKSPACE
    assert lib.gmm_fwd_silu_mul(None, 32, None, 1, _p(FAKE), _p(FAKE), 4, 64, 64, 64, 1, _p(FAKE), ws, need,
                                None) == mg.MG_EINVAL                   # no x


def test_router_rejects_bad_arguments(lib):
    r = lambda T, E, k, ids: lib.moe_route_topk(_p(FAKE), T, E, k, 0, ids, _p(FAKE), None)
    assert r(-1, 8, 2, _p(FAKE)) == mg.MG_EINVAL
    assert r(16, 0, 1, _p(FAKE)) == mg.MG_EINVAL
    assert r(16, 1025, 2, _p(FAKE)) == mg.MG_EINVAL
    assert r(16, 8, 9, _p(FAKE)) == mg.MG_EINVAL          # top_k > E
    assert r(16, 128, 65, _p(FAKE)) == mg.MG_EINVAL       # top_k > 64
    assert r(16, 8, 2, None) == mg.MG_EINVAL
    assert r(0, 8, 2, None) == mg.MG_OK                   # nothing to route
