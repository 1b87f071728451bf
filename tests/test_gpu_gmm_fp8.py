"""GPU parity: fp8 grouped GEMM (forward, dX, dynamic-K dW with per-group
colwise scales) and the F8I4 sparse-M grouped GEMM.  The oracle and the GPU
get the identical quantized operands, produced by the oracle's quantizers."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import (FP8_TOL, GEMM_FP8, assert_close, bf16_dev, bf16_host, dev, dw_norms, dx_norms, fwd_norms, gpu,
                      group_rows, require_gpu, vec_norms)

pytestmark = gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _f64(t):
    return oracle.bf16_to_f64(bf16_host(t))


def _fp8_problem(E, M, K, N, seed, zero_frac=0.25):
    sizes = wl.random_group_sizes(E, M, seed, zero_frac=zero_frac)
    X = wl.normal_bf16((M, K), 1.0, seed, wl.T_X)
    dY = wl.normal_bf16((M, N), 1.0, seed, wl.T_DY)
    W = wl.stacked_normal_bf16(E, (K, N), 0.02, seed, wl.T_W)
    return sizes, X, dY, W


@pytest.mark.parametrize("E,M,K,N,seed", [(4, 300, 256, 200, 0), (9, 1000, 384, 136, 1), (1, 130, 128, 128, 2),
                                          (16, 2048, 2048, 1408, 3)])
def test_fp8_forward(E, M, K, N, seed):
    sizes, X, _, W = _fp8_problem(E, M, K, N, seed)
    xq, sx = oracle.quant_rowwise(X)
    # weights: per-(e, n) scales over K, column-major codes [N][E*K]
    wq, sw = oracle.quant_colwise(W.reshape(E * K, N), np.full(E, K, np.int32))
    y = mg.gmm_fwd_fp8(dev(xq), dev(sx), dev(wq), dev(sw), E * K, K, dev(sizes), N)
    torch.cuda.synchronize()
    A = oracle.dequant_rowwise(xq, sx)
    Wd = oracle.dequant_colwise(wq, sw, np.full(E, K, np.int32)).reshape(E, K, N)
    assert_close(_f64(y), oracle.gmm_fwd(A, Wd, sizes), FP8_TOL, GEMM_FP8, "Y", fwd_norms(A, Wd, sizes))


@pytest.mark.parametrize("E,M,K,N,seed", [(4, 304, 256, 208, 0), (9, 1008, 136, 384, 1), (16, 2048, 1408, 2048, 3)])
def test_fp8_backward(E, M, K, N, seed):
    sizes, X, dY, W = _fp8_problem(E, M, K, N, seed)
    dyq, sdy = oracle.quant_rowwise(dY)
    wq, sw = oracle.quant_rowwise(W.reshape(E * K, N))          # per (e, k) over N
    dyc, sdyc = oracle.quant_colwise(dY, sizes)
    xc, sxc = oracle.quant_colwise(X, sizes)
    dx, dw = mg.gmm_bwd_fp8(dev(sizes), K, N, dyq=dev(dyq), sdy=dev(sdy), wq=dev(wq), sw=dev(sw), w_ld=N,
                            w_expert_stride=K * N, xc=dev(xc), sxc=dev(sxc), dyc=dev(dyc), sdyc=dev(sdyc))
    torch.cuda.synchronize()
    Wd = oracle.dequant_rowwise(wq, sw).reshape(E, K, N)
    dYd = oracle.dequant_rowwise(dyq, sdy)
    assert_close(_f64(dx), oracle.gmm_dx(dYd, Wd, sizes), FP8_TOL, GEMM_FP8, "dX", dx_norms(dYd, Wd, sizes))
    Xc, dYc = oracle.dequant_colwise(xc, sxc, sizes), oracle.dequant_colwise(dyc, sdyc, sizes)
    dwh = _f64(dw)
    assert_close(dwh, oracle.gmm_dw(Xc, dYc, sizes), FP8_TOL, GEMM_FP8, "dW", dw_norms(Xc, dYc, sizes))
    for g in np.flatnonzero(sizes == 0):
        assert (dwh[g] == 0).all()
    # xc and dyc in rows of a padded stride whose pad bytes are NaN codes:
    # same bits (the dW reads nothing past total_M in a row)
    ld = M + 48
    xp = torch.full((K, ld), 0x7F, dtype=torch.uint8, device="cuda")
    dp = torch.full((N, ld), 0x7F, dtype=torch.uint8, device="cuda")
    xp[:, :M].copy_(dev(xc))
    dp[:, :M].copy_(dev(dyc))
    _, dw2 = mg.gmm_bwd_fp8(dev(sizes), K, N, xc=xp[:, :M], sxc=dev(sxc), dyc=dp[:, :M], sdyc=dev(sdyc),
                            need_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dw2, dw)


def test_fp8_dw_without_rows_is_zero():
    """No rows: every group is empty and dW is zero, whatever the empty
    operands' strides."""
    E, K, N = 3, 64, 48
    gs = torch.zeros(E, dtype=torch.int32, device="cuda")
    xc = torch.empty(K, 0, dtype=torch.uint8, device="cuda")
    dyc = torch.empty(N, 0, dtype=torch.uint8, device="cuda")
    sc = torch.ones(E, K, dtype=torch.float32, device="cuda")
    sd = torch.ones(E, N, dtype=torch.float32, device="cuda")
    dw = torch.full((E, K, N), 7.0, dtype=torch.bfloat16, device="cuda")
    mg.gmm_bwd_fp8(gs, K, N, xc=xc, sxc=sc, dyc=dyc, sdyc=sd, need_dx=False, dw=dw)
    torch.cuda.synchronize()
    assert (dw == 0).all()


def test_fp8_weight_row_stride_must_match_the_codes():
    wq = torch.zeros(64, 256, dtype=torch.uint8, device="cuda")[:, :128]
    sw = torch.ones(1, 64, dtype=torch.float32, device="cuda")
    xq = torch.zeros(16, 128, dtype=torch.uint8, device="cuda")
    sx = torch.ones(16, dtype=torch.float32, device="cuda")
    gs = torch.tensor([16], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        mg.gmm_fwd_fp8(xq, sx, wq, sw, 128, 128, gs, 64)   # the view's rows are 256 bytes apart
    y = mg.gmm_fwd_fp8(xq, sx, wq, sw, None, 128, gs, 64)
    torch.cuda.synchronize()
    assert (y == 0).all()


def _f8i4_case(E, total_M, K, N, seed, counts=None):
    if counts is None:
        counts = wl.uniform_expert_rows(total_M, E, seed)
    X = wl.normal_bf16((total_M, K), 1.0, seed, wl.T_X)
    xq, sx = oracle.quant_rowwise(X)
    Xd = oracle.dequant_rowwise(xq, sx)
    offs = oracle.offsets(counts)
    w4 = torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, device="cuda")   # never read for empty experts
    sw = torch.randn(E, K // 128, N, device="cuda").to(torch.bfloat16)
    ref = np.zeros((total_M, N))
    cn = np.zeros((E, N))
    for e in np.flatnonzero(counts):
        We = oracle.bf16_to_f64(wl.normal_bf16((K, N), 0.02, seed, wl.T_W, int(e)))[None]
        p, s = oracle.quant_int4(We, 128)
        w4[e] = dev(p[0])
        sw[e] = bf16_dev(s[0])
        rows = slice(offs[e], offs[e + 1])
        Wq = oracle.dequant_int4(p, s, 128)
        ref[rows] = oracle.gmm_fwd(Xd[rows], Wq, np.array([counts[e]]))
        cn[e] = vec_norms(Wq[0], 0)
    y = mg.gmm_fwd_f8i4(dev(xq), dev(sx), w4, sw, dev(counts))
    torch.cuda.synchronize()
    return _f64(y), ref, (vec_norms(Xd, 1), cn, group_rows(counts, total_M))


@pytest.mark.parametrize("E,total_M,K,N,seed", [(8, 5, 256, 64, 0), (16, 100, 512, 136, 1), (128, 1, 5120, 8192, 2),
                                                (128, 16, 5120, 8192, 3),
                                                # 70 chunks: the 8-wave kernel, 9 chunks per wave but 7 in the last
                                                (4, 7, 8960, 96, 4),
                                                # an odd chunk count with a wave past the last chunk
                                                # (9 chunks in runs of 4; 1 chunk in runs of 2): that
                                                # wave has no lines and adds nothing
                                                (4, 6, 1152, 72, 5), (6, 9, 128, 40, 6)])
def test_f8i4_sparse_m(E, total_M, K, N, seed):
    got, ref, norms = _f8i4_case(E, total_M, K, N, seed)
    assert_close(got, ref, FP8_TOL, GEMM_FP8, "Y", norms)


def test_f8i4_one_token_over_128_groups_matches_single_group():
    """The routed row gives the same result whether the expert sits among 127
    empty ones or alone (empty groups are skipped, not looped over)."""
    K, N = 1024, 256
    X = wl.normal_bf16((1, K), 1.0, 0, wl.T_X)
    xq, sx = oracle.quant_rowwise(X)
    W = oracle.bf16_to_f64(wl.normal_bf16((1, K, N), 0.02, 0, wl.T_W))
    p, s = oracle.quant_int4(W, 128)
    sizes = np.zeros(128, np.int32)
    sizes[77] = 1
    w4 = torch.zeros(128, N, K // 2, dtype=torch.uint8, device="cuda")
    sw = torch.zeros(128, K // 128, N, dtype=torch.bfloat16, device="cuda")
    w4[77] = dev(p[0])
    sw[77] = bf16_dev(s[0])
    y128 = mg.gmm_fwd_f8i4(dev(xq), dev(sx), w4, sw, dev(sizes))
    y1 = mg.gmm_fwd_f8i4(dev(xq), dev(sx), dev(p), bf16_dev(s), dev(np.array([1], np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(y128, y1)
    A, Wq = oracle.dequant_rowwise(xq, sx), oracle.dequant_int4(p, s, 128)
    assert_close(_f64(y1), oracle.gmm_fwd(A, Wq, np.array([1])), FP8_TOL, GEMM_FP8, "Y", fwd_norms(A, Wq, [1]))


@pytest.mark.parametrize("E,counts,K,N,seed", [
    # one expert holds every row, the rest are empty: the (row tile,
    # 32-column) items fill at most half of a grid sized for one tile per
    # routed row, so K is split across workgroups -- 4 pieces here, with a
    # ragged row count and a ragged last column slice
    (8, [0, 0, 5, 0, 0, 0, 0, 0], 4096, 200, 5),      # 4-wave kernel, 32 chunks
    (8, [0, 0, 0, 0, 0, 0, 0, 9], 8960, 96, 6),       # 8-wave kernel, 70 chunks
])
def test_f8i4_k_split_pieces(E, counts, K, N, seed):
    counts = np.array(counts, np.int32)
    got, ref, norms = _f8i4_case(E, int(counts.sum()), K, N, seed, counts=counts)
    assert_close(got, ref, FP8_TOL, GEMM_FP8, "Y", norms)
