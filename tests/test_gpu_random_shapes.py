"""GPU parity on seeded random small shapes, beyond the fixed
parametrizations: group counts, row counts (with empty groups and rows past
the groups), contraction and output widths are drawn per case.  Every
output is a view at the start of a larger buffer filled with a marker, and
the marker after the view must survive the call (an overrun past the output
-- the colwise scale store, a ragged last tile -- fails here even where the
parity check cannot see it)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import (BF16_TOL, CHAIN_ELEM, FP8_TOL, GEMM_BF16, GEMM_FP8, assert_close, bf16_dev, bf16_host, dev,
                      dw_norms, dx_norms, fwd_norms, gpu, group_rows, host, require_gpu, vec_norms)

pytestmark = gpu

GUARD = 4096   # elements of marker after every output


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _draw(seed, mult):
    """One case: E groups, M rows of which the groups cover `covered`,
    contraction K and width N (multiples of `mult`)."""
    r = np.random.default_rng(1000 + seed)
    E = int(r.integers(1, 25))
    M = int(r.integers(1, 900))
    covered = M - int(r.integers(0, min(M, 40) + 1))
    K = mult * int(r.integers(1, 400 // mult + 1))
    N = mult * int(r.integers(1, 400 // mult + 1))
    sizes = wl.random_group_sizes(E, covered, seed, zero_frac=0.3) if E > 1 else np.array([covered], np.int32)
    return E, M, K, N, sizes.astype(np.int32)


def _guarded(shape, dtype, fill):
    """A view of `shape` at the start of a buffer with GUARD marker elements after it."""
    n = int(np.prod(shape))
    buf = torch.full((n + GUARD,), fill, dtype=dtype, device="cuda")
    return buf, buf[:n].view(*shape)


def _guard_intact(buf, n, fill):
    tail = buf[n:]
    if tail.dtype == torch.float32 and np.isnan(fill):
        return bool(torch.isnan(tail).all())
    return bool((tail == fill).all())


@pytest.mark.parametrize("seed", range(16))
def test_bf16_random_shapes(seed):
    E, M, K, N, sizes = _draw(seed, 8)
    trans_b = bool(seed % 2)
    covered = int(sizes.sum())
    X = wl.normal_bf16((M, K), 1.0, seed, wl.T_X)
    W = wl.normal_bf16((E, K, N), 0.5, seed, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, seed, wl.T_DY)
    Wg = np.ascontiguousarray(np.transpose(W, (0, 2, 1))) if trans_b else W
    x, w, dy, gs = bf16_dev(X), bf16_dev(Wg), bf16_dev(dY), dev(sizes)
    yb, y = _guarded((M, N), torch.bfloat16, 7.0)
    dxb, dx = _guarded((M, K), torch.bfloat16, 7.0)
    dwb, dw = _guarded(tuple(Wg.shape), torch.bfloat16, 7.0)
    ws = mg.workspace(E, M)
    mg.gmm_fwd(x, w, gs, trans_b=trans_b, out=y, ws=ws)
    mg.gmm_bwd(dy, x, w, gs, trans_b=trans_b, dx=dx, dw=dw, ws=ws)
    torch.cuda.synchronize()
    for b, t in ((yb, y), (dxb, dx), (dwb, dw)):
        assert _guard_intact(b, t.numel(), 7.0)
    assert mg.workspace_error(ws) == 0
    f = lambda t: oracle.bf16_to_f64(bf16_host(t))
    Xf, Wf, dYf = (oracle.bf16_to_f64(a) for a in (X, W, dY))
    yh, dxh, dwh = f(y), f(dx), f(dw)
    if trans_b:
        dwh = np.transpose(dwh, (0, 2, 1))
    assert (yh[covered:] == 7.0).all() and (dxh[covered:] == 7.0).all()   # rows past the groups untouched
    c = covered
    assert_close(yh[:c], oracle.gmm_fwd(Xf[:c], Wf, sizes), BF16_TOL, GEMM_BF16, "Y", fwd_norms(Xf[:c], Wf, sizes))
    assert_close(dxh[:c], oracle.gmm_dx(dYf[:c], Wf, sizes), BF16_TOL, GEMM_BF16, "dX",
                 dx_norms(dYf[:c], Wf, sizes))
    assert_close(dwh, oracle.gmm_dw(Xf[:c], dYf[:c], sizes), BF16_TOL, GEMM_BF16, "dW",
                 dw_norms(Xf[:c], dYf[:c], sizes))


@pytest.mark.parametrize("seed", range(12))
def test_fp8_random_shapes(seed):
    E, M, K, N, sizes = _draw(seed, 16)
    M = max(16, M - M % 16)                      # the e4m3 dW reads its contraction in 16-row steps
    sizes = wl.random_group_sizes(E, M, seed, zero_frac=0.3) if E > 1 else np.array([M], np.int32)
    X = wl.normal_bf16((M, K), 1.0, seed, wl.T_X)
    dY = wl.normal_bf16((M, N), 1.0, seed, wl.T_DY)
    W = wl.stacked_normal_bf16(E, (K, N), 0.02, seed, wl.T_W)
    xq, sx = oracle.quant_rowwise(X)
    wqc, swc = oracle.quant_colwise(W.reshape(E * K, N), np.full(E, K, np.int32))
    dyq, sdy = oracle.quant_rowwise(dY)
    wqr, swr = oracle.quant_rowwise(W.reshape(E * K, N))
    dyc, sdyc = oracle.quant_colwise(dY, sizes)
    xc, sxc = oracle.quant_colwise(X, sizes)
    gs = dev(sizes)
    ws = mg.workspace(E, M)
    yb, y = _guarded((M, N), torch.bfloat16, 7.0)
    mg.gmm_fwd_fp8(dev(xq), dev(sx), dev(wqc), dev(swc), E * K, K, gs, N, out=y, ws=ws)
    dxb, dx = _guarded((M, K), torch.bfloat16, 7.0)
    dwb, dw = _guarded((E, K, N), torch.bfloat16, 7.0)
    mg.gmm_bwd_fp8(gs, K, N, dyq=dev(dyq), sdy=dev(sdy), wq=dev(wqr), sw=dev(swr), w_ld=N, w_expert_stride=K * N,
                   xc=dev(xc), sxc=dev(sxc), dyc=dev(dyc), sdyc=dev(sdyc), dx=dx, dw=dw, ws=ws)
    torch.cuda.synchronize()
    for b, t in ((yb, y), (dxb, dx), (dwb, dw)):
        assert _guard_intact(b, t.numel(), 7.0)
    f = lambda t: oracle.bf16_to_f64(bf16_host(t))
    A = oracle.dequant_rowwise(xq, sx)
    Wc = oracle.dequant_colwise(wqc, swc, np.full(E, K, np.int32)).reshape(E, K, N)
    assert_close(f(y), oracle.gmm_fwd(A, Wc, sizes), FP8_TOL, GEMM_FP8, "Y", fwd_norms(A, Wc, sizes))
    Wr = oracle.dequant_rowwise(wqr, swr).reshape(E, K, N)
    dYr = oracle.dequant_rowwise(dyq, sdy)
    assert_close(f(dx), oracle.gmm_dx(dYr, Wr, sizes), FP8_TOL, GEMM_FP8, "dX", dx_norms(dYr, Wr, sizes))
    Xc, dYc = oracle.dequant_colwise(xc, sxc, sizes), oracle.dequant_colwise(dyc, sdyc, sizes)
    assert_close(f(dw), oracle.gmm_dw(Xc, dYc, sizes), FP8_TOL, GEMM_FP8, "dW", dw_norms(Xc, dYc, sizes))


@pytest.mark.parametrize("seed", range(16))
def test_quantizers_random_shapes(seed):
    E, M, C, C2, sizes = _draw(seed, 8)
    covered = int(sizes.sum())
    a = wl.normal_bf16((M, C), 1.0, seed, wl.T_DY)
    b = wl.normal_bf16((M, C2), 1.0, seed, wl.T_X)
    # rowwise
    qb_, q = _guarded((M, C), torch.uint8, 0xA5)
    sb_, s = _guarded((M,), torch.float32, float("nan"))
    mg.quantize_rowwise_fp8(bf16_dev(a), q=q, scales=s)
    # colwise, dual
    qab, qa = _guarded((C, M), torch.uint8, 0xA5)
    sab, sa = _guarded((E, C), torch.float32, float("nan"))
    qbb, qbv = _guarded((C2, M), torch.uint8, 0xA5)
    sbb, sbv = _guarded((E, C2), torch.float32, float("nan"))
    mg.quantize_colwise_per_group_fp8(bf16_dev(a), dev(sizes), b=bf16_dev(b), out=(qa, sa, qbv, sbv))
    torch.cuda.synchronize()
    assert _guard_intact(qb_, q.numel(), 0xA5) and _guard_intact(sb_, s.numel(), float("nan"))
    for buf, t, fill in ((qab, qa, 0xA5), (sab, sa, float("nan")), (qbb, qbv, 0xA5), (sbb, sbv, float("nan"))):
        assert _guard_intact(buf, t.numel(), fill)
    q_ref, s_ref = oracle.quant_rowwise(a)
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)
    for x, qq, ss in ((a, qa, sa), (b, qbv, sbv)):
        qr, sr = oracle.quant_colwise(x, sizes)
        np.testing.assert_array_equal(host(ss), sr)
        np.testing.assert_array_equal(host(qq)[:, :covered], qr[:, :covered])
        assert (host(qq)[:, covered:] == 0xA5).all()   # rows past the groups untouched


@pytest.mark.parametrize("seed", range(10))
def test_f8i4_random_shapes(seed):
    """Sparse M: a few routed rows over many int4-weight experts."""
    r = np.random.default_rng(2000 + seed)
    E = int(r.integers(1, 65))
    total_M = int(r.integers(1, 48))
    K = 128 * int(r.integers(1, 41))
    N = 8 * int(r.integers(1, 65))
    counts = wl.uniform_expert_rows(total_M, E, seed)
    X = wl.normal_bf16((total_M, K), 1.0, seed, wl.T_X)
    xq, sx = oracle.quant_rowwise(X)
    Xd = oracle.dequant_rowwise(xq, sx)
    offs = oracle.offsets(counts)
    w4 = torch.zeros(E, N, K // 2, dtype=torch.uint8, device="cuda")
    sw = torch.zeros(E, K // 128, N, dtype=torch.bfloat16, device="cuda")
    ref = np.zeros((total_M, N))
    cn = np.zeros((E, N))
    for e in np.flatnonzero(counts):
        We = oracle.bf16_to_f64(wl.normal_bf16((K, N), 0.02, seed, wl.T_W, int(e)))[None]
        p, q = oracle.quant_int4(We, 128)
        w4[e] = dev(p[0])
        sw[e] = bf16_dev(q[0])
        Wq = oracle.dequant_int4(p, q, 128)
        rows = slice(offs[e], offs[e + 1])
        ref[rows] = oracle.gmm_fwd(Xd[rows], Wq, np.array([counts[e]]))
        cn[e] = vec_norms(Wq[0], 0)
    yb, y = _guarded((total_M, N), torch.bfloat16, 7.0)
    ws = mg.workspace(E, total_M)
    mg.gmm_fwd_f8i4(dev(xq), dev(sx), w4, sw, dev(counts), out=y, ws=ws)
    torch.cuda.synchronize()
    assert _guard_intact(yb, y.numel(), 7.0)
    assert mg.workspace_error(ws) == 0
    assert_close(oracle.bf16_to_f64(bf16_host(y)), ref, FP8_TOL, GEMM_FP8, "Y",
                 (vec_norms(Xd, 1), cn, group_rows(counts, total_M)))


@pytest.mark.parametrize("seed", range(10))
def test_fused_moe_random_shapes(seed):
    """The token-sorted FFN end to end (align, gathered GEMM1 with the
    SiLU*mul epilogue, GEMM2, combine) on drawn token counts, expert counts,
    top-k, widths and block sizes, in both weight layouts."""
    r = np.random.default_rng(3000 + seed)
    E = int(r.integers(1, 33))
    k = int(r.integers(1, min(E, 8) + 1))
    T = int(r.integers(1, 300))
    H = 16 * int(r.integers(1, 33))
    I = 16 * int(r.integers(1, 25))
    bm = int(r.choice([16, 32, 64, 128]))
    ids, w = wl.softmax_topk_routing(T, E, k, seed)
    x = wl.normal_bf16((T, H), 1.0, seed, wl.T_X)
    w1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, seed, wl.T_W1)
    w2 = wl.stacked_normal_bf16(E, (I, H), 0.05, seed, wl.T_W2)
    out, _ = mg.fused_moe(bf16_dev(x), bf16_dev(w1), bf16_dev(w2), dev(ids), dev(w), block_m=bm)
    t = lambda a: bf16_dev(np.ascontiguousarray(np.transpose(a, (0, 2, 1))))
    out_t, _ = mg.fused_moe(bf16_dev(x), t(w1), t(w2), dev(ids), dev(w), block_m=bm, trans_b=True)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_moe(x, w1, w2, ids, w, bm)
    assert_close(oracle.bf16_to_f64(bf16_host(out)), ref, BF16_TOL, CHAIN_ELEM)
    assert torch.equal(out, out_t)


@pytest.mark.parametrize("seed", range(6))
def test_wide_tiles_random_shapes(seed):
    """Drawn shapes large enough for the 256 x 256-tile kernel (at least two
    rounds of its tiles, contractions of 1024 or more): bf16 forward and dX
    in either B layout, e4m3 forward, dX and dW.  Tile counts, and so the
    size of the last round (whole, or cut along the contraction), vary with
    the draw."""
    r = np.random.default_rng(4000 + seed)
    E = int(r.integers(1, 13))
    ct = int(r.integers(5, 10))                       # column tiles of 256
    N = 16 * int(r.integers((ct - 1) * 16 + 1, ct * 16 + 1))
    K = 16 * int(r.integers(64, 101))                 # 1024 .. 1600
    M = -(-520 // ct) * 256 + 16 * int(r.integers(0, 190))
    sizes = wl.random_group_sizes(E, M, seed, zero_frac=0.2) if E > 1 else np.array([M], np.int32)
    trans_b = bool(seed % 2)
    # dX (output width K) takes the wide tiles only with two rounds of them
    dx_wide = (M // 256 + min(M, E)) * (-(-K // 256)) >= 2 * 256
    X = wl.normal_bf16((M, K), 1.0, seed, wl.T_X)
    W = wl.stacked_normal_bf16(E, (K, N), 0.05, seed, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, seed, wl.T_DY)
    Wg = np.ascontiguousarray(np.transpose(W, (0, 2, 1))) if trans_b else W
    x, w, dy, gs = bf16_dev(X), bf16_dev(Wg), bf16_dev(dY), dev(sizes)
    ws = mg.workspace(E, M)
    yb, y = _guarded((M, N), torch.bfloat16, 7.0)
    mg.gmm_fwd(x, w, gs, trans_b=trans_b, out=y, ws=ws)
    assert mg.last_gemm_tile_m() == 256
    dxb, dx = _guarded((M, K), torch.bfloat16, 7.0)
    mg.gmm_bwd(dy, x, w, gs, trans_b=trans_b, need_dw=False, dx=dx, ws=ws)
    assert mg.last_gemm_tile_m() == (256 if dx_wide else 128)
    torch.cuda.synchronize()
    assert _guard_intact(yb, y.numel(), 7.0) and _guard_intact(dxb, dx.numel(), 7.0)
    f = lambda t: oracle.bf16_to_f64(bf16_host(t))
    Xf, Wf, dYf = (oracle.bf16_to_f64(a) for a in (X, W, dY))
    assert_close(f(y), oracle.gmm_fwd(Xf, Wf, sizes), BF16_TOL, GEMM_BF16, "Y", fwd_norms(Xf, Wf, sizes))
    assert_close(f(dx), oracle.gmm_dx(dYf, Wf, sizes), BF16_TOL, GEMM_BF16, "dX", dx_norms(dYf, Wf, sizes))
    # e4m3 on the same operands
    xq, sx = oracle.quant_rowwise(X)
    wqc, swc = oracle.quant_colwise(W.reshape(E * K, N), np.full(E, K, np.int32))
    dyq, sdy = oracle.quant_rowwise(dY)
    wqr, swr = oracle.quant_rowwise(W.reshape(E * K, N))
    yb8, y8 = _guarded((M, N), torch.bfloat16, 7.0)
    mg.gmm_fwd_fp8(dev(xq), dev(sx), dev(wqc), dev(swc), E * K, K, gs, N, out=y8, ws=ws)
    assert mg.last_gemm_tile_m() == 256
    dxb8, dx8 = _guarded((M, K), torch.bfloat16, 7.0)
    mg.gmm_bwd_fp8(gs, K, N, dyq=dev(dyq), sdy=dev(sdy), wq=dev(wqr), sw=dev(swr), w_ld=N, w_expert_stride=K * N,
                   need_dw=False, dx=dx8, ws=ws)
    assert mg.last_gemm_tile_m() == (256 if dx_wide else 128)
    dyc, sdyc = oracle.quant_colwise(dY, sizes)
    xc, sxc = oracle.quant_colwise(X, sizes)
    dwb8, dw8 = _guarded((E, K, N), torch.bfloat16, 7.0)
    mg.gmm_bwd_fp8(gs, K, N, xc=dev(xc), sxc=dev(sxc), dyc=dev(dyc), sdyc=dev(sdyc), need_dx=False, dw=dw8, ws=ws)
    torch.cuda.synchronize()
    for b, t in ((yb8, y8), (dxb8, dx8), (dwb8, dw8)):
        assert _guard_intact(b, t.numel(), 7.0)
    assert mg.workspace_error(ws) == 0
    A = oracle.dequant_rowwise(xq, sx)
    Wc = oracle.dequant_colwise(wqc, swc, np.full(E, K, np.int32)).reshape(E, K, N)
    assert_close(f(y8), oracle.gmm_fwd(A, Wc, sizes), FP8_TOL, GEMM_FP8, "Y8", fwd_norms(A, Wc, sizes))
    Wr = oracle.dequant_rowwise(wqr, swr).reshape(E, K, N)
    dYr = oracle.dequant_rowwise(dyq, sdy)
    assert_close(f(dx8), oracle.gmm_dx(dYr, Wr, sizes), FP8_TOL, GEMM_FP8, "dX8", dx_norms(dYr, Wr, sizes))
    Xc, dYc = oracle.dequant_colwise(xc, sxc, sizes), oracle.dequant_colwise(dyc, sdyc, sizes)
    assert_close(f(dw8), oracle.gmm_dw(Xc, dYc, sizes), FP8_TOL, GEMM_FP8, "dW8", dw_norms(Xc, dYc, sizes))


@pytest.mark.parametrize("seed", range(8))
def test_f8i4_split_random_shapes(seed):
    """Sparse M with the rows in one to three experts of up to 16: the items
    then fill a fraction of a grid sized for one tile per possible expert,
    so the contraction is split across workgroups (pieces summed by the
    last to arrive); odd chunk counts and the 8-wave kernel (64 chunks or
    more) come up among the draws."""
    r = np.random.default_rng(5000 + seed)
    E = int(r.integers(2, 17))
    touched = r.choice(E, size=int(r.integers(1, 4)), replace=False)
    total_M = int(r.integers(1, 61))
    K = 128 * int(r.integers(1, 81))
    N = 8 * int(r.integers(1, 65))
    counts = np.zeros(E, np.int32)
    for i in range(total_M):
        counts[touched[i % len(touched)]] += 1
    X = wl.normal_bf16((total_M, K), 1.0, seed, wl.T_X)
    xq, sx = oracle.quant_rowwise(X)
    Xd = oracle.dequant_rowwise(xq, sx)
    offs = oracle.offsets(counts)
    w4 = torch.zeros(E, N, K // 2, dtype=torch.uint8, device="cuda")
    sw = torch.zeros(E, K // 128, N, dtype=torch.bfloat16, device="cuda")
    ref = np.zeros((total_M, N))
    cn = np.zeros((E, N))
    for e in np.flatnonzero(counts):
        We = oracle.bf16_to_f64(wl.normal_bf16((K, N), 0.02, seed, wl.T_W, int(e)))[None]
        p, q = oracle.quant_int4(We, 128)
        w4[e] = dev(p[0])
        sw[e] = bf16_dev(q[0])
        Wq = oracle.dequant_int4(p, q, 128)
        rows = slice(offs[e], offs[e + 1])
        ref[rows] = oracle.gmm_fwd(Xd[rows], Wq, np.array([counts[e]]))
        cn[e] = vec_norms(Wq[0], 0)
    yb, y = _guarded((total_M, N), torch.bfloat16, 7.0)
    ws = mg.workspace(E, total_M)
    mg.gmm_fwd_f8i4(dev(xq), dev(sx), w4, sw, dev(counts), out=y, ws=ws)
    y2 = mg.gmm_fwd_f8i4(dev(xq), dev(sx), w4, sw, dev(counts), ws=ws)   # counters back at zero: same bits
    torch.cuda.synchronize()
    assert _guard_intact(yb, y.numel(), 7.0)
    assert torch.equal(y, y2)
    assert mg.workspace_error(ws) == 0
    assert_close(oracle.bf16_to_f64(bf16_host(y)), ref, FP8_TOL, GEMM_FP8, "Y",
                 (vec_norms(Xd, 1), cn, group_rows(counts, total_M)))
