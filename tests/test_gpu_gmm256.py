"""GPU parity of the grouped GEMM on 256 x 256 tiles -- the kernel large
fixed-M launches take (mg.last_gemm_tile_m() says which ran) -- against the
fp64 oracle, every output element.  The shapes are the smallest that route
there (at least two rounds of 256 x 256 tiles on a 256-CU grid, contractions
of 1024 or more, 192 or more rows per group on average) and ragged where it
matters: the contraction ends inside a k-step, the last column tile is
partial, group ends cut row tiles, one group is empty.  Covered: bf16 with B
as [K, N] and as [N, K], dX, e4m3 forward and dX with row and column scales,
the A rows taken through the token-sorted index with and without the
SiLU*mul epilogue, the e4m3 dynamic-K dW over skewed groups whose row
ranges start and end inside 16-byte chunks, a captured launch replayed
after the device group sizes change, and last rounds whose tiles are cut
along the contraction into pieces summed by the last to arrive."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import (BF16_TOL, FP8_TOL, GEMM_BF16, GEMM_FP8, SWIGLU_ELEM, assert_close, bf16_dev, bf16_host, dev,
                      dw_norms, dx_norms, fwd_norms, gpu, group_rows, require_gpu, vec_norms)

pytestmark = gpu

SIZES = np.array([5000, 0, 11384], np.int32)   # M = 16384: 67 row tiles of 256
K, N = 2056, 2000                               # 64.25 bf16 k-steps; 7.8 column tiles


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _f64(t):
    return oracle.bf16_to_f64(bf16_host(t))


def _wide():
    assert mg.last_gemm_tile_m() == 256, "the launch did not take the 256 x 256-tile kernel"


@pytest.mark.parametrize("trans_b", [False, True])
def test_bf16_forward_and_dx(trans_b):
    E, M = len(SIZES), int(SIZES.sum())
    X = wl.normal_bf16((M, K), 1.0, 40, wl.T_X)
    W = wl.stacked_normal_bf16(E, (K, N), 0.05, 40, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 40, wl.T_DY)
    Wg = np.ascontiguousarray(np.transpose(W, (0, 2, 1))) if trans_b else W
    x, w, dy, gs = bf16_dev(X), bf16_dev(Wg), bf16_dev(dY), dev(SIZES)
    y = mg.gmm_fwd(x, w, gs, trans_b=trans_b)
    _wide()
    dx, _ = mg.gmm_bwd(dy, x, w, gs, trans_b=trans_b, need_dw=False)
    _wide()
    torch.cuda.synchronize()
    Xf, Wf, dYf = (oracle.bf16_to_f64(a) for a in (X, W, dY))
    assert_close(_f64(y), oracle.gmm_fwd(Xf, Wf, SIZES), BF16_TOL, GEMM_BF16, "Y", fwd_norms(Xf, Wf, SIZES))
    assert_close(_f64(dx), oracle.gmm_dx(dYf, Wf, SIZES), BF16_TOL, GEMM_BF16, "dX", dx_norms(dYf, Wf, SIZES))


def test_rows_past_the_groups_are_untouched():
    """A row count above the sizes' sum: the rows past it keep their bytes."""
    E, M = len(SIZES), int(SIZES.sum()) + 300
    x = bf16_dev(wl.normal_bf16((M, K), 1.0, 41, wl.T_X))
    w = bf16_dev(wl.stacked_normal_bf16(E, (K, N), 0.05, 41, wl.T_W))
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    mg.gmm_fwd(x, w, dev(SIZES), out=y)
    _wide()
    torch.cuda.synchronize()
    assert (y[int(SIZES.sum()):] == 3.0).all()


def _codes(g, shape):
    mag = g.integers(0, 0x7F, size=shape, dtype=np.uint8)          # 0x7F is NaN
    return mag | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7)


def _scales(g, shape):
    return np.exp2(g.integers(3, 9, size=shape)).astype(np.float32)


def test_fp8_forward_and_dx():
    """e4m3 codes over every binade with power-of-two row and column scales;
    K = 2064 leaves 16 bytes in the last 64-byte k-step."""
    E, M, Kq, Nq = len(SIZES), int(SIZES.sum()), 2064, 2000
    g = wl.rng(42, wl.T_W)
    xq, sx = _codes(g, (M, Kq)), _scales(g, M)
    dyq, sdy = _codes(g, (M, Nq)), _scales(g, M)
    wq_c, sw_c = _codes(g, (E, Nq, Kq)), _scales(g, (E, Nq))   # fwd: W(e,k,n) at (e*Nq + n)*Kq + k, per (e, n)
    wq_r, sw_r = _codes(g, (E * Kq, Nq)), _scales(g, E * Kq)   # dX: W(e,k,n) at (e*Kq + k)*Nq + n, per (e, k)
    gs = dev(SIZES)
    y = mg.gmm_fwd_fp8(dev(xq), dev(sx), dev(wq_c), dev(sw_c), Kq, Nq * Kq, gs, Nq)
    _wide()
    dx, _ = mg.gmm_bwd_fp8(gs, Kq, Nq, dyq=dev(dyq), sdy=dev(sdy), wq=dev(wq_r), sw=dev(sw_r), w_ld=Nq,
                           w_expert_stride=Kq * Nq, need_dw=False)
    _wide()
    torch.cuda.synchronize()
    A = oracle.dequant_rowwise(xq, sx)
    Wf = np.transpose(oracle.dequant_rowwise(wq_c.reshape(E * Nq, Kq), sw_c.reshape(E * Nq)).reshape(E, Nq, Kq),
                      (0, 2, 1))
    assert_close(_f64(y), oracle.gmm_fwd(A, Wf, SIZES), FP8_TOL, GEMM_FP8, "Y", fwd_norms(A, Wf, SIZES))
    A = oracle.dequant_rowwise(dyq, sdy)
    Wr = oracle.dequant_rowwise(wq_r, sw_r).reshape(E, Kq, Nq)
    assert_close(_f64(dx), oracle.gmm_dx(A, Wr, SIZES), FP8_TOL, GEMM_FP8, "dX", dx_norms(A, Wr, SIZES))


def test_fp8_dw_skewed_groups():
    """dW[g] = Xc_g^T . dYc_g over 8 groups of very different sizes (one
    empty, one of 77 rows), so items are dealt longest first in snake order;
    group boundaries fall inside 16-byte chunks, whose bytes of the
    neighbouring groups must not count.  Output 2056 x 2000 per group."""
    sizes = np.array([3001, 0, 517, 9000, 1203, 77, 4100, 2486], np.int32)
    E, M, Kq, Nq = len(sizes), int(sizes.sum()), 2056, 2000
    g = wl.rng(45, wl.T_W)
    xc, sxc = _codes(g, (Kq, M)), _scales(g, (E, Kq))     # column-major codes, per (group, column)
    dyc, sdyc = _codes(g, (Nq, M)), _scales(g, (E, Nq))
    ws = mg.workspace(E, M)
    args = dict(xc=dev(xc), sxc=dev(sxc), dyc=dev(dyc), sdyc=dev(sdyc), need_dx=False, ws=ws)
    _, dw = mg.gmm_bwd_fp8(dev(sizes), Kq, Nq, **args)
    _wide()
    # the items come from a work queue in the workspace header, and the
    # split tiles' arrival counters follow it: both are back at zero after
    # the call, and a second call with the same workspace gives the same bits
    _, dw2 = mg.gmm_bwd_fp8(dev(sizes), Kq, Nq, **args)
    torch.cuda.synchronize()
    assert (ws[:1280].view(torch.int32)[1:] == 0).all()
    assert torch.equal(dw, dw2)
    dwh = _f64(dw)
    Xc, dYc = oracle.dequant_colwise(xc, sxc, sizes), oracle.dequant_colwise(dyc, sdyc, sizes)
    assert_close(dwh, oracle.gmm_dw(Xc, dYc, sizes), FP8_TOL, GEMM_FP8, "dW", dw_norms(Xc, dYc, sizes))
    assert (dwh[1] == 0).all()
    # the same codes in rows of a padded stride (the library's own, and a
    # 16-byte multiple off every power of two) whose pad bytes are NaN
    # codes: the pads are never used, so the bits do not change
    for ld in (mg.colwise_ld(M), M + 48):
        xp = torch.full((Kq, ld), 0x7F, dtype=torch.uint8, device="cuda")
        dp = torch.full((Nq, ld), 0x7F, dtype=torch.uint8, device="cuda")
        xp[:, :M].copy_(dev(xc))
        dp[:, :M].copy_(dev(dyc))
        _, dw3 = mg.gmm_bwd_fp8(dev(sizes), Kq, Nq, xc=xp[:, :M], sxc=dev(sxc), dyc=dp[:, :M], sdyc=dev(sdyc),
                                need_dx=False, ws=ws)
        _wide()
        torch.cuda.synchronize()
        assert torch.equal(dw3, dw), ld


@pytest.mark.parametrize("trans_b", [False, True])
def test_gathered_rows_and_silu_mul_epilogue(trans_b):
    """The token-sorted GEMM1: A rows through sorted_token_ids / top_k with
    zero rows for the padding sentinel, against the oracle on the gathered
    rows; and the same with SiLU*mul in the epilogue (gate and up columns of
    one 256-column tile), against the oracle's GEMM rounded to bf16 and
    passed through its SiLU*mul.  With trans_b the weights are [E, 2I, H]
    (gate rows, then up rows)."""
    T, k, E, H, I = 4096, 2, 8, 1032, 1600
    x = wl.normal_bf16((T, H), 1.0, 43, wl.T_X)
    W1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, 43, wl.T_W)
    ids, _ = wl.softmax_topk_routing(T, E, k, 43)
    xd = bf16_dev(x)
    w1d = bf16_dev(np.ascontiguousarray(np.transpose(W1, (0, 2, 1))) if trans_b else W1)
    p = mg.moe_permute(dev(ids), E, 128)
    sids, sizes = p["sorted_token_ids"], p["padded_sizes"]
    h = mg.gmm_fwd_gather(xd, sids, k, w1d, sizes, trans_b=trans_b)
    _wide()
    act = mg.gmm_fwd_silu_mul(xd, w1d, sizes, sorted_token_ids=sids, top_k=k, trans_b=trans_b)
    _wide()
    torch.cuda.synchronize()
    sz = sizes.cpu().numpy()
    n = int(sz.sum())
    xs = oracle.gather_rows(x, k, sids.cpu().numpy()[:n])
    cn = np.stack([vec_norms(oracle.bf16_to_f64(W1[e]), 0) for e in range(E)])
    h_ref = oracle.gmm_fwd_bf16(xs, W1, sz)
    assert_close(_f64(h)[:n], h_ref, BF16_TOL, GEMM_BF16, "h", (vec_norms(oracle.bf16_to_f64(xs), 1), cn,
                                                                 group_rows(sz, n)))
    assert_close(_f64(act)[:n], oracle.silu_mul(oracle.bf16_to_f64(oracle.f64_to_bf16(h_ref))), BF16_TOL,
                 SWIGLU_ELEM, "act")


def test_captured_launch_follows_device_sizes_changed_between_replays():
    """The group table is built on the device from the sizes at run time: a
    captured launch replayed after the sizes change in place equals a fresh
    eager launch with the new sizes, bit for bit."""
    E, M = 4, 16384
    x = bf16_dev(wl.normal_bf16((M, K), 1.0, 44, wl.T_X))
    w = bf16_dev(wl.stacked_normal_bf16(E, (K, N), 0.05, 44, wl.T_W))
    gs = dev(np.array([4096, 4096, 4096, 4096], np.int32))
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = mg.workspace(E, M)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mg.gmm_fwd(x, w, gs, out=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.gmm_fwd(x, w, gs, out=y, ws=ws)
    for sizes in (np.array([1000, 9000, 0, 6384], np.int32), np.array([16384, 0, 0, 0], np.int32),
                  np.array([3000, 3000, 3000, 7384], np.int32)):
        gs.copy_(dev(sizes))
        y.fill_(5.0)
        g.replay()
        torch.cuda.synchronize()
        y_e = mg.gmm_fwd(x, w, dev(sizes))
        _wide()
        torch.cuda.synchronize()
        assert torch.equal(y, y_e)


def _last_round_pieces(sizes, n_cols, k_steps):
    """(r, P) per XCD of a fixed-M launch: the last round's r tiles and the
    pieces each is cut into (1: whole), from the kernel's rule -- the XCD's
    n tiles over its gx = G / 8 workgroups leave r = n % gx; r <= gx / 4
    cuts each into min(8, gx / r, k_steps / 32) pieces."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = int(sum((int(s) + 255) // 256 for s in sizes)) * ((n_cols + 255) // 256)
    G = min(tiles, cus)
    assert G % 8 == 0
    gx, plan = G // 8, []
    for x in range(8):
        n = (x + 1) * tiles // 8 - x * tiles // 8
        r = n % gx
        p = min(8, gx // r, k_steps // 32) if 0 < 4 * r <= gx else 1
        plan.append((r, p if p >= 2 else 1))
    return plan


LAST_SIZES = np.array([8701, 0, 9211], np.int32)   # 34 + 36 row tiles: 560 tiles of 2000 columns, 70 per XCD
K_LAST, N_LAST = 5128, 2000                         # 160.25 bf16 k-steps; 7.8 column tiles


@pytest.mark.parametrize("trans_b", [False, True])
def test_bf16_last_round_in_pieces(trans_b):
    """560 tiles on 256 CUs: every XCD runs 2 full rounds and a last round of
    6 tiles, each cut into 5 pieces of 32 or 33 k-steps (K = 5128: the last
    piece ends inside a k-step; group ends cut the row tiles).  The arrival
    counters are back at zero after the call, and a second call gives the
    same bits (the pieces are summed in piece order)."""
    E, M = len(LAST_SIZES), int(LAST_SIZES.sum())
    assert set(_last_round_pieces(LAST_SIZES, N_LAST, 161)) == {(6, 5)}
    X = wl.normal_bf16((M, K_LAST), 1.0, 46, wl.T_X)
    W = wl.stacked_normal_bf16(E, (K_LAST, N_LAST), 0.05, 46, wl.T_W)
    Wg = np.ascontiguousarray(np.transpose(W, (0, 2, 1))) if trans_b else W
    x, w, gs = bf16_dev(X), bf16_dev(Wg), dev(LAST_SIZES)
    ws = mg.workspace(E, M)
    y = mg.gmm_fwd(x, w, gs, trans_b=trans_b, ws=ws)
    _wide()
    y2 = mg.gmm_fwd(x, w, gs, trans_b=trans_b, ws=ws)
    torch.cuda.synchronize()
    assert (ws[:1280].view(torch.int32)[1:] == 0).all()
    assert torch.equal(y, y2)
    Xf, Wf = oracle.bf16_to_f64(X), oracle.bf16_to_f64(W)
    assert_close(_f64(y), oracle.gmm_fwd(Xf, Wf, LAST_SIZES), BF16_TOL, GEMM_BF16, "Y",
                 fwd_norms(Xf, Wf, LAST_SIZES))


def test_gathered_rows_last_round_in_pieces():
    """The token-sorted A load on the same 560-tile launch: rows through
    sorted_token_ids / top_k (T = 8192 tokens, top-2), a padding sentinel
    every 40th row giving zero rows."""
    E, M, T, k = len(LAST_SIZES), int(LAST_SIZES.sum()), 8192, 2
    g = wl.rng(47, wl.T_X)
    sids = g.integers(0, T * k, size=M).astype(np.int32)
    sids[::40] = T * k
    x = wl.normal_bf16((T, K_LAST), 1.0, 47, wl.T_X)
    W = wl.stacked_normal_bf16(E, (K_LAST, N_LAST), 0.05, 47, wl.T_W)
    h = mg.gmm_fwd_gather(bf16_dev(x), dev(sids), k, bf16_dev(W), dev(LAST_SIZES))
    _wide()
    torch.cuda.synchronize()
    xs = oracle.gather_rows(x, k, sids)
    Xf, Wf = oracle.bf16_to_f64(xs), oracle.bf16_to_f64(W)
    assert_close(_f64(h), oracle.gmm_fwd(Xf, Wf, LAST_SIZES), BF16_TOL, GEMM_BF16, "h",
                 fwd_norms(Xf, Wf, LAST_SIZES))


def test_fp8_last_round_in_pieces():
    """e4m3 with row and column scales on the 560-tile launch: K = 5136 is 81
    k-steps of 64 bytes, so the 6 last-round tiles of each XCD are cut into
    2 pieces of 40 and 41 k-steps, the scales applied once to their sum."""
    E, M, Kq, Nq = len(LAST_SIZES), int(LAST_SIZES.sum()), 5136, N_LAST
    assert set(_last_round_pieces(LAST_SIZES, Nq, 81)) == {(6, 2)}
    g = wl.rng(48, wl.T_W)
    xq, sx = _codes(g, (M, Kq)), _scales(g, M)
    wq_c, sw_c = _codes(g, (E, Nq, Kq)), _scales(g, (E, Nq))
    y = mg.gmm_fwd_fp8(dev(xq), dev(sx), dev(wq_c), dev(sw_c), Kq, Nq * Kq, dev(LAST_SIZES), Nq)
    _wide()
    torch.cuda.synchronize()
    A = oracle.dequant_rowwise(xq, sx)
    Wf = np.transpose(oracle.dequant_rowwise(wq_c.reshape(E * Nq, Kq), sw_c.reshape(E * Nq)).reshape(E, Nq, Kq),
                      (0, 2, 1))
    assert_close(_f64(y), oracle.gmm_fwd(A, Wf, LAST_SIZES), FP8_TOL, GEMM_FP8, "Y", fwd_norms(A, Wf, LAST_SIZES))
