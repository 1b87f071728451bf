"""GPU parity: device argument builder and the bf16 grouped GEMM (forward,
dX, dynamic-K dW) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import (BF16_TOL, GEMM_BF16, assert_close, bf16_dev, bf16_host, dev, dw_norms, dx_norms, fwd_norms,
                      gpu, host, require_gpu)

pytestmark = gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


# --------------------------------------------------------------------------
# builder
# --------------------------------------------------------------------------

@pytest.mark.parametrize("E,total,bm,seed", [
    (4, 37, 16, 0), (8, 1024, 128, 1), (128, 1, 32, 2), (128, 16, 32, 3), (128, 128, 32, 4),
    (64, 5000, 128, 5), (1024, 20000, 16, 6), (1, 0, 128, 7), (7, 3, 1, 8), (300, 777, 64, 9),
    (65, 5000, 128, 10), (63, 999, 16, 11), (1, 77, 16, 12),
    # four groups per lane of one wave (65..256 groups), ragged last lane
    (129, 3000, 32, 13), (255, 70000, 128, 14), (256, 256, 1, 15), (256, 0, 32, 16), (257, 4000, 64, 17),
    (200, 9, 16, 18),
])
def test_builder_fixed_m_bit_exact(E, total, bm, seed):
    sizes = wl.random_group_sizes(E, total, seed, zero_frac=0.5)
    offs, count, ent = mg.build_worklist(mg.MG_WL_FIXED_M, dev(sizes), total, bm)
    torch.cuda.synchronize()
    n_ref, ent_ref = oracle.worklist_fixed_m(sizes, bm)
    np.testing.assert_array_equal(host(offs), oracle.offsets(sizes))
    assert int(host(count)[0]) == n_ref
    np.testing.assert_array_equal(host(ent)[:n_ref], ent_ref)


@pytest.mark.parametrize("E,total,seed", [(8, 1024, 0), (64, 98304, 1), (1024, 3000, 2), (3, 0, 3), (128, 1, 4),
                                          (65, 4000, 5), (1, 9, 6), (129, 5000, 7), (256, 100000, 8),
                                          (255, 300, 9), (257, 6000, 10), (200, 0, 11)])
def test_builder_dynamic_k_bit_exact(E, total, seed):
    sizes = wl.random_group_sizes(E, total, seed, zero_frac=0.3)
    sizes[: E // 3] = sizes[0]   # ties
    total = int(sizes.sum())
    offs, count, ent = mg.build_worklist(mg.MG_WL_DYNAMIC_K, dev(sizes), total, 128)
    torch.cuda.synchronize()
    assert int(host(count)[0]) == E
    np.testing.assert_array_equal(host(ent), oracle.worklist_dynamic_k(sizes))
    np.testing.assert_array_equal(host(offs), oracle.offsets(sizes))


def test_builder_flags_bad_sizes_without_writing_out_of_bounds():
    E, M, K, N = 4, 64, 64, 64
    x = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(E, K, N, dtype=torch.bfloat16, device="cuda")
    canary = torch.full((M + 64, N), 7.0, dtype=torch.bfloat16, device="cuda")
    y = canary[:M]
    big = 2**31 - 1   # running sums past int32: the error is still "sum past total_M"
    for sizes, code in [([10, -5, 20, 30], 1), ([40, 40, 0, 0], 2), ([big, big, big, 0], 2), ([big, -1, big, 3], 1)]:
        ws = mg.workspace(E, M)
        mg.workspace_clear(ws)
        mg.gmm_fwd(x, w, dev(np.array(sizes, np.int32)), out=y, ws=ws)
        torch.cuda.synchronize()
        assert mg.workspace_error(ws) == code
        assert (canary[M:] == 7.0).all()
    ws = mg.workspace(E, M)
    mg.workspace_clear(ws)
    mg.gmm_fwd(x, w, dev(np.array([10, 20, 30, 4], np.int32)), out=y, ws=ws)
    torch.cuda.synchronize()
    assert mg.workspace_error(ws) == 0


@pytest.mark.parametrize("E", [64, 65, 256, 257])   # one group per lane, four per lane, workgroup-wide
def test_builder_flags_survive_int32_running_sums(E):
    M, K, N = 64, 64, 64
    big = 2**31 - 1
    x = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(E, K, N, dtype=torch.bfloat16, device="cuda")
    canary = torch.full((M + 64, N), 7.0, dtype=torch.bfloat16, device="cuda")
    y = canary[:M]
    over = [big, big, big] + [0] * (E - 3)
    neg = [big, -1] + [1] * (E - 2)
    for sizes, code in [(over, 2), (neg, 1)]:
        ws = mg.workspace(E, M)
        mg.workspace_clear(ws)
        mg.gmm_fwd(x, w, dev(np.array(sizes, np.int32)), out=y, ws=ws)
        torch.cuda.synchronize()
        assert mg.workspace_error(ws) == code
        assert (canary[M:] == 7.0).all()


# --------------------------------------------------------------------------
# bf16 grouped GEMM
# --------------------------------------------------------------------------

def _run_all(X, W, dY, sizes, trans_b):
    """GPU forward/dX/dW from numpy bf16 bits; returns fp64 numpy results."""
    Wg = np.ascontiguousarray(np.transpose(W, (0, 2, 1))) if trans_b else W
    gs = dev(sizes)
    y = mg.gmm_fwd(bf16_dev(X), bf16_dev(Wg), gs, trans_b=trans_b)
    dx, dw = mg.gmm_bwd(bf16_dev(dY), bf16_dev(X), bf16_dev(Wg), gs, trans_b=trans_b)
    torch.cuda.synchronize()
    f = lambda t: oracle.bf16_to_f64(bf16_host(t))
    dwh = f(dw)
    if trans_b:
        dwh = np.transpose(dwh, (0, 2, 1))
    return f(y), f(dx), dwh


def _check_products(y, dx, dw, X, W, dY, sizes):
    """Y, dX and dW (fp64 of the library's bf16, dW laid out [E, K, N])
    against the oracle on the same bf16 operands, every element."""
    Xf, Wf, dYf = (oracle.bf16_to_f64(a) for a in (X, W, dY))
    assert_close(y, oracle.gmm_fwd(Xf, Wf, sizes), BF16_TOL, GEMM_BF16, "Y", fwd_norms(Xf, Wf, sizes))
    assert_close(dx, oracle.gmm_dx(dYf, Wf, sizes), BF16_TOL, GEMM_BF16, "dX", dx_norms(dYf, Wf, sizes))
    assert_close(dw, oracle.gmm_dw(Xf, dYf, sizes), BF16_TOL, GEMM_BF16, "dW", dw_norms(Xf, dYf, sizes))


def test_tiny_config_forward_and_backward():
    c = wl.tiny_bf16(seed=0)
    dY = wl.normal_bf16((c["M"], c["N"]), 1.0, 0, wl.T_DY)
    y, dx, dw = _run_all(c["X"], c["W"], dY, c["sizes"], False)
    _check_products(y, dx, dw, c["X"], c["W"], dY, c["sizes"])
    assert (dw[0] == 0).all()   # the empty group


@pytest.mark.parametrize("trans_b", [False, True])
@pytest.mark.parametrize("E,M,K,N,seed", [
    (5, 300, 200, 264, 0),      # ragged in every dimension, several tiles
    (3, 513, 136, 392, 1),
    (1, 129, 64, 128, 2),       # one group: plain GEMM
    (17, 700, 72, 40, 3),       # many groups, some empty
    (8, 1024, 256, 384, 4),     # balanced
    # more than 256 rows per group on average: dW on 128 x 256 tiles with
    # three stages (the cases above take the 256 x 256 two-stage dW tiles)
    (2, 1100, 136, 392, 5),
    (3, 2000, 72, 264, 6),
])
def test_bf16_gmm_matches_oracle(E, M, K, N, seed, trans_b):
    sizes = wl.random_group_sizes(E, M, seed, zero_frac=0.25) if E > 1 else np.array([M], np.int32)
    if E == 8:
        sizes = np.full(8, M // 8, np.int32)
    X = wl.normal_bf16((M, K), 1.0, seed, wl.T_X)
    W = wl.normal_bf16((E, K, N), 0.5, seed, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, seed, wl.T_DY)
    y, dx, dw = _run_all(X, W, dY, sizes, trans_b)
    _check_products(y, dx, dw, X, W, dY, sizes)
    for g in np.flatnonzero(sizes == 0):
        assert (dw[g] == 0).all()


@pytest.mark.parametrize("M,N,K", [
    (1280, 5120, 256),   # 200 tiles on 256 workgroups: whole tiles, partial last round spread over the XCDs
    (4352, 4096, 256),   # 544 tiles: one whole round, then stream-K over the last 288 tiles (2-3 pieces each)
    (384, 1024, 1024),   # 12 tiles: stream-K only, 16 k-steps each cut into many pieces
])
def test_fixed_m_schedule_paths(M, N, K):
    """One group, so the tile count is chosen exactly; forward and dX take
    every schedule the fixed-M kernel has on a full 256-CU grid."""
    sizes = np.array([M], np.int32)
    X = wl.normal_bf16((M, K), 1.0, 7, wl.T_X)
    W = wl.normal_bf16((1, K, N), 0.5, 7, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 7, wl.T_DY)
    x, w, dy, gs = bf16_dev(X), bf16_dev(W), bf16_dev(dY), dev(sizes)
    y = mg.gmm_fwd(x, w, gs)
    dx, _ = mg.gmm_bwd(dy, x, w, gs, need_dw=False)
    torch.cuda.synchronize()
    Xf, Wf, dYf = (oracle.bf16_to_f64(a) for a in (X, W, dY))
    assert_close(oracle.bf16_to_f64(bf16_host(y)), oracle.gmm_fwd(Xf, Wf, sizes), BF16_TOL, GEMM_BF16, "Y",
                 fwd_norms(Xf, Wf, sizes))
    assert_close(oracle.bf16_to_f64(bf16_host(dx)), oracle.gmm_dx(dYf, Wf, sizes), BF16_TOL, GEMM_BF16, "dX",
                 dx_norms(dYf, Wf, sizes))


def test_rows_past_the_groups_are_untouched():
    E, M, K, N = 4, 200, 64, 64
    sizes = np.array([30, 0, 50, 20], np.int32)     # sum 100 < 200
    X = wl.normal_bf16((M, K), 1.0, 0, wl.T_X)
    W = wl.normal_bf16((E, K, N), 1.0, 0, wl.T_W)
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    mg.gmm_fwd(bf16_dev(X), bf16_dev(W), dev(sizes), out=y)
    torch.cuda.synchronize()
    yh = oracle.bf16_to_f64(bf16_host(y))
    assert (yh[100:] == 3.0).all()
    Xf, Wf = oracle.bf16_to_f64(X[:100]), oracle.bf16_to_f64(W)
    assert_close(yh[:100], oracle.gmm_fwd(Xf, Wf, sizes), BF16_TOL, GEMM_BF16, "Y", fwd_norms(Xf, Wf, sizes))


def test_zero_group_insertion_is_bitwise_invariant():
    E, M, K, N = 5, 260, 128, 192
    sizes = wl.random_group_sizes(E, M, 3, zero_frac=0.0)
    X = wl.normal_bf16((M, K), 1.0, 1, wl.T_X)
    W = wl.normal_bf16((E, K, N), 1.0, 1, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 1, wl.T_DY)
    base = _run_all(X, W, dY, sizes, False)
    junk = wl.normal_bf16((K, N), 100.0, 9, wl.T_W)
    for pos in [0, 2, 5]:
        s2 = np.insert(sizes, pos, 0)
        W2 = np.insert(W, pos, junk, axis=0)
        y, dx, dw = _run_all(X, W2, dY, s2, False)
        np.testing.assert_array_equal(y, base[0])
        np.testing.assert_array_equal(dx, base[1])
        np.testing.assert_array_equal(np.delete(dw, pos, axis=0), base[2])
        assert (dw[pos] == 0).all()


def test_deterministic_and_empty_total():
    E, M, K, N = 6, 333, 96, 104
    sizes = wl.random_group_sizes(E, M, 5)
    X = wl.normal_bf16((M, K), 1.0, 5, wl.T_X)
    W = wl.normal_bf16((E, K, N), 1.0, 5, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 5, wl.T_DY)
    a = _run_all(X, W, dY, sizes, False)
    b = _run_all(X, W, dY, sizes, False)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    # total_M = 0: forward is a no-op, dW is all zeros
    x0 = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    dy0 = torch.empty(0, N, dtype=torch.bfloat16, device="cuda")
    w = bf16_dev(W)
    gs = dev(np.zeros(E, np.int32))
    assert mg.gmm_fwd(x0, w, gs).shape == (0, N)
    dw = torch.full_like(w, 5.0)
    mg.gmm_bwd(dy0, x0, w, gs, need_dx=False, dw=dw)
    torch.cuda.synchronize()
    assert (dw == 0).all()


def test_balanced_config_full_size():
    """E=8, M=1024 (128 rows each), K=4096, N=6400; X, W uniform[0,1);
    dY = ones.  Every element: Y against the oracle's forward, dX and dW
    against closed forms evaluated in fp64 (dX[r,k] = sum_n W[g,k,n];
    dW[g,k,n] = sum_{r in g} X[r,k] for every n)."""
    c = wl.balanced_bf16(seed=0)
    E, M, K, N = c["E"], c["M"], c["K"], c["N"]
    sizes = c["sizes"]
    gs = dev(sizes)
    x, w, dy = bf16_dev(c["X"]), bf16_dev(c["W"]), bf16_dev(c["dY"])
    y = mg.gmm_fwd(x, w, gs)
    dx, dw = mg.gmm_bwd(dy, x, w, gs)
    torch.cuda.synchronize()
    Xf, Wf, dYf = (oracle.bf16_to_f64(a) for a in (c["X"], c["W"], c["dY"]))
    assert_close(oracle.bf16_to_f64(bf16_host(y)), oracle.gmm_fwd(Xf, Wf, sizes), BF16_TOL, GEMM_BF16, "Y",
                 fwd_norms(Xf, Wf, sizes))
    # dX in full
    dx_ref = np.repeat(Wf.sum(axis=2), 128, axis=0)
    assert_close(oracle.bf16_to_f64(bf16_host(dx)), dx_ref, BF16_TOL, GEMM_BF16, "dX", dx_norms(dYf, Wf, sizes))
    del Wf, dx_ref
    # dW: constant along n, equal to the group's column sums of X
    dwh = oracle.bf16_to_f64(bf16_host(dw))
    colsum = Xf.reshape(E, 128, K).sum(axis=1)
    assert_close(dwh[:, :, :1], colsum[:, :, None], BF16_TOL, GEMM_BF16, "dW", dw_norms(Xf, dYf[:, :1], sizes))
    assert (dwh == dwh[:, :, :1]).all()


def test_captured_step_replays_bitwise():
    """The library's calls are legal under stream capture (no allocation, no
    synchronization, no memset): a captured forward + dX + dW, plus both
    fp8 quantizers, replayed several times with eager work between the
    replays, reproduces the eager outputs bit for bit each time."""
    E, M, K, N = 5, 300, 128, 192
    sizes = wl.random_group_sizes(E, M, 4, zero_frac=0.2)
    X = wl.normal_bf16((M, K), 1.0, 4, wl.T_X)
    W = wl.normal_bf16((E, K, N), 0.5, 4, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 4, wl.T_DY)
    x, w, dy, gs = bf16_dev(X), bf16_dev(W), bf16_dev(dY), dev(sizes)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty_like(w)
    xq = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    cq = (torch.zeros(N, M, dtype=torch.uint8, device="cuda"), torch.empty(E, N, dtype=torch.float32, device="cuda"))
    ws = mg.workspace(E, M)
    cws = torch.zeros(mg.colwise_workspace_bytes(E, M, N), dtype=torch.uint8, device="cuda")

    def step():
        mg.gmm_fwd(x, w, gs, out=y, ws=ws)
        mg.gmm_bwd(dy, x, w, gs, need_dw=False, dx=dx, ws=ws)
        mg.gmm_bwd(dy, x, w, gs, need_dx=False, dw=dw, ws=ws)
        mg.quantize_rowwise_fp8(x, q=xq, scales=sx)
        mg.quantize_colwise_per_group_fp8(dy, gs, out=cq, ws=cws)

    outs = (y, dx, dw, xq, sx, cq[0], cq[1])
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r)
        step()   # eager work between the replays
        torch.cuda.synchronize()


def test_captured_step_follows_device_sizes_changed_between_replays():
    """The group sizes are read on the device at run time, never on the host,
    so one captured forward + dX + dW serves every routing: the sizes (and
    the token rows) are overwritten in place between replays -- empty
    groups, a sum below the row count, one group holding everything -- and
    each replay equals a fresh eager run with the new sizes, bit for bit."""
    E, M, K, N = 6, 400, 128, 192
    W = wl.normal_bf16((E, K, N), 0.5, 8, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 8, wl.T_DY)
    w, dy = bf16_dev(W), bf16_dev(dY)
    x = bf16_dev(wl.normal_bf16((M, K), 1.0, 8, wl.T_X))
    gs = dev(wl.random_group_sizes(E, M, 8))
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty_like(w)
    ws = mg.workspace(E, M)

    def step():
        mg.gmm_fwd(x, w, gs, out=y, ws=ws)
        mg.gmm_bwd(dy, x, w, gs, dx=dx, dw=dw, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    cases = [wl.random_group_sizes(E, M, 21, zero_frac=0.4), np.array([0, 0, M, 0, 0, 0], np.int32),
             np.array([10, 0, 130, 7, 0, 53], np.int32), wl.random_group_sizes(E, M, 22)]
    for i, sizes in enumerate(cases):
        xs = wl.normal_bf16((M, K), 1.0, 30 + i, wl.T_X)
        gs.copy_(dev(sizes))
        x.copy_(bf16_dev(xs))
        for t in (y, dx, dw):
            t.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        s = int(sizes.sum())
        ws2 = mg.workspace(E, M)
        y_e = mg.gmm_fwd(x, w, dev(sizes), ws=ws2)
        dx_e, dw_e = mg.gmm_bwd(dy, x, w, dev(sizes), ws=ws2)
        torch.cuda.synchronize()
        assert torch.equal(y[:s], y_e[:s]) and torch.equal(dx[:s], dx_e[:s]) and torch.equal(dw, dw_e)
        assert (y[s:] == 7.0).all() and (dx[s:] == 7.0).all()
        Xf, Wf = oracle.bf16_to_f64(xs[:s]), oracle.bf16_to_f64(W)
        assert_close(oracle.bf16_to_f64(bf16_host(y[:s])), oracle.gmm_fwd(Xf, Wf, sizes), BF16_TOL, GEMM_BF16, "Y",
                     fwd_norms(Xf, Wf, sizes))


def _zipf_sizes(E, M, s=1.1):
    w = 1.0 / np.arange(1, E + 1) ** s
    sz = np.floor(M * w / w.sum()).astype(np.int32)
    sz[0] += M - int(sz.sum())
    return sz


@pytest.mark.parametrize("E,sizes,K,N,trans_b", [
    # one group holds 95% of the rows: its tiles' contraction (60 k-steps)
    # is cut into 8 pieces summed by the last to arrive
    (4, [3800, 100, 0, 100], 264, 392, False),
    (4, [3800, 100, 0, 100], 264, 392, True),
    # Zipf(1.1) loads over 16 groups
    (16, "zipf", 136, 200, False),
    # one very large group among many small ones
    (64, [20000] + [50] * 63, 128, 128, False),
])
def test_dw_split_contraction_skewed_groups(E, sizes, K, N, trans_b):
    """dW of skewed groups, where the long contractions are split across
    workgroups, matches the oracle element by element and is the same bits
    on every run (the pieces are summed in piece order)."""
    sizes = _zipf_sizes(E, 9000) if sizes == "zipf" else np.array(sizes, np.int32)
    M = int(sizes.sum())
    X = wl.normal_bf16((M, K), 1.0, 13, wl.T_X)
    W = wl.normal_bf16((E, K, N), 0.5, 13, wl.T_W)
    dY = wl.normal_bf16((M, N), 1.0, 13, wl.T_DY)
    Wg = np.ascontiguousarray(np.transpose(W, (0, 2, 1))) if trans_b else W
    x, w, dy, gs = bf16_dev(X), bf16_dev(Wg), bf16_dev(dY), dev(sizes)
    _, dw1 = mg.gmm_bwd(dy, x, w, gs, trans_b=trans_b, need_dx=False)
    _, dw2 = mg.gmm_bwd(dy, x, w, gs, trans_b=trans_b, need_dx=False)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2)
    dwh = oracle.bf16_to_f64(bf16_host(dw1))
    if trans_b:
        dwh = np.ascontiguousarray(np.transpose(dwh, (0, 2, 1)))
    Xf, dYf = oracle.bf16_to_f64(X), oracle.bf16_to_f64(dY)
    assert_close(dwh, oracle.gmm_dw(Xf, dYf, sizes), BF16_TOL, GEMM_BF16, "dW", dw_norms(Xf, dYf, sizes))
    for g in np.flatnonzero(sizes == 0):
        assert (dwh[g] == 0).all()
