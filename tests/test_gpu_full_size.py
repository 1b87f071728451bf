"""GPU parity at the full sizes of the sparse-M, fp8 and fused-FFN workloads,
in the launch configurations bench.py times, on sampled outputs that the
oracle computes from the identical operands (the oracle runs its own GEMM
routine on the sampled rows and columns only).  The balanced bf16 workload
is covered at full size in test_gpu_gmm_bf16.py."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import BF16_TOL, FP8_TOL, bf16_dev, bf16_host, dev, gpu, host, rel_fro, require_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _f64(t):
    return oracle.bf16_to_f64(bf16_host(t))


def _rows_by_group(rows, offs):
    """Sampled rows (sorted) -> sizes of the sub-problem's groups."""
    return np.array([np.sum((rows >= offs[g]) & (rows < offs[g + 1])) for g in range(offs.size - 1)], np.int32)


# --------------------------------------------------------------------------
# FP8 layer share: 16384 tokens, 64 experts, top-6 Zipf(1.1), hidden 2048,
# expert intermediate 1408 (M = 98304 routed rows).  The GEMMs take e4m3
# codes and fp32 scales, whatever produced them, so the codes are drawn
# directly (every finite e4m3 pattern but the NaNs) with power-of-two scales
# like the quantizers' (the quantizers are checked bit-exactly on their own).
# --------------------------------------------------------------------------

def _codes(g, shape):
    mag = g.integers(0, 0x7F, size=shape, dtype=np.uint8)          # 0x7F is NaN
    return mag | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7)


def _scales(g, shape):
    return np.exp2(g.integers(3, 9, size=shape)).astype(np.float32)


def test_fp8_layer_share_full_size_sampled():
    T, E, k, H, I = 16384, 64, 6, 2048, 1408
    ids = wl.zipf_topk_routing(T, E, k, 1.1, seed=0)
    sizes = np.bincount(ids.ravel(), minlength=E).astype(np.int32)
    M = int(sizes.sum())
    offs = oracle.offsets(sizes)
    g = wl.rng(0, wl.T_W)
    xq, sx = _codes(g, (M, H)), _scales(g, M)
    dyq, sdy = _codes(g, (M, I)), _scales(g, M)
    wq_c, sw_c = _codes(g, (I, E * H)), _scales(g, (E, I))      # fwd: W(e,k,n) at n*E*H + e*H + k, per (e, n)
    wq_r, sw_r = _codes(g, (E * H, I)), _scales(g, E * H)       # dX: W(e,k,n) at (e*H + k)*I + n, per (e, k)
    xc, sxc = _codes(g, (H, M)), _scales(g, (E, H))             # dW: column-major codes, per (group, column)
    dyc, sdyc = _codes(g, (I, M)), _scales(g, (E, I))
    gs = dev(sizes)
    y = mg.gmm_fwd_fp8(dev(xq), dev(sx), dev(wq_c), dev(sw_c), E * H, H, gs, I)
    dx, dw = mg.gmm_bwd_fp8(gs, H, I, dyq=dev(dyq), sdy=dev(sdy), wq=dev(wq_r), sw=dev(sw_r), w_ld=I,
                            w_expert_stride=H * I, xc=dev(xc), sxc=dev(sxc), dyc=dev(dyc), sdyc=dev(sdyc))
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    # rows from every group, including the largest and the smallest
    rows = np.unique(np.concatenate([rng.choice(M, 40, replace=False),
                                     offs[np.argmax(sizes)] + np.arange(3), offs[np.argmin(sizes)] + np.arange(2)]))
    sub = _rows_by_group(rows, offs)
    ncol = np.sort(rng.choice(I, 24, replace=False))
    kcol = np.sort(rng.choice(H, 24, replace=False))

    # forward: Y[r, n] for sampled rows and columns
    w_f = oracle.dequant_colwise(wq_c[ncol], sw_c[:, ncol], np.full(E, H, np.int32)).reshape(E, H, ncol.size)
    y_ref = oracle.gmm_fwd(oracle.dequant_rowwise(xq[rows], sx[rows]), w_f, sub)
    assert rel_fro(_f64(y)[np.ix_(rows, ncol)], y_ref) <= FP8_TOL

    # dX: dX[r, k] for sampled rows and k
    wrows = (np.arange(E)[:, None] * H + kcol[None, :]).ravel()       # W rows (e, k) of the sampled k
    w_r = oracle.dequant_rowwise(wq_r[wrows], sw_r[wrows]).reshape(E, kcol.size, I)
    dx_ref = oracle.gmm_dx(oracle.dequant_rowwise(dyq[rows], sdy[rows]), w_r, sub)
    assert rel_fro(_f64(dx)[np.ix_(rows, kcol)], dx_ref) <= FP8_TOL

    # dW: dW[g, k, n] for sampled k and n over every group (all M rows)
    xd = oracle.dequant_colwise(xc[kcol], sxc[:, kcol], sizes)
    dyd = oracle.dequant_colwise(dyc[ncol], sdyc[:, ncol], sizes)
    dw_ref = oracle.gmm_dw(xd, dyd, sizes)
    dwh = _f64(dw)[:, kcol][:, :, ncol]
    assert rel_fro(dwh, dw_ref) <= FP8_TOL
    for e in np.flatnonzero(sizes == 0):
        assert (dwh[e] == 0).all()


# --------------------------------------------------------------------------
# Sparse-M F8I4: 128 groups, 128 routed rows (83 experts touched), K=5120,
# N=8192.  The int4 codes (uniform in [-8, 7]) and their bf16 chunk scales
# are drawn directly, per touched expert; the other experts' weights are
# zero and never read.
# --------------------------------------------------------------------------

def test_f8i4_128_rows_full_size_sampled():
    E, total_M, K, N = 128, 128, 5120, 8192
    counts = wl.uniform_expert_rows(total_M, E, 5)
    X = wl.normal_bf16((total_M, K), 1.0, 5, wl.T_X)
    xq, sx = oracle.quant_rowwise(X)
    rng = np.random.default_rng(5)
    ncol = np.sort(rng.choice(N, 32, replace=False))
    w4 = torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.zeros((E, K // 128, N), dtype=torch.bfloat16, device="cuda")
    w4_s, sw_s = {}, {}
    for e in np.flatnonzero(counts):
        g = wl.rng(5, wl.T_W, int(e))
        p = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        s = wl.f32_to_bf16_bits(g.uniform(0.001, 0.01, size=(K // 128, N)).astype(np.float32))
        w4[e] = dev(p)
        sw[e] = bf16_dev(s)
        w4_s[e], sw_s[e] = p[ncol][None], s[:, ncol][None]
    y = mg.gmm_fwd_f8i4(dev(xq), dev(sx), w4, sw, dev(counts))
    torch.cuda.synchronize()
    offs = oracle.offsets(counts)
    xd = oracle.dequant_rowwise(xq, sx)
    ref = np.zeros((total_M, ncol.size))
    for e in np.flatnonzero(counts):
        r = slice(offs[e], offs[e + 1])
        ref[r] = oracle.gmm_fwd(xd[r], oracle.dequant_int4(w4_s[e], sw_s[e], 128), np.array([counts[e]], np.int32))
    assert rel_fro(_f64(y)[:, ncol], ref) <= FP8_TOL


# --------------------------------------------------------------------------
# Token-sorted fused FFN, Mixtral-8x7B expert shapes: E=8, top-2, hidden
# 4096, W1 [8, 4096, 28672], W2 [8, 14336, 4096]; sampled tokens, each one
# through the oracle's own permute -> GEMM -> SiLU*mul -> GEMM -> combine
# (a token's output depends on its own rows only).
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def mixtral_weights():
    """W1 [8, 4096, 28672] and W2 [8, 14336, 4096] bf16 N(0, 0.02), host bits
    and device copies, generated once for the module."""
    E, H, I = 8, 4096, 14336
    w1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.02, 0, wl.T_W1)
    w2 = wl.stacked_normal_bf16(E, (I, H), 0.02, 0, wl.T_W2)
    return w1, w2, bf16_dev(w1), bf16_dev(w2)


@pytest.mark.parametrize("T", [1, 64, 4096])   # block_m 16, 16 and 128 (the benchmarked launch)
def test_fused_ffn_mixtral_full_size_sampled(T, mixtral_weights):
    E, k, H, I = 8, 2, 4096, 14336
    w1, w2, w1d, w2d = mixtral_weights
    ids, w = wl.softmax_topk_routing(T, E, k, 0)
    x = wl.normal_bf16((T, H), 1.0, 0, wl.T_X)
    out, _ = mg.fused_moe(bf16_dev(x), w1d, w2d, dev(ids), dev(w))
    torch.cuda.synchronize()
    got = _f64(out)
    toks = np.unique(np.random.default_rng(1).choice(T, min(T, 4), replace=False))
    if T > 64:
        toks = np.unique(np.concatenate([toks, [0, T - 1]]))   # first and last token too
    for t in toks:
        used = np.unique(ids[t])
        remap = np.searchsorted(used, ids[t:t + 1])
        ref, _ = oracle.fused_moe(x[t:t + 1], np.ascontiguousarray(w1[used]), np.ascontiguousarray(w2[used]),
                                  remap.astype(np.int32), w[t:t + 1], 1)
        assert rel_fro(got[t:t + 1], ref) <= BF16_TOL


@pytest.mark.parametrize("T", [1, 64])
def test_fused_ffn_f8i4_mixtral_full_size_sampled(T, mixtral_weights):
    """The int4-weight fused FFN at the Mixtral shapes, stage by stage at
    the sorted rows of sampled tokens, against the oracle fed the same
    quantized operands: e4m3 codes and int4 weights bit-exact, the two F8I4
    GEMMs within the fp8 tolerance, SiLU*mul and the combine within bf16
    rounding."""
    E, k, H, I = 8, 2, 4096, 14336
    w1, w2, w1d, w2d = mixtral_weights
    ids, w = wl.softmax_topk_routing(T, E, k, 0)
    x = wl.normal_bf16((T, H), 1.0, 0, wl.T_X)
    w1_4, s1 = mg.quantize_int4_weights(w1d)
    w2_4, s2 = mg.quantize_int4_weights(w2d)
    out, st = mg.fused_moe_f8i4(bf16_dev(x), w1_4, s1, w2_4, s2, dev(ids), dev(w))
    torch.cuda.synchronize()
    inv = host(st["permute"]["inv"])
    xq, sx, aq, sa = host(st["xq"]), host(st["sx"]), host(st["aq"]), host(st["sa"])
    h1, act, y2 = bf16_host(st["h1"]), bf16_host(st["act"]), bf16_host(st["y2"])
    got = _f64(out)
    codes = {}   # expert -> GPU int4 codes and scales of W1 and W2, checked bit-exact once

    def expert_codes(e):
        if e not in codes:
            q1, c1 = oracle.quant_int4(oracle.bf16_to_f64(w1[e:e + 1]), 128)
            q2, c2 = oracle.quant_int4(oracle.bf16_to_f64(w2[e:e + 1]), 128)
            got_codes = (host(w1_4[e:e + 1]), bf16_host(s1[e:e + 1]), host(w2_4[e:e + 1]), bf16_host(s2[e:e + 1]))
            for a, b in zip(got_codes, (q1, c1, q2, c2)):
                np.testing.assert_array_equal(a, b)
            codes[e] = got_codes
        return codes[e]

    one = np.array([1], np.int32)
    toks = np.unique(np.random.default_rng(2).choice(T, min(T, 2), replace=False))
    for t in toks:
        y2_rows = []
        for j in range(k):
            e, p = int(ids[t, j]), int(inv[t * k + j])
            q1, c1, q2, c2 = expert_codes(e)
            rq, rs = oracle.quant_rowwise(x[t:t + 1])
            np.testing.assert_array_equal(xq[p:p + 1], rq)
            np.testing.assert_array_equal(sx[p:p + 1], rs)
            h_ref = oracle.gmm_fwd(oracle.dequant_rowwise(rq, rs), oracle.dequant_int4(q1, c1, 128), one)
            assert rel_fro(oracle.bf16_to_f64(h1[p:p + 1]), h_ref) <= FP8_TOL
            act_ref = oracle.silu_mul(oracle.bf16_to_f64(h1[p:p + 1]))
            assert rel_fro(oracle.bf16_to_f64(act[p:p + 1]), act_ref) <= 4e-3
            aq_ref, as_ref = oracle.quant_rowwise(act[p:p + 1])
            np.testing.assert_array_equal(aq[p:p + 1], aq_ref)
            np.testing.assert_array_equal(sa[p:p + 1], as_ref)
            y_ref = oracle.gmm_fwd(oracle.dequant_rowwise(aq_ref, as_ref), oracle.dequant_int4(q2, c2, 128), one)
            assert rel_fro(oracle.bf16_to_f64(y2[p:p + 1]), y_ref) <= FP8_TOL
            y2_rows.append(oracle.bf16_to_f64(y2[p:p + 1]))
        ref = sum(float(w[t, j]) * y2_rows[j] for j in range(k))
        assert rel_fro(got[t:t + 1], ref) <= BF16_TOL


@pytest.mark.parametrize("T", [1, 64, 4096])   # block_m 16, 16 and 128
def test_fused_ffn_fp8_mixtral_full_size_sampled(T, mixtral_weights):
    """The fp8-weight fused FFN at the Mixtral shapes, stage by stage at the
    sorted rows of sampled tokens, against the oracle fed the same quantized
    operands: weight codes, per-(expert, column) scales and activation codes
    bit-exact, the two fp8 GEMMs within the fp8 tolerance, SiLU*mul and the
    combine within bf16 rounding."""
    E, k, H, I = 8, 2, 4096, 14336
    w1, w2, w1d, w2d = mixtral_weights
    ids, w = wl.softmax_topk_routing(T, E, k, 0)
    x = wl.normal_bf16((T, H), 1.0, 0, wl.T_X)
    w1q, s1 = mg.quantize_fp8_expert_weights(w1d)
    w2q, s2 = mg.quantize_fp8_expert_weights(w2d)
    out, st = mg.fused_moe_fp8(bf16_dev(x), w1q, s1, w2q, s2, dev(ids), dev(w))
    torch.cuda.synchronize()
    inv = host(st["permute"]["inv"])
    xq, sx, aq, sa = host(st["xq"]), host(st["sx"]), host(st["aq"]), host(st["sa"])
    h1, act, y2 = bf16_host(st["h1"]), bf16_host(st["act"]), bf16_host(st["y2"])
    got = _f64(out)
    one = np.array([1], np.int32)
    deq = {}   # expert -> dequantized W1 and W2 of the GPU codes, checked bit-exact once

    def expert_weights(e):
        if e not in deq:
            q1, c1 = oracle.quant_colwise(w1[e], np.array([H], np.int32))
            q2, c2 = oracle.quant_colwise(w2[e], np.array([I], np.int32))
            np.testing.assert_array_equal(host(w1q[:, e * H:(e + 1) * H]), q1)
            np.testing.assert_array_equal(host(s1[e:e + 1]), c1)
            np.testing.assert_array_equal(host(w2q[:, e * I:(e + 1) * I]), q2)
            np.testing.assert_array_equal(host(s2[e:e + 1]), c2)
            deq[e] = (oracle.dequant_colwise(q1, c1, np.array([H], np.int32)).reshape(1, H, 2 * I),
                      oracle.dequant_colwise(q2, c2, np.array([I], np.int32)).reshape(1, I, H))
        return deq[e]

    toks = np.unique(np.random.default_rng(3).choice(T, min(T, 2), replace=False))
    for t in toks:
        y2_rows = []
        for j in range(k):
            e, p = int(ids[t, j]), int(inv[t * k + j])
            d1, d2 = expert_weights(e)
            rq, rs = oracle.quant_rowwise(x[t:t + 1])
            np.testing.assert_array_equal(xq[p:p + 1], rq)
            np.testing.assert_array_equal(sx[p:p + 1], rs)
            h_ref = oracle.gmm_fwd(oracle.dequant_rowwise(rq, rs), d1, one)
            assert rel_fro(oracle.bf16_to_f64(h1[p:p + 1]), h_ref) <= FP8_TOL
            act_ref = oracle.silu_mul(oracle.bf16_to_f64(h1[p:p + 1]))
            assert rel_fro(oracle.bf16_to_f64(act[p:p + 1]), act_ref) <= 4e-3
            aq_ref, as_ref = oracle.quant_rowwise(act[p:p + 1])
            np.testing.assert_array_equal(aq[p:p + 1], aq_ref)
            np.testing.assert_array_equal(sa[p:p + 1], as_ref)
            y_ref = oracle.gmm_fwd(oracle.dequant_rowwise(aq_ref, as_ref), d2, one)
            assert rel_fro(oracle.bf16_to_f64(y2[p:p + 1]), y_ref) <= FP8_TOL
            y2_rows.append(oracle.bf16_to_f64(y2[p:p + 1]))
        ref = sum(float(w[t, j]) * y2_rows[j] for j in range(k))
        assert rel_fro(got[t:t + 1], ref) <= BF16_TOL
