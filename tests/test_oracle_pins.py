"""Pins for the fp64 CPU oracle: each check ties it to something other than
itself -- numpy/torch library routines, closed forms, brute force, invariants
and the worked example printed on the pages.  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# offsets and work lists
# --------------------------------------------------------------------------

def test_offsets_are_prefix_sums():
    for seed in range(5):
        sizes = wl.random_group_sizes(17, 300, seed)
        offs = oracle.offsets(sizes)
        assert offs[0] == 0
        np.testing.assert_array_equal(offs[1:], np.cumsum(sizes.astype(np.int64)))


def _brute_fixed_m(sizes, bm):
    """Enumerate tiles row by row: a row r of group g lies in tile
    (g, (r - start_g) // bm); list distinct tiles in order of first row."""
    tiles = {}
    r = 0
    for g, s in enumerate(sizes):
        for i in range(s):
            key = (g, i // bm)
            if key not in tiles:
                tiles[key] = [g, r, 0, 0]
            tiles[key][2] += 1
            r += 1
    return np.array(list(tiles.values()), np.int32).reshape(-1, 4)


def test_worklist_tiny_config_bm16():
    n, ent = oracle.worklist_fixed_m(np.array([0, 20, 9, 8]), 16)
    assert n == 4
    np.testing.assert_array_equal(ent[:, :3], [[1, 0, 16], [1, 16, 4], [2, 20, 9], [3, 29, 8]])


@pytest.mark.parametrize("bm", [1, 16, 32, 64, 128])
def test_worklist_fixed_m_brute_force(bm):
    for seed in range(6):
        E = [1, 3, 8, 40, 128, 5][seed]
        sizes = wl.random_group_sizes(E, [0, 1, 77, 500, 1, 1000][seed], seed)
        n, ent = oracle.worklist_fixed_m(sizes, bm)
        ref = _brute_fixed_m(sizes, bm)
        assert n == len(ref)
        np.testing.assert_array_equal(ent, ref)
        total = int(sizes.sum())
        assert n <= total // bm + min(total, E)   # min(total_M, groups) bound
        assert all(sizes[e[0]] > 0 for e in ent)


def test_worklist_dynamic_k_is_stable_descending():
    for seed in range(5):
        sizes = wl.random_group_sizes(33, 400, seed, zero_frac=0.4)
        sizes[3] = sizes[7] = sizes[9] = 11  # force ties
        ent = oracle.worklist_dynamic_k(sizes)
        order = sorted(range(33), key=lambda g: -int(sizes[g]))   # python sort is stable
        np.testing.assert_array_equal(ent[:, 0], order)
        offs = np.concatenate([[0], np.cumsum(sizes)])
        np.testing.assert_array_equal(ent[:, 1], offs[order])
        np.testing.assert_array_equal(ent[:, 2], sizes[order])


# --------------------------------------------------------------------------
# grouped GEMMs
# --------------------------------------------------------------------------

def _block_diag_rows(A, sizes):
    """Arow[r, g(r)*C + c] = A[r, c]; zero elsewhere."""
    M, C = A.shape
    E = len(sizes)
    out = np.zeros((M, E * C))
    r = 0
    for g, s in enumerate(sizes):
        out[r:r + s, g * C:(g + 1) * C] = A[r:r + s]
        r += s
    return out


def _small_problem(seed, E=5, M=29, K=7, N=11):
    g = np.random.default_rng(seed)
    sizes = wl.random_group_sizes(E, M, seed, zero_frac=0.3)
    X = g.standard_normal((M, K))
    W = g.standard_normal((E, K, N))
    dY = g.standard_normal((M, N))
    return sizes, X, W, dY


@pytest.mark.parametrize("seed", range(4))
def test_gmm_fwd_equals_block_diagonal_matmul(seed):
    sizes, X, W, _ = _small_problem(seed)
    Y = oracle.gmm_fwd(X, W, sizes)
    E, K, N = W.shape
    ref = _block_diag_rows(X, sizes) @ W.reshape(E * K, N)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_gmm_dx_equals_block_diagonal_matmul(seed):
    sizes, _, W, dY = _small_problem(seed)
    dX = oracle.gmm_dx(dY, W, sizes)
    E, K, N = W.shape
    Wt = np.transpose(W, (0, 2, 1)).reshape(E * N, K)
    ref = _block_diag_rows(dY, sizes) @ Wt
    np.testing.assert_allclose(dX, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_gmm_dw_equals_block_diagonal_matmul(seed):
    sizes, X, _, dY = _small_problem(seed)
    dW = oracle.gmm_dw(X, dY, sizes)
    E = len(sizes)
    K, N = X.shape[1], dY.shape[1]
    ref = (_block_diag_rows(X, sizes).T @ dY).reshape(E, K, N)
    np.testing.assert_allclose(dW, ref, rtol=1e-12, atol=1e-12)
    for g in np.flatnonzero(sizes == 0):
        assert (dW[g] == 0).all()


def test_single_group_is_plain_matmul():
    g = np.random.default_rng(3)
    X, W, dY = g.standard_normal((13, 9)), g.standard_normal((1, 9, 6)), g.standard_normal((13, 6))
    s = np.array([13])
    np.testing.assert_allclose(oracle.gmm_fwd(X, W, s), X @ W[0], rtol=1e-12)
    np.testing.assert_allclose(oracle.gmm_dx(dY, W, s), dY @ W[0].T, rtol=1e-12)
    np.testing.assert_allclose(oracle.gmm_dw(X, dY, s)[0], X.T @ dY, rtol=1e-12)


def test_inserting_empty_groups_changes_nothing():
    sizes, X, W, dY = _small_problem(11, E=4)
    Y0 = oracle.gmm_fwd(X, W, sizes)
    dX0 = oracle.gmm_dx(dY, W, sizes)
    dW0 = oracle.gmm_dw(X, dY, sizes)
    g = np.random.default_rng(0)
    for pos in [0, 2, 4]:
        s2 = np.insert(sizes, pos, 0)
        W2 = np.insert(W, pos, g.standard_normal(W.shape[1:]) * 1e6, axis=0)   # garbage slice
        np.testing.assert_array_equal(oracle.gmm_fwd(X, W2, s2), Y0)
        np.testing.assert_array_equal(oracle.gmm_dx(dY, W2, s2), dX0)
        dW2 = oracle.gmm_dw(X, dY, s2)
        assert (dW2[pos] == 0).all()
        np.testing.assert_array_equal(np.delete(dW2, pos, axis=0), dW0)


def test_grad_of_sum_closed_forms():
    """dY = ones (gradient of out.sum()): dX[r,k] = sum_n W[g(r),k,n] and
    dW[g,k,n] = sum_{r in g} X[r,k] for every n."""
    w = wl.balanced_bf16(seed=0, E=4, M=64, K=32, N=24)
    X = oracle.bf16_to_f64(w["X"])
    W = oracle.bf16_to_f64(w["W"])
    dY = oracle.bf16_to_f64(w["dY"])
    assert (dY == 1.0).all()
    sizes = w["sizes"]
    dX = oracle.gmm_dx(dY, W, sizes)
    dW = oracle.gmm_dw(X, dY, sizes)
    rows = np.repeat(np.arange(4), sizes)
    np.testing.assert_allclose(dX, W.sum(axis=2)[rows], rtol=1e-13)
    for g in range(4):
        colsum = X[rows == g].sum(axis=0)
        np.testing.assert_allclose(dW[g], np.repeat(colsum[:, None], 24, axis=1), rtol=1e-13)


def test_transpose_identities():
    """dX(dY, W) = forward(dY, W^T); dW of one group = forward(X_g^T, dY_g)."""
    sizes, X, W, dY = _small_problem(5)
    Wt = np.ascontiguousarray(np.transpose(W, (0, 2, 1)))
    np.testing.assert_allclose(oracle.gmm_dx(dY, W, sizes), oracle.gmm_fwd(dY, Wt, sizes), rtol=1e-12)
    dW = oracle.gmm_dw(X, dY, sizes)
    offs = oracle.offsets(sizes)
    for g in range(len(sizes)):
        if sizes[g] == 0:
            continue
        Xg = X[offs[g]:offs[g + 1]]
        dYg = dY[offs[g]:offs[g + 1]]
        ref = oracle.gmm_fwd(Xg.T.copy(), dYg[None], np.array([Xg.shape[1]]))
        np.testing.assert_allclose(dW[g], ref, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(vals[finite], ref[finite])


def test_bf16_encode_matches_torch_on_fp32_inputs():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.5]]).astype(np.float32)
    ours = oracle.f64_to_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(ours, wl.f32_to_bf16_bits(x))


def _bf16_nearest_exact(x):
    """Reference double -> bf16 bits by exact rational arithmetic: the finite
    bf16 value nearest to x, a tie going to the pattern with an even last
    bit.  Positive bf16 patterns are ordered like their values, so the two
    neighbours of |x| come from a binary search over patterns compared as
    exact fractions; no float rounding enters anywhere.  Defined for |x| up
    to the largest finite bf16 value."""
    import struct
    from fractions import Fraction

    def val(p):   # exact value of a positive finite bf16 pattern
        return Fraction(struct.unpack("<f", struct.pack("<I", p << 16))[0])

    a = Fraction(abs(x))
    lo, hi = 0, 0x7F7F            # val(lo) <= a < val(hi) is kept below
    if a > val(hi):
        raise ValueError("beyond the largest finite bf16 value")
    if a == val(hi):
        p = hi
    else:
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if val(mid) <= a:
                lo = mid
            else:
                hi = mid
        dlo, dhi = a - val(lo), val(hi) - a
        p = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
    return p | (0x8000 if np.signbit(x) else 0)


def _bf16_pin_inputs():
    """Doubles that are not fp32 values: random magnitudes over the whole
    normal range, near-ties just above and below bf16 midpoints (off by far
    less than an fp32 ulp, so rounding through fp32 first lands exactly on
    the midpoint), subnormals, and the normal/subnormal boundary."""
    g = np.random.default_rng(7)
    xs = list(g.standard_normal(3000) * np.exp2(g.uniform(-125, 127, 3000)))
    base = wl.bf16_bits_to_f32(g.integers(0x0080, 0x7F7F, 600).astype(np.uint16)).astype(np.float64)
    mids = base + np.exp2(np.floor(np.log2(base)) - 8)        # halfway to the next bf16 value
    for eps in (2.0 ** -40, 2.0 ** -30, 2.0 ** -26):
        xs += list(mids * (1 + eps)) + list(mids * (1 - eps))
    sub = np.exp2(-133.0)                                      # bf16 subnormal spacing
    ks = g.integers(0, 128, 400).astype(np.float64)
    xs += list((ks + 0.5) * sub) + list((ks + 0.5) * sub * (1 + 2.0 ** -35)) + list((ks + 0.5) * sub * (1 - 2.0 ** -35))
    xs += list(g.uniform(0, 128, 400) * sub) + list(g.uniform(0, 1, 100) * sub * 2.0 ** -5)
    tiny_normal = np.exp2(-126.0)
    xs += [tiny_normal, tiny_normal * (1 - 2.0 ** -9), tiny_normal * (1 - 2.0 ** -9) * (1 + 2.0 ** -40),
           tiny_normal * (1 - 2.0 ** -9) * (1 - 2.0 ** -40), tiny_normal * (1 + 2.0 ** -9), 127.5 * sub,
           0.5 * sub, 0.5 * sub * (1 + 2.0 ** -40), 0.5 * sub * (1 - 2.0 ** -40), 2.0 ** -1000]
    x = np.array(xs, np.float64)
    signs = np.where(g.integers(0, 2, x.size) == 1, -1.0, 1.0)
    return x * signs


def test_bf16_encode_of_doubles_is_exact_rounding():
    """The oracle's double -> bf16 (used on fp64 GEMM results and on the int4
    scales) equals the exact nearest-even rounding of the double itself."""
    x = _bf16_pin_inputs()
    ref = np.array([_bf16_nearest_exact(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16(x), ref)


def test_bf16_pin_rejects_rounding_through_fp32():
    """The inputs above separate correct rounding from double rounding
    through fp32 (the mistake the pin is there to catch): rounding each
    double to fp32 first and then to bf16 disagrees with the exact result on
    many of them."""
    x = _bf16_pin_inputs()
    ref = np.array([_bf16_nearest_exact(float(v)) for v in x], np.uint16)
    via_f32 = wl.f32_to_bf16_bits(x.astype(np.float32))
    assert int((via_f32 != ref).sum()) >= 200


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(vals[nan]).all()
    np.testing.assert_array_equal(vals[~nan], ref[~nan])
    assert np.nanmax(vals) == 448.0 and oracle.e4m3_to_f64(np.array([1], np.uint8))[0] == 2.0 ** -9


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_to_f64(codes).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_encode_special_values():
    x = np.array([464, 17, 19, 2.0 ** -10, 1.5 * 2.0 ** -9, -1e-9, 0.0, -0.0, 448, -448], np.float32)
    q = oracle.e4m3_encode(np.clip(x, -448, 448))
    dec = oracle.e4m3_to_f64(q)
    assert list(dec[:5]) == [448, 16, 20, 0, 2 * 2.0 ** -9]
    assert q[5] == 0x80 and q[6] == 0x00 and q[7] == 0x80
    assert q[8] == 0x7E and q[9] == 0xFE


def test_e4m3_encode_exhaustive_bf16_times_pow2_vs_torch():
    """Every finite bf16 pattern times a set of power-of-two scales, clamped to
    +-448, encoded and compared with torch's CPU fp32 -> e4m3fn cast (round to
    nearest even with subnormals; it agrees with a saturating cast once the
    input is clamped)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = wl.bf16_bits_to_f32(bits)
    x = x[np.isfinite(x)]
    for t in [-130, -20, -9, -3, 0, 5, 40]:
        v = np.clip(x.astype(np.float64) * 2.0 ** t, -448, 448).astype(np.float32)
        ours = oracle.e4m3_encode(v)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(ours, ref)


# --------------------------------------------------------------------------
# FP8 quantizers
# --------------------------------------------------------------------------

def _torch_rowwise(x_bits):
    """The unfused three-step definition (amax -> pow2 scale -> saturated
    cast) composed from torch library operations."""
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float()
    amax = x.abs().amax(dim=1).double()
    s = (448.0 / torch.clamp(amax, min=1e-12)).float()
    s = torch.exp2(torch.floor(torch.log2(s)))
    q = torch.clamp(x * s[:, None], -448, 448).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), s.numpy()


def test_rowwise_matches_torch_composite():
    x = wl.normal_bf16((64, 300), 1.0, 0, wl.T_X)
    x[3] = 0                                                # all-zero row
    x[5] = wl.f32_to_bf16_bits(np.full(300, 1e-30, np.float32))
    q, s = oracle.quant_rowwise(x)
    qr, sr = _torch_rowwise(x)
    np.testing.assert_array_equal(q, qr)
    np.testing.assert_array_equal(s, sr)


def test_rowwise_invariants():
    x = wl.normal_bf16((16, 257), 1.0, 1, wl.T_X)
    q, s = oracle.quant_rowwise(x)
    assert np.all(np.log2(s) == np.floor(np.log2(s)))           # powers of two
    for t in [-7, 3, 12]:
        xs = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(x) * np.float32(2.0 ** t))
        q2, s2 = oracle.quant_rowwise(xs)
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, s * np.float32(2.0 ** -t))
    z = np.zeros((2, 8), np.uint16)
    qz, sz = oracle.quant_rowwise(z)
    assert (qz == 0).all() and (sz == np.float32(2.0 ** 48)).all()
    for j in [-3, 0, 5]:
        row = np.linspace(-1, 1, 64).astype(np.float32) * np.float32(448 * 2.0 ** -j)
        qj, sj = oracle.quant_rowwise(wl.f32_to_bf16_bits(row)[None])
        assert sj[0] == 2.0 ** j and (qj & 0x7F).max() == 0x7E
        assert qj[0, 0] == 0xFE and qj[0, -1] == 0x7E
    # dequantization error: within half an e4m3 step of the scaled value
    deq = oracle.dequant_rowwise(q, s)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    assert np.all(np.abs(deq - xf) <= np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 / s[:, None]))


def test_colwise_single_group_is_rowwise_of_transpose():
    x = wl.normal_bf16((96, 40), 1.0, 2, wl.T_X)
    q, s = oracle.quant_colwise(x, np.array([96]))
    qr, sr = oracle.quant_rowwise(np.ascontiguousarray(x.T))
    np.testing.assert_array_equal(q, qr)
    np.testing.assert_array_equal(s[0], sr)


def test_colwise_groups_are_rowwise_of_each_transposed_slice():
    x = wl.normal_bf16((160, 24), 1.0, 3, wl.T_X)
    sizes = np.array([16, 0, 48, 32, 0, 64], np.int32)
    q, s = oracle.quant_colwise(x, sizes)
    offs = oracle.offsets(sizes)
    for g in range(len(sizes)):
        a, b = offs[g], offs[g + 1]
        if a == b:
            assert (s[g] == np.float32(2.0 ** 48)).all()
            continue
        qr, sr = _torch_rowwise(np.ascontiguousarray(x[a:b].T))
        np.testing.assert_array_equal(q[:, a:b], qr)
        np.testing.assert_array_equal(s[g], sr)
    deq = oracle.dequant_colwise(q, s, sizes)
    np.testing.assert_allclose(deq, wl.bf16_bits_to_f32(x), rtol=2 ** -4, atol=2 ** -9)


# --------------------------------------------------------------------------
# int4 weights
# --------------------------------------------------------------------------

def test_int4_recovers_exact_grid_weights():
    g = np.random.default_rng(4)
    E, K, N, grp = 2, 256, 8, 128
    q = g.integers(-7, 8, size=(E, K, N))
    q[:, 0, :] = 7          # each (e, chunk, n) reaches |q| = 7
    q[:, 128, :] = -7
    s_bits = wl.f32_to_bf16_bits(np.abs(g.standard_normal((E, K // grp, N))).astype(np.float32) * 0.01 + 1e-3)
    s = wl.bf16_bits_to_f32(s_bits).astype(np.float64)
    W = q * np.repeat(s, grp, axis=1)
    packed, scales = oracle.quant_int4(W, grp)
    np.testing.assert_array_equal(scales, s_bits)
    lo = (packed & 0xF).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    nib = np.stack([lo, hi], axis=-1).reshape(E, N, K)
    nib = np.where(nib >= 8, nib - 16, nib)
    np.testing.assert_array_equal(nib, np.transpose(q, (0, 2, 1)))
    np.testing.assert_array_equal(oracle.dequant_int4(packed, scales, grp), W)


def test_int4_error_bound():
    W = oracle.bf16_to_f64(wl.normal_bf16((3, 384, 16), 0.02, 0, wl.T_W))
    packed, scales = oracle.quant_int4(W, 128)
    Wd = oracle.dequant_int4(packed, scales, 128)
    s = np.repeat(oracle.bf16_to_f64(scales), 128, axis=1)
    assert np.all(np.abs(W - Wd) <= s * 0.5 + 1e-15 + np.abs(W) * 2 ** -7)


# --------------------------------------------------------------------------
# permutation, activation, combine
# --------------------------------------------------------------------------

def test_moe_align_worked_example():
    with open(os.path.join(GOLDEN, "moe_align_example.json")) as f:
        ex = json.load(f)
    ids = np.array(ex["topk_ids_printed"], np.int32) - 1
    al = oracle.moe_align(ids, ex["num_experts"], ex["block_size"])
    n = ex["expected_num_tokens_post_padded"]
    assert al["num_tokens_post_padded"] == n
    np.testing.assert_array_equal(al["sorted_token_ids"][:n], ex["expected_sorted_token_ids"])
    assert (al["sorted_token_ids"][n:] == ids.size).all()
    np.testing.assert_array_equal(al["expert_ids"][:n // ex["block_size"]], ex["expected_expert_ids"])


@pytest.mark.parametrize("T,k,E,bm", [(1, 2, 8, 16), (37, 2, 8, 4), (50, 6, 64, 16), (9, 1, 3, 1)])
def test_moe_align_brute_force(T, k, E, bm):
    g = np.random.default_rng(T * 100 + E)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    al = oracle.moe_align(ids, E, bm)
    flat = ids.reshape(-1)
    seq = []
    blocks = []
    for e in range(E):
        members = [f for f in range(T * k) if flat[f] == e]
        if members:
            pad = -len(members) % bm
            seq += members + [T * k] * pad
            blocks += [e] * ((len(members) + pad) // bm)
    n = al["num_tokens_post_padded"]
    assert n == len(seq)
    np.testing.assert_array_equal(al["sorted_token_ids"][:n], seq)
    np.testing.assert_array_equal(al["expert_ids"][:len(blocks)], blocks)
    assert sorted(al["inv"].tolist()) == [i for i, f in enumerate(seq) if f < T * k]
    np.testing.assert_array_equal(al["sorted_token_ids"][al["inv"]], np.arange(T * k))


def test_silu_mul_matches_scipy():
    from scipy.special import expit
    g = np.random.default_rng(7)
    h = g.standard_normal((5, 20)) * 4
    act = oracle.silu_mul(h)
    ref = h[:, :10] * expit(h[:, :10]) * h[:, 10:]
    np.testing.assert_allclose(act, ref, rtol=1e-14, atol=1e-300)


def test_permute_unpermute_identity_returns_input():
    T, k, E, H = 23, 2, 8, 16
    g = np.random.default_rng(2)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = wl.normal_bf16((T, H), 1.0, 0, wl.T_X)
    al = oracle.moe_align(ids, E, 4)
    xs = oracle.gather_rows(x, k, al["sorted_token_ids"])
    out = oracle.unpermute(oracle.bf16_to_f64(xs), al["inv"], np.full((T, k), 0.5, np.float32), T, k)
    np.testing.assert_array_equal(out, oracle.bf16_to_f64(x))


def test_fused_moe_single_expert_is_dense_ffn():
    T, H, I = 19, 32, 24
    x = wl.normal_bf16((T, H), 1.0, 0, wl.T_X)
    w1 = wl.normal_bf16((1, H, 2 * I), 0.2, 0, wl.T_W1)
    w2 = wl.normal_bf16((1, I, H), 0.2, 0, wl.T_W2)
    ids = np.zeros((T, 1), np.int32)
    out, _ = oracle.fused_moe(x, w1, w2, ids, np.ones((T, 1), np.float32), block_m=8)
    # dense gated FFN in torch fp64, rounding to bf16 at the same points
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double()
    X, W1, W2 = tb(x), tb(w1)[0], tb(w2)[0]
    h = (X @ W1).to(torch.bfloat16).double()
    a = (torch.nn.functional.silu(h[:, :I]) * h[:, I:]).to(torch.bfloat16).double()
    y = (a @ W2).to(torch.bfloat16).double()
    np.testing.assert_allclose(out, y.numpy(), rtol=2 ** -7, atol=1e-6)


# --------------------------------------------------------------------------
# Router: softmax -> top-k -> optional renormalization (applied-ai issue
# "Column-major fused MoE", fused_moe)
# --------------------------------------------------------------------------

def test_route_topk_known_probabilities():
    """Logits ln 1, ln 2, ln 5 give probabilities 1/8, 2/8, 5/8 exactly (up to
    the fp32 rounding of the logarithms); top-2 renormalized is 5/7, 2/7."""
    z = np.log(np.array([[1.0, 2.0, 5.0]])).astype(np.float32)
    ids, w = oracle.route_topk(z, 2)
    np.testing.assert_array_equal(ids, [[2, 1]])
    np.testing.assert_allclose(w, [[5 / 8, 2 / 8]], rtol=1e-6)
    ids, w = oracle.route_topk(z, 2, renormalize=True)
    np.testing.assert_allclose(w, [[5 / 7, 2 / 7]], rtol=1e-6)


def test_route_topk_two_experts_is_the_logistic():
    """With two experts the larger probability is the logistic function of
    the logit difference."""
    rng = np.random.default_rng(0)
    z = rng.standard_normal((50, 2)).astype(np.float32)
    ids, w = oracle.route_topk(z, 1)
    d = np.abs(z[:, 0].astype(np.float64) - z[:, 1].astype(np.float64))
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(-d)), rtol=1e-12)
    np.testing.assert_array_equal(ids[:, 0], np.where(z[:, 1] > z[:, 0], 1, 0))


def test_route_topk_matches_a_full_sort_and_is_shift_invariant():
    """ids equal a full lexicographic sort by (-logit, index) on small random
    inputs with repeated values; adding a constant to a token's logits
    changes nothing; k = E with renormalization sums to 1 and puts all
    experts in descending order."""
    rng = np.random.default_rng(1)
    z = rng.integers(-3, 4, size=(40, 9)).astype(np.float32)   # many ties
    for k in (1, 3, 9):
        ids, w = oracle.route_topk(z, k)
        for t in range(z.shape[0]):
            order = sorted(range(9), key=lambda e: (-z[t, e], e))[:k]
            assert list(ids[t]) == order
        assert np.all(np.diff(w, axis=1) <= 0)
        ids2, w2 = oracle.route_topk(z + np.float32(2.0), k)
        np.testing.assert_array_equal(ids2, ids)
        np.testing.assert_allclose(w2, w, rtol=1e-12)
    ids, w = oracle.route_topk(z, 9, renormalize=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)
    assert all(sorted(r) == list(range(9)) for r in ids)


def test_route_topk_equal_logits():
    """All logits equal: experts 0..k-1 in order, each with probability 1/E."""
    ids, w = oracle.route_topk(np.zeros((3, 6), np.float32), 4)
    np.testing.assert_array_equal(ids, np.tile(np.arange(4), (3, 1)))
    np.testing.assert_allclose(w, 1 / 6, rtol=1e-15)
