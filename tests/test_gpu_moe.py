"""GPU parity: token permutation (align + gather), SiLU-and-mul, the top-k
weighted combine and the token-sorted fused MoE path."""
import json
import os

import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import (BF16_TOL, CHAIN_ELEM, EW_ELEM, FP8_TOL, GEMM_BF16, GEMM_FP8, SWIGLU_ELEM, assert_close, bf16_dev,
                      bf16_host, dev, fwd_norms, gpu, host, require_gpu)

pytestmark = gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check_permute(ids, E, bm, x=None):
    p = mg.moe_permute(dev(ids), E, bm, x=None if x is None else bf16_dev(x))
    torch.cuda.synchronize()
    ref = oracle.moe_align(ids, E, bm)
    n = ref["num_tokens_post_padded"]
    assert int(host(p["num_tokens_post_padded"])[0]) == n
    np.testing.assert_array_equal(host(p["sorted_token_ids"]), ref["sorted_token_ids"])
    np.testing.assert_array_equal(host(p["expert_ids"])[: n // bm], ref["expert_ids"][: n // bm])
    np.testing.assert_array_equal(host(p["inv"]), ref["inv"])
    np.testing.assert_array_equal(host(p["padded_sizes"]), ref["padded_sizes"])
    if x is not None:
        np.testing.assert_array_equal(bf16_host(p["x_sorted"]),
                                      oracle.gather_rows(x, ids.shape[1], ref["sorted_token_ids"]))
    return p, ref


def test_permute_worked_example():
    with open(os.path.join(GOLDEN, "moe_align_example.json")) as f:
        ex = json.load(f)
    ids = np.array(ex["topk_ids_printed"], np.int32) - 1
    p, _ = _check_permute(ids, ex["num_experts"], ex["block_size"])
    np.testing.assert_array_equal(host(p["sorted_token_ids"])[:16], ex["expected_sorted_token_ids"])


@pytest.mark.parametrize("T,k,E,bm,seed", [
    (1, 2, 8, 16, 0), (64, 2, 8, 16, 1), (4096, 2, 8, 128, 2), (37, 6, 64, 16, 3), (16384, 6, 64, 128, 4),
    (5, 1, 3, 1, 5), (3000, 4, 1024, 32, 6),
    # both sides of the one-workgroup path's limit of 1024 pairs
    (512, 2, 8, 16, 7), (1025, 1, 8, 16, 8), (171, 6, 1024, 8, 9), (128, 8, 1024, 1, 10), (1024, 1, 1, 64, 11),
])
def test_permute_random(T, k, E, bm, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = wl.normal_bf16((T, 64), 1.0, seed, wl.T_X) if T <= 4096 else None
    _check_permute(ids, E, bm, x)


def test_permute_skewed_routing():
    ids = wl.zipf_topk_routing(2000, 64, 6, 1.1, 0)
    _check_permute(ids, 64, 64)
    # one-workgroup path: many pairs of one expert spread over all waves
    ids = wl.zipf_topk_routing(170, 64, 6, 1.1, 1)
    _check_permute(ids, 64, 16)


def test_silu_mul_and_unpermute():
    rows, I = 300, 136
    h = wl.normal_bf16((rows, 2 * I), 2.0, 0, wl.T_X)
    act = mg.silu_mul(bf16_dev(h))
    torch.cuda.synchronize()
    ref = oracle.silu_mul(oracle.bf16_to_f64(h))
    got = oracle.bf16_to_f64(bf16_host(act))
    assert_close(got, ref, 4e-3, EW_ELEM)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -7 + 1e-30)

    T, k, E, H = 123, 2, 8, 64
    rng = np.random.default_rng(1)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    al = oracle.moe_align(ids, E, 16)
    y = wl.normal_bf16((al["sorted_token_ids"].size, H), 1.0, 2, wl.T_DY)
    out = mg.moe_unpermute(bf16_dev(y), dev(al["inv"]), dev(w), T, k)
    torch.cuda.synchronize()
    ref = oracle.unpermute(oracle.bf16_to_f64(y), al["inv"], w, T, k)
    got = oracle.bf16_to_f64(bf16_host(out))
    assert_close(got, ref, BF16_TOL, EW_ELEM)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)


def test_unpermute_past_one_grid_row_per_token():
    """More tokens than the 65535 workgroup rows of one launch: the rows
    stride over the tokens."""
    T, k, H = 70001, 1, 16
    rng = np.random.default_rng(3)
    inv = rng.permutation(T).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y = wl.normal_bf16((T, H), 1.0, 3, wl.T_DY)
    out = mg.moe_unpermute(bf16_dev(y), dev(inv), dev(w), T, k)
    torch.cuda.synchronize()
    ref = oracle.unpermute(oracle.bf16_to_f64(y), inv, w, T, k)
    got = oracle.bf16_to_f64(bf16_host(out))
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)


@pytest.mark.parametrize("T,bm", [(1, 16), (64, 16), (200, 32)])
def test_fused_moe_small_matches_oracle(T, bm):
    E, k, H, I = 8, 2, 256, 128
    ids, w = wl.softmax_topk_routing(T, E, k, 0)
    x = wl.normal_bf16((T, H), 1.0, 0, wl.T_X)
    w1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, 0, wl.T_W1)
    w2 = wl.stacked_normal_bf16(E, (I, H), 0.05, 0, wl.T_W2)
    out, _ = mg.fused_moe(bf16_dev(x), bf16_dev(w1), bf16_dev(w2), dev(ids), dev(w), block_m=bm)
    # the same weights in the (E, N, K) layout give the same bits
    t = lambda a: bf16_dev(np.ascontiguousarray(np.transpose(a, (0, 2, 1))))
    out_t, _ = mg.fused_moe(bf16_dev(x), t(w1), t(w2), dev(ids), dev(w), block_m=bm, trans_b=True)
    torch.cuda.synchronize()
    ref, _ = oracle.fused_moe(x, w1, w2, ids, w, bm)
    assert_close(oracle.bf16_to_f64(bf16_host(out)), ref, BF16_TOL, CHAIN_ELEM)
    assert torch.equal(out, out_t)


@pytest.mark.parametrize("T,k,E,bm,K,N,trans_b", [
    (1, 2, 8, 16, 256, 128, False),       # one token: two rows, the rest of each block is padding
    (64, 2, 8, 16, 136, 264, True),
    (300, 6, 64, 32, 200, 392, False),    # many experts, some empty
    (1500, 2, 8, 128, 1024, 512, False),  # several row tiles per expert
])
def test_gmm_fwd_gather_equals_the_sorted_copy(T, k, E, bm, K, N, trans_b):
    """GEMM over token rows looked up through sorted_token_ids // top_k is
    bit-identical to the GEMM over the gathered copy, and matches the oracle
    on the gathered rows (padding rows are zero rows)."""
    rng = np.random.default_rng(T + K)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = wl.normal_bf16((T, K), 1.0, 7, wl.T_X)
    W = wl.stacked_normal_bf16(E, (N, K) if trans_b else (K, N), 0.5, 7, wl.T_W)
    p = mg.moe_permute(dev(ids), E, bm, x=bf16_dev(x))
    sizes = p["padded_sizes"]
    w = bf16_dev(W)
    y_copy = mg.gmm_fwd(p["x_sorted"], w, sizes, trans_b=trans_b)
    y_gath = mg.gmm_fwd_gather(bf16_dev(x), p["sorted_token_ids"], k, w, sizes, trans_b=trans_b)
    torch.cuda.synchronize()
    n = int(host(p["num_tokens_post_padded"])[0])
    np.testing.assert_array_equal(bf16_host(y_gath)[:n], bf16_host(y_copy)[:n])
    al = oracle.moe_align(ids, E, bm)
    xs = oracle.gather_rows(x, k, al["sorted_token_ids"])[:n]
    A, Wf = oracle.bf16_to_f64(xs), oracle.bf16_to_f64(W)
    ref = oracle.gmm_fwd_bf16(xs, W, al["padded_sizes"], trans_b=trans_b)
    assert_close(oracle.bf16_to_f64(bf16_host(y_gath)[:n]), ref, BF16_TOL, GEMM_BF16, "Y",
                 fwd_norms(A, Wf, al["padded_sizes"], trans_b))


@pytest.mark.parametrize("case", [
    dict(E=3, M=300, K=136, I=136, gather=None),            # two column tiles, the second 8 wide
    dict(E=5, M=700, K=64, I=264, gather=None),
    dict(E=8, T=64, k=2, bm=16, K=256, I=128, gather=True),
    dict(E=64, T=300, k=6, bm=32, K=200, I=392, gather=True),
    dict(E=8, T=1500, k=2, bm=128, K=512, I=1024, gather=True),
])
@pytest.mark.parametrize("trans_b", [False, True])
def test_gmm_fwd_silu_mul_equals_the_unfused_steps(case, trans_b):
    """The GEMM with SiLU-and-mul in its epilogue is bit-identical to the GEMM
    into h followed by the silu_mul kernel, with and without the gathered A
    rows (at these shapes every tile is whole, so both kernels sum each
    element in the same order; where the schedule splits tiles along K the
    split points differ between the two and only the oracle bars hold), and
    matches the oracle's silu_mul of the oracle GEMM rounded to bf16 (both
    halves are rounded to bf16 before SiLU*mul, as the fused path stores
    them).  With trans_b the weights are [E, 2I, K]: gate rows, then up
    rows."""
    E, K, I = case["E"], case["K"], case["I"]
    W1 = wl.stacked_normal_bf16(E, (K, 2 * I), 0.3, 11, wl.T_W1)
    w1 = bf16_dev(np.ascontiguousarray(np.transpose(W1, (0, 2, 1))) if trans_b else W1)
    if case["gather"]:
        T, k, bm = case["T"], case["k"], case["bm"]
        rng = np.random.default_rng(T)
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        x = wl.normal_bf16((T, K), 1.0, 11, wl.T_X)
        p = mg.moe_permute(dev(ids), E, bm)
        sizes, sids = p["padded_sizes"], p["sorted_token_ids"]
        h = mg.gmm_fwd_gather(bf16_dev(x), sids, k, w1, sizes, trans_b=trans_b)
        act = mg.gmm_fwd_silu_mul(bf16_dev(x), w1, sizes, sorted_token_ids=sids, top_k=k, trans_b=trans_b)
        n = int(host(p["num_tokens_post_padded"])[0])
        al = oracle.moe_align(ids, E, bm)
        xa = oracle.gather_rows(x, k, al["sorted_token_ids"])[:n]
        osz = al["padded_sizes"]
    else:
        M = case["M"]
        osz = wl.random_group_sizes(E, M, 11, zero_frac=0.25)
        x = wl.normal_bf16((M, K), 1.0, 11, wl.T_X)
        sizes = dev(osz)
        h = mg.gmm_fwd(bf16_dev(x), w1, sizes, trans_b=trans_b)
        act = mg.gmm_fwd_silu_mul(bf16_dev(x), w1, sizes, trans_b=trans_b)
        n, xa = M, x
    ref_act = mg.silu_mul(h[:n].contiguous())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(act)[:n], bf16_host(ref_act))
    ref = oracle.silu_mul(oracle.bf16_to_f64(oracle.f64_to_bf16(oracle.gmm_fwd_bf16(xa, W1, osz))))
    assert_close(oracle.bf16_to_f64(bf16_host(act)[:n]), ref, BF16_TOL, SWIGLU_ELEM)


@pytest.mark.parametrize("T,E,k,renorm", [
    (1, 8, 2, False), (4096, 8, 2, False), (16384, 64, 6, True), (300, 1024, 8, True),
    (77, 65, 3, False), (50, 130, 64, True), (10, 3, 3, True),
])
def test_route_topk_matches_oracle(T, E, k, renorm):
    """Expert ids bit-exact (the choice is made on the fp32 logits on both
    sides, ties to the lower index: a quarter of the logits are rounded to
    integers so ties occur); probabilities within fp32 rounding of the fp64
    softmax."""
    rng = np.random.default_rng(T + E)
    z = rng.standard_normal((T, E)).astype(np.float32)
    z[:, : max(E // 4, 1)] = np.round(z[:, : max(E // 4, 1)])
    ids, w = mg.route_topk(dev(z), k, renormalize=renorm)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route_topk(z, k, renormalize=renorm)
    np.testing.assert_array_equal(host(ids), ref_ids)
    np.testing.assert_allclose(host(w), ref_w, rtol=1e-5, atol=1e-30)


def test_router_feeds_the_fused_path():
    """Router logits -> device top-k -> align -> fused FFN, against the oracle
    taking the same steps."""
    T, E, k, H, I = 96, 8, 2, 256, 128
    rng = np.random.default_rng(5)
    z = rng.standard_normal((T, E)).astype(np.float32)
    x = wl.normal_bf16((T, H), 1.0, 5, wl.T_X)
    w1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, 5, wl.T_W1)
    w2 = wl.stacked_normal_bf16(E, (I, H), 0.05, 5, wl.T_W2)
    ids, w = mg.route_topk(dev(z), k, renormalize=True)
    out, _ = mg.fused_moe(bf16_dev(x), bf16_dev(w1), bf16_dev(w2), ids, w, block_m=16)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route_topk(z, k, renormalize=True)
    np.testing.assert_array_equal(host(ids), ref_ids)
    ref, _ = oracle.fused_moe(x, w1, w2, ref_ids, ref_w.astype(np.float32), 16)
    assert_close(oracle.bf16_to_f64(bf16_host(out)), ref, BF16_TOL, CHAIN_ELEM)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_fused_moe_f8i4_stages_match_the_oracle(T):
    """The int4-weight fused FFN, stage by stage, against the oracle fed the
    same quantized operands: the int4 weights and the e4m3 codes of the
    gathered rows and of the activations are bit-exact; each F8I4 GEMM is
    within the fp8 tolerance of the oracle's fp64 product of the dequantized
    operands; SiLU*mul and the combine within bf16 rounding."""
    E, k, H, I, bm = 8, 2, 256, 256, 16
    ids, w = wl.softmax_topk_routing(T, E, k, 3)
    x = wl.normal_bf16((T, H), 1.0, 3, wl.T_X)
    W1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, 3, wl.T_W1)
    W2 = wl.stacked_normal_bf16(E, (I, H), 0.05, 3, wl.T_W2)
    w1_4, s1 = mg.quantize_int4_weights(bf16_dev(W1))
    w2_4, s2 = mg.quantize_int4_weights(bf16_dev(W2))
    out, st = mg.fused_moe_f8i4(bf16_dev(x), w1_4, s1, w2_4, s2, dev(ids), dev(w), block_m=bm, keep_act=True)
    torch.cuda.synchronize()
    p1, q1 = oracle.quant_int4(oracle.bf16_to_f64(W1), 128)
    p2, q2 = oracle.quant_int4(oracle.bf16_to_f64(W2), 128)
    np.testing.assert_array_equal(host(w1_4), p1)
    np.testing.assert_array_equal(bf16_host(s1), q1)
    np.testing.assert_array_equal(host(w2_4), p2)
    np.testing.assert_array_equal(bf16_host(s2), q2)
    al = oracle.moe_align(ids, E, bm)
    n, sizes = al["num_tokens_post_padded"], al["padded_sizes"]
    xq, sx = oracle.quant_rowwise(oracle.gather_rows(x, k, al["sorted_token_ids"])[:n])
    np.testing.assert_array_equal(host(st["xq"])[:n], xq)
    np.testing.assert_array_equal(host(st["sx"])[:n], sx)
    A, W1d = oracle.dequant_rowwise(xq, sx), oracle.dequant_int4(p1, q1, 128)
    h1 = bf16_host(st["h1"])[:n]
    assert_close(oracle.bf16_to_f64(h1), oracle.gmm_fwd(A, W1d, sizes), FP8_TOL, GEMM_FP8, "h1",
                 fwd_norms(A, W1d, sizes))
    act_ref = oracle.silu_mul(oracle.bf16_to_f64(h1))
    act = bf16_host(st["act"])[:n]
    assert_close(oracle.bf16_to_f64(act), act_ref, 4e-3, EW_ELEM)
    aq, sa = oracle.quant_rowwise(act)
    np.testing.assert_array_equal(host(st["aq"])[:n], aq)
    np.testing.assert_array_equal(host(st["sa"])[:n], sa)
    A, W2d = oracle.dequant_rowwise(aq, sa), oracle.dequant_int4(p2, q2, 128)
    y2 = bf16_host(st["y2"])[:n]
    assert_close(oracle.bf16_to_f64(y2), oracle.gmm_fwd(A, W2d, sizes), FP8_TOL, GEMM_FP8, "y2",
                 fwd_norms(A, W2d, sizes))
    out_ref = oracle.unpermute(oracle.bf16_to_f64(y2), al["inv"], w, T, k)
    assert_close(oracle.bf16_to_f64(bf16_host(out)), out_ref, BF16_TOL, EW_ELEM)


@pytest.mark.parametrize("T", [1, 64, 300])
def test_fused_moe_fp8_stages_match_the_oracle(T):
    """The fp8-weight fused FFN, stage by stage, against the oracle fed the
    same quantized operands: the weight codes and per-(expert, column)
    scales, and the e4m3 codes of the gathered rows and of the activations,
    bit-exact; each fp8 GEMM within the fp8 tolerance of the oracle's fp64
    product of the dequantized operands; SiLU*mul and the combine within
    bf16 rounding.  T=300 takes 128-row blocks."""
    E, k, H, I = 8, 2, 256, 384
    ids, w = wl.softmax_topk_routing(T, E, k, 5)
    x = wl.normal_bf16((T, H), 1.0, 5, wl.T_X)
    W1 = wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, 5, wl.T_W1)
    W2 = wl.stacked_normal_bf16(E, (I, H), 0.05, 5, wl.T_W2)
    w1q, s1 = mg.quantize_fp8_expert_weights(bf16_dev(W1))
    w2q, s2 = mg.quantize_fp8_expert_weights(bf16_dev(W2))
    out, st = mg.fused_moe_fp8(bf16_dev(x), w1q, s1, w2q, s2, dev(ids), dev(w), keep_act=True)
    torch.cuda.synchronize()
    bm = 16 if T * k <= 64 * E else 128
    full = lambda n: np.full(E, n, np.int32)
    p1, q1 = oracle.quant_colwise(W1.reshape(E * H, 2 * I), full(H))
    p2, q2 = oracle.quant_colwise(W2.reshape(E * I, H), full(I))
    np.testing.assert_array_equal(host(w1q), p1)
    np.testing.assert_array_equal(host(s1), q1)
    np.testing.assert_array_equal(host(w2q), p2)
    np.testing.assert_array_equal(host(s2), q2)
    al = oracle.moe_align(ids, E, bm)
    n, sizes = al["num_tokens_post_padded"], al["padded_sizes"]
    xq, sx = oracle.quant_rowwise(oracle.gather_rows(x, k, al["sorted_token_ids"])[:n])
    np.testing.assert_array_equal(host(st["xq"])[:n], xq)
    np.testing.assert_array_equal(host(st["sx"])[:n], sx)
    A, W1d = oracle.dequant_rowwise(xq, sx), oracle.dequant_colwise(p1, q1, full(H)).reshape(E, H, 2 * I)
    h1 = bf16_host(st["h1"])[:n]
    assert_close(oracle.bf16_to_f64(h1), oracle.gmm_fwd(A, W1d, sizes), FP8_TOL, GEMM_FP8, "h1",
                 fwd_norms(A, W1d, sizes))
    act_ref = oracle.silu_mul(oracle.bf16_to_f64(h1))
    act = bf16_host(st["act"])[:n]
    assert_close(oracle.bf16_to_f64(act), act_ref, 4e-3, EW_ELEM)
    aq, sa = oracle.quant_rowwise(act)
    np.testing.assert_array_equal(host(st["aq"])[:n], aq)
    np.testing.assert_array_equal(host(st["sa"])[:n], sa)
    A, W2d = oracle.dequant_rowwise(aq, sa), oracle.dequant_colwise(p2, q2, full(I)).reshape(E, I, H)
    y2 = bf16_host(st["y2"])[:n]
    assert_close(oracle.bf16_to_f64(y2), oracle.gmm_fwd(A, W2d, sizes), FP8_TOL, GEMM_FP8, "y2",
                 fwd_norms(A, W2d, sizes))
    out_ref = oracle.unpermute(oracle.bf16_to_f64(y2), al["inv"], w, T, k)
    assert_close(oracle.bf16_to_f64(bf16_host(out)), out_ref, BF16_TOL, EW_ELEM)


@pytest.mark.parametrize("path", ["bf16", "fp8", "int4"])
def test_captured_decode_ffn_replays_bitwise(path):
    """A one-token fused FFN step captured in a HIP graph (no allocation
    outside torch's graph pool, no synchronization, no memset): every replay,
    with eager steps between the replays, reproduces the eager output bit for
    bit.  At these shapes the int4 path's F8I4 GEMMs split K across
    workgroups and the bf16 GEMM2 runs stream-K pieces, so the workspace's
    arrival counters, which reset themselves, are exercised across replays."""
    E, k, H, I = 8, 2, 2048, 2048
    ids, w = wl.softmax_topk_routing(1, E, k, 7)
    x = bf16_dev(wl.normal_bf16((1, H), 1.0, 7, wl.T_X))
    W1 = bf16_dev(wl.stacked_normal_bf16(E, (H, 2 * I), 0.02, 7, wl.T_W1))
    W2 = bf16_dev(wl.stacked_normal_bf16(E, (I, H), 0.02, 7, wl.T_W2))
    ids_d, w_d = dev(ids), dev(w)
    ws = mg.workspace(E, 256)
    if path == "bf16":
        step = lambda: mg.fused_moe(x, W1, W2, ids_d, w_d, ws=ws)[0]
    elif path == "fp8":
        w1q, s1 = mg.quantize_fp8_expert_weights(W1)
        w2q, s2 = mg.quantize_fp8_expert_weights(W2)
        step = lambda: mg.fused_moe_fp8(x, w1q, s1, w2q, s2, ids_d, w_d, ws=ws)[0]
    else:
        w1_4, s1 = mg.quantize_int4_weights(W1)
        w2_4, s2 = mg.quantize_int4_weights(W2)
        step = lambda: mg.fused_moe_f8i4(x, w1_4, s1, w2_4, s2, ids_d, w_d, ws=ws)[0]
    ref = step().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(step(), ref)   # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["bf16", "fp8", "int4"])
def test_captured_ffn_follows_routing_changed_between_replays(path):
    """Routing lives on the device: one captured fused FFN step serves any
    routing of its T tokens.  topk_ids and topk_weights (and the tokens) are
    overwritten in place between replays -- spread over all experts, all on
    one expert, a new random draw -- and each replay equals a fresh eager
    step with the new routing, bit for bit."""
    E, k, H, I, T = 8, 2, 256, 256, 24
    W1 = bf16_dev(wl.stacked_normal_bf16(E, (H, 2 * I), 0.05, 9, wl.T_W1))
    W2 = bf16_dev(wl.stacked_normal_bf16(E, (I, H), 0.05, 9, wl.T_W2))
    ids0, w0 = wl.softmax_topk_routing(T, E, k, 9)
    x = bf16_dev(wl.normal_bf16((T, H), 1.0, 9, wl.T_X))
    ids_d, w_d = dev(ids0), dev(w0)
    ws = mg.workspace(E, 1024)
    if path == "bf16":
        run = lambda i, wt, xx, s: mg.fused_moe(xx, W1, W2, i, wt, block_m=16, ws=s)[0]
    elif path == "fp8":
        w1q, s1 = mg.quantize_fp8_expert_weights(W1)
        w2q, s2 = mg.quantize_fp8_expert_weights(W2)
        run = lambda i, wt, xx, s: mg.fused_moe_fp8(xx, w1q, s1, w2q, s2, i, wt, block_m=16, ws=s)[0]
    else:
        w1_4, s1 = mg.quantize_int4_weights(W1)
        w2_4, s2 = mg.quantize_int4_weights(W2)
        run = lambda i, wt, xx, s: mg.fused_moe_f8i4(xx, w1_4, s1, w2_4, s2, i, wt, block_m=16, ws=s)[0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(ids_d, w_d, x, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = run(ids_d, w_d, x, ws)
    spread = np.stack([np.arange(T) % E, (np.arange(T) + 3) % E], axis=1).astype(np.int32)
    one = np.stack([np.full(T, 5), np.full(T, 2)], axis=1).astype(np.int32)
    drawn, _ = wl.softmax_topk_routing(T, E, k, 19)
    for i, ids in enumerate([spread, one, drawn]):
        wts = np.random.default_rng(i).random((T, k)).astype(np.float32)
        xs = wl.normal_bf16((T, H), 1.0, 40 + i, wl.T_X)
        ids_d.copy_(dev(ids))
        w_d.copy_(dev(wts))
        x.copy_(bf16_dev(xs))
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        ref = run(dev(ids), dev(wts), bf16_dev(xs), mg.workspace(E, 1024))
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
