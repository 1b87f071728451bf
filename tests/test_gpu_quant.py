"""GPU parity: fp8 rowwise and per-group colwise (single and dual) quantizers
and the int4 weight quantizer, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import oracle
import workloads as wl
from gpu_util import bf16_dev, bf16_host, dev, gpu, host, require_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _all_finite_bf16_rows(cols):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = wl.bf16_bits_to_f32(bits)
    bits = bits[np.isfinite(f)]
    pad = (-bits.size) % cols
    bits = np.concatenate([bits, np.zeros(pad, np.uint16)])
    return bits.reshape(-1, cols)


@pytest.mark.parametrize("cols", [128, 1024])
def test_rowwise_every_bf16_pattern_bit_exact(cols):
    x = _all_finite_bf16_rows(cols)
    # shuffle within rows so each row mixes magnitudes; also a shuffled copy by rows
    rng = np.random.default_rng(cols)
    x = np.concatenate([x, rng.permuted(x, axis=1)], axis=0)
    q, s = mg.quantize_rowwise_fp8(bf16_dev(x))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rowwise(x)
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


def test_rowwise_each_bf16_value_against_many_scales():
    """Rows whose amax sets scales 2^-126 .. 2^48, each row containing a
    spread of bf16 values below its amax: hits subnormal e4m3 codes, ties and
    the top code for every scale."""
    rng = np.random.default_rng(1)
    rows = []
    for e in range(-120, 120, 3):
        amax = np.float32(2.0 ** e * 1.37)
        vals = rng.uniform(-1, 1, 255).astype(np.float32) * amax
        rows.append(np.concatenate([[amax], vals]))
    x = wl.f32_to_bf16_bits(np.array(rows, np.float32))
    q, s = mg.quantize_rowwise_fp8(bf16_dev(x))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rowwise(x)
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


@pytest.mark.parametrize("rows,cols,ld", [(1, 8, 8), (37, 200, 208), (4096, 2048, 2048), (64, 14336, 14336),
                                          (3, 8192 + 8, 8192 + 8),
                                          # both sides of the workgroup-per-row kernel's limits
                                          (1024, 2048, 2056), (1025, 2048, 2048), (122, 2040, 2040),
                                          (5, 20480, 20480)])
def test_rowwise_shapes(rows, cols, ld):
    full = wl.normal_bf16((rows, ld), 1.0, rows, wl.T_X)
    full[rows // 2] = 0
    xt = bf16_dev(full)[:, :cols]
    q, s = mg.quantize_rowwise_fp8(xt)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rowwise(np.ascontiguousarray(full[:, :cols]))
    np.testing.assert_array_equal(host(s), s_ref)
    np.testing.assert_array_equal(host(q), q_ref)


def _check_colwise(x, sizes, q, s):
    q_ref, s_ref = oracle.quant_colwise(x, sizes)
    np.testing.assert_array_equal(host(s), s_ref)
    covered = int(sizes.sum())
    np.testing.assert_array_equal(host(q)[:, :covered], q_ref[:, :covered])


@pytest.mark.parametrize("M,C,G,mult,seed", [
    (1000, 64, 5, 1, 0), (16640, 2048, 64, 16, 1), (777, 200, 9, 1, 2), (4096, 1408, 64, 1, 3),
    (64, 8, 3, 1, 4), (3000, 520, 128, 1, 5),
])
def test_colwise_single_bit_exact(M, C, G, mult, seed):
    if mult > 1:
        sizes = wl.jagged_sizes_multiple_of(G, M, mult, seed)
    else:
        sizes = wl.random_group_sizes(G, M, seed, zero_frac=0.2)
    x = wl.normal_bf16((M, C), 1.0, seed, wl.T_DY)
    qa, sa = mg.quantize_colwise_per_group_fp8(bf16_dev(x), dev(sizes))
    torch.cuda.synchronize()
    _check_colwise(x, sizes, qa, sa)


def test_colwise_dual_equals_two_singles_and_oracle():
    M, G = 5000, 64
    sizes = wl.random_group_sizes(G, M, 7, zero_frac=0.2)
    a = wl.normal_bf16((M, 1408), 1.0, 7, wl.T_DY)
    b = wl.normal_bf16((M, 2048), 1.0, 7, wl.T_X)
    gs = dev(sizes)
    qa, sa, qb, sb = mg.quantize_colwise_per_group_fp8(bf16_dev(a), gs, b=bf16_dev(b))
    qa1, sa1 = mg.quantize_colwise_per_group_fp8(bf16_dev(a), gs)
    qb1, sb1 = mg.quantize_colwise_per_group_fp8(bf16_dev(b), gs)
    torch.cuda.synchronize()
    for u, v in [(qa, qa1), (sa, sa1), (qb, qb1), (sb, sb1)]:
        assert torch.equal(u, v)
    _check_colwise(a, sizes, qa, sa)
    _check_colwise(b, sizes, qb, sb)


@pytest.mark.parametrize("pad", [37, None])   # an odd stride, and the library's own (colwise_ld)
def test_colwise_padded_code_rows(pad):
    """Code rows ld bytes apart: the codes equal those of contiguous rows,
    and the bytes past M of every row keep what they held."""
    M, G = 3000, 6
    sizes = wl.random_group_sizes(G, M, 11, zero_frac=0.2)
    a = wl.normal_bf16((M, 136), 1.0, 11, wl.T_DY)
    b = wl.normal_bf16((M, 264), 1.0, 11, wl.T_X)
    gs = dev(sizes)
    ld = M + pad if pad is not None else mg.colwise_ld(M)
    qa = torch.full((136, ld), 0xA5, dtype=torch.uint8, device="cuda")
    qb = torch.full((264, ld), 0xA5, dtype=torch.uint8, device="cuda")
    out = (qa[:, :M], torch.empty(G, 136, dtype=torch.float32, device="cuda"),
           qb[:, :M], torch.empty(G, 264, dtype=torch.float32, device="cuda"))
    mg.quantize_colwise_per_group_fp8(bf16_dev(a), gs, b=bf16_dev(b), out=out)
    ref = (torch.empty(136, M, dtype=torch.uint8, device="cuda"), torch.empty(G, 136, dtype=torch.float32, device="cuda"),
           torch.empty(264, M, dtype=torch.uint8, device="cuda"), torch.empty(G, 264, dtype=torch.float32, device="cuda"))
    mg.quantize_colwise_per_group_fp8(bf16_dev(a), gs, b=bf16_dev(b), out=ref)
    torch.cuda.synchronize()
    for u, v in zip(out, ref):
        assert torch.equal(u, v)
    assert (qa[:, M:] == 0xA5).all() and (qb[:, M:] == 0xA5).all()
    _check_colwise(a, sizes, out[0], out[1])


def test_colwise_rows_outside_groups_untouched():
    M, C = 300, 64
    sizes = np.array([50, 0, 70], np.int32)       # covers 120 rows
    x = wl.normal_bf16((M, C), 1.0, 0, wl.T_X)
    qa = torch.full((C, M), 0xA5, dtype=torch.uint8, device="cuda")
    sa = torch.empty(3, C, dtype=torch.float32, device="cuda")
    mg.quantize_colwise_per_group_fp8(bf16_dev(x), dev(sizes), out=(qa, sa))
    torch.cuda.synchronize()
    assert (host(qa)[:, 120:] == 0xA5).all()
    _check_colwise(x, sizes, qa, sa)


@pytest.mark.parametrize("M,C,sizes", [
    # groups over several 512-row blocks (the second pass), one-chunk groups
    # that straddle a block boundary, starts and ends off the 16-byte grid,
    # a row count that is not a multiple of 16 (every column's run sits
    # differently in its pieces), a partial last 64-column block, empty
    # groups and rows past the groups
    (20001, 200, [1, 5000, 0, 9000, 3, 5990]),
    (8200, 72, [1023, 1025, 2048, 0, 4097]),
    (3072, 8, [3072]),
    (5000, 64, [300, 400, 5, 511, 512, 513, 1, 2000]),
    (2000, 72, [255, 256, 257, 1, 512, 513, 0, 100]),
])
def test_colwise_sets_of_several_chunks(M, C, sizes):
    sizes = np.array(sizes, np.int32)
    x = wl.normal_bf16((M, C), 1.0, 11, wl.T_DY)
    qa, sa = mg.quantize_colwise_per_group_fp8(bf16_dev(x), dev(sizes))
    torch.cuda.synchronize()
    _check_colwise(x, sizes, qa, sa)


def test_colwise_group_longer_than_128_blocks():
    # 150000 rows from row 17 touch 294 blocks of 512 rows: each chunk takes
    # three blocks (the first pass folds them all, the second reads them
    # again for the cast)
    M, C = 153200, 64
    sizes = np.array([17, 150000, 3000], np.int32)
    x = wl.normal_bf16((M, C), 1.0, 12, wl.T_X)
    qa, sa = mg.quantize_colwise_per_group_fp8(bf16_dev(x), dev(sizes))
    torch.cuda.synchronize()
    _check_colwise(x, sizes, qa, sa)


def test_colwise_repeated_calls_share_a_workspace():
    # the workspace carries partial maxima from the first pass to the second
    # and nothing from one call to the next: calls of different chunkings in
    # a row, on one workspace that is never cleared, each match the oracle
    M, C, G = 12000, 136, 4
    ws = torch.full((mg.colwise_workspace_bytes(G, M, C, 64),), 0x5A, dtype=torch.uint8, device="cuda")
    ws[:4].zero_()   # the sticky error word
    a = wl.normal_bf16((M, C), 1.0, 13, wl.T_DY)
    b = wl.normal_bf16((M, 64), 1.0, 13, wl.T_X)
    for sizes in ([5000, 0, 6500, 400], [1, 11998, 0, 1], [3000, 3000, 3000, 3000], [512, 513, 1024, 0]):
        sizes = np.array(sizes, np.int32)
        qa, sa, qb, sb = mg.quantize_colwise_per_group_fp8(bf16_dev(a), dev(sizes), b=bf16_dev(b), ws=ws)
        torch.cuda.synchronize()
        _check_colwise(a, sizes, qa, sa)
        _check_colwise(b, sizes, qb, sb)
        assert mg.workspace_error(ws) == 0


def test_colwise_rejects_a_small_workspace():
    x = bf16_dev(wl.normal_bf16((2048, 64), 1.0, 0, wl.T_X))
    gs = dev(np.array([2048], np.int32))
    ws = torch.zeros(mg.colwise_workspace_bytes(1, 2048, 64) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        mg.quantize_colwise_per_group_fp8(x, gs, ws=ws)


def test_colwise_graph_replay_follows_new_group_sizes():
    """The quantizer captured in a graph reads the device group sizes at every
    replay, so replays after the sizes change in place match fresh eager
    calls."""
    M, C, G = 9000, 136, 5
    x = bf16_dev(wl.normal_bf16((M, C), 1.0, 14, wl.T_DY))
    gs = dev(np.array([2000, 2000, 2000, 2000, 1000], np.int32))
    ws = torch.zeros(mg.colwise_workspace_bytes(G, M, C), dtype=torch.uint8, device="cuda")
    qa = torch.zeros(C, M, dtype=torch.uint8, device="cuda")
    sa = torch.zeros(G, C, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mg.quantize_colwise_per_group_fp8(x, gs, out=(qa, sa), ws=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.quantize_colwise_per_group_fp8(x, gs, out=(qa, sa), ws=ws)
    for sizes in ([2000, 2000, 2000, 2000, 1000], [0, 8999, 0, 1, 0], [1500, 1, 3000, 0, 4000],
                  [9000, 0, 0, 0, 0]):
        gs.copy_(dev(np.array(sizes, np.int32)))
        qa.zero_()
        g.replay()
        torch.cuda.synchronize()
        qr, sr = mg.quantize_colwise_per_group_fp8(x, gs, ws=torch.zeros_like(ws))
        torch.cuda.synchronize()
        covered = int(sum(sizes))
        assert torch.equal(sa, sr)
        assert torch.equal(qa[:, :covered], qr[:, :covered])
    assert mg.workspace_error(ws) == 0


def test_quantizers_reject_mismatched_output_buffers():
    x = bf16_dev(wl.normal_bf16((64, 32), 1.0, 0, wl.T_X))
    with pytest.raises(ValueError):
        mg.quantize_rowwise_fp8(x, q=torch.empty(63, 32, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        mg.quantize_rowwise_fp8(x, scales=torch.empty(64, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):
        mg.quantize_rowwise_fp8(x, q=torch.empty(32, 64, dtype=torch.uint8, device="cuda").t())
    ids = dev(np.arange(64, dtype=np.int32))
    with pytest.raises(ValueError):
        mg.quantize_rowwise_fp8_gather(x, ids, 1, scales=torch.empty(10, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        mg.quantize_colwise_per_group_fp8(x, dev(np.array([64], np.int32)),
                                          out=(torch.empty(32, 60, dtype=torch.uint8, device="cuda"),
                                               torch.empty(1, 32, dtype=torch.float32, device="cuda")))


@pytest.mark.parametrize("E,K,N", [(2, 256, 64), (3, 5120, 136)])
def test_int4_quantizer_bit_exact(E, K, N):
    w = wl.stacked_normal_bf16(E, (K, N), 0.02, 0, wl.T_W)
    w4, sw = mg.quantize_int4_weights(bf16_dev(w))
    torch.cuda.synchronize()
    p_ref, s_ref = oracle.quant_int4(oracle.bf16_to_f64(w), 128)
    np.testing.assert_array_equal(bf16_host(sw), s_ref)
    np.testing.assert_array_equal(host(w4), p_ref)


@pytest.mark.parametrize("T,k,E,bm,cols", [(1, 2, 8, 16, 4096), (64, 2, 8, 16, 14336), (300, 6, 64, 16, 512),
                                           (2000, 2, 8, 128, 2048),
                                           (600, 2, 8, 16, 8192),    # rows past the register-held chunks
                                           (8, 2, 8, 16, 20480)])    # few rows past 16384 columns, sentinels
def test_rowwise_gather_bit_exact(T, k, E, bm, cols):
    """Rowwise e4m3 of the token rows in sorted order, padding sentinels
    included, equals the oracle's rowwise quantizer on the oracle's gather,
    codes and scales bit for bit (few long rows take the workgroup-per-row
    kernel, many rows the wave-per-row one)."""
    ids, _ = wl.softmax_topk_routing(T, E, k, cols)
    x = wl.normal_bf16((T, cols), 1.0, cols, wl.T_X)
    x[T // 2] = 0
    al = oracle.moe_align(ids, E, bm)
    sids = al["sorted_token_ids"]
    q, s = mg.quantize_rowwise_fp8_gather(bf16_dev(x), dev(sids), k)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rowwise(oracle.gather_rows(x, k, sids))
    np.testing.assert_array_equal(host(q), q_ref)
    np.testing.assert_array_equal(host(s), s_ref)


@pytest.mark.parametrize("rows,inter", [(1, 8), (7, 1408), (300, 14336), (5, 16392), (3, 40000)])
def test_silu_mul_quantize_rowwise_one_pass(rows, inter):
    """SiLU*mul and rowwise e4m3 in one pass: codes and scales bit-exact
    against the oracle's rowwise quantizer applied to the library's own
    SiLU*mul output, and the same bits as silu_mul followed by
    quantize_rowwise_fp8, with and without the bf16 activations written
    out.  Rows of 16392 and 40000 values are longer than the registers
    hold (the cast recomputes act from h); one row is zero, one spans
    large magnitudes."""
    g = wl.rng(60 + rows, wl.T_X)
    h = wl.normal_bf16((rows, 2 * inter), 1.0, 60 + rows, wl.T_X)
    hf = wl.bf16_bits_to_f32(h)
    if rows > 2:
        h[1] = 0
        hf[2] *= np.float32(2.0) ** g.integers(-20, 20, size=2 * inter)
        h[2] = wl.f32_to_bf16_bits(hf[2])
    hd = bf16_dev(h)
    act = mg.silu_mul(hd)
    q2, s2 = mg.quantize_rowwise_fp8(act)
    q1, s1 = mg.silu_mul_quantize_rowwise_fp8(hd)
    act1 = torch.empty_like(act)
    q3, s3 = mg.silu_mul_quantize_rowwise_fp8(hd, act=act1)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rowwise(bf16_host(act))
    np.testing.assert_array_equal(host(s1), s_ref)
    np.testing.assert_array_equal(host(q1), q_ref)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    assert torch.equal(q1, q3) and torch.equal(s1, s3)
    assert torch.equal(act1, act)
