"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import pytest
import torch

DEV = torch.device("cuda:0")

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_dev(bits):
    """numpy uint16 bf16 bit patterns -> device bfloat16 tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host(t):
    """device bfloat16 tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


BF16_TOL = 5e-3
FP8_TOL = 2e-2

# Element-wise bars beside the relative Frobenius one, so that one wrong
# element, row or tile fails even when it barely moves the norm.  Each is a
# pair (rel, u): every element must satisfy
#     |got - ref| <= rel * |ref| + u * scale
# where scale is, for a product, the element's own ||a_r|| ||b_n|| (the
# norms of the row and column it contracts, which bound sum_k |a_k b_k| by
# Cauchy-Schwarz), and otherwise the output's rms.
#   Products: the library rounds its sum to bf16 (at most 2^-8 |value|) and
#     its summation error is a small multiple of sum_k |a_k b_k|.  Measured
#     on MI355X, beyond half an output ulp: the bf16 MFMA at most 2^-25 of
#     ||a|| ||b|| (fp32-exact summation); the e4m3 MFMA (f8f6f4) at most
#     2^-17.5 of ||a|| ||b|| (2^-15 of sum |ab|) with codes spread over every
#     e4m3 binade, 2^-19.5 with quantized normal data -- its block sums keep
#     fewer bits than fp32.  GEMM_BF16 and GEMM_FP8 leave a margin of at
#     least 2^4 over those.
#   EW_ELEM: an element-wise stage (SiLU*mul, the top-k combine) on the
#     identical inputs: fp32 arithmetic, then one bf16 rounding.
#   SWIGLU_ELEM: SiLU*mul applied to the two halves of a product, which both
#     sides round to bf16 first; the library's fp32 sum and the oracle's
#     exact one can round a half to neighbouring bf16 values (about one
#     element in a thousand).  SiLU's relative slope |1 + g (1 - sigmoid(g))|
#     stays below 2^3 for |g| < 9, so a step of 2^-7 in either half plus the
#     final rounding moves such an element by less than 2^-3 of itself.
#   CHAIN_ELEM: the whole FFN against the oracle's own chain, whose bf16
#     intermediates can differ from the library's by one rounding step:
#     an output row then moves by at most 2^-7 of each weighted expert row,
#     a few times the output's rms at the extremes.
GEMM_BF16 = (2.0 ** -7, 2.0 ** -18)
GEMM_FP8 = (2.0 ** -7, 2.0 ** -13)
EW_ELEM = (2.0 ** -7, 2.0 ** -16)
SWIGLU_ELEM = (2.0 ** -3, 2.0 ** -12)
CHAIN_ELEM = (2.0 ** -6, 2.0 ** -4)


def group_rows(sizes, M):
    """Group of each of M stacked rows (-1 past the groups)."""
    grp = np.full(M, -1, np.int64)
    o = 0
    for g, n in enumerate(np.asarray(sizes, np.int64)):
        grp[o:o + n] = g
        o += n
    return grp


def vec_norms(a, axis):
    """Euclidean norms along axis, in fp64."""
    return np.sqrt(np.sum(np.square(np.asarray(a, np.float64)), axis=axis))


def fwd_norms(A, W, sizes, trans_b=False):
    """Scale terms of Y[r] = A[r] . W[g(r)] (W [E, K, N], or [E, N, K] with
    trans_b): row norms of A, column norms of each W[g], and g(r)."""
    cn = np.stack([vec_norms(W[e], 1 if trans_b else 0) for e in range(W.shape[0])])
    return vec_norms(A, 1), cn, group_rows(sizes, A.shape[0])


def dx_norms(dY, W, sizes, trans_b=False):
    """Scale terms of dX[r] = dY[r] . W[g(r)]^T (contraction over N)."""
    cn = np.stack([vec_norms(W[e], 0 if trans_b else 1) for e in range(W.shape[0])])
    return vec_norms(dY, 1), cn, group_rows(sizes, dY.shape[0])


def dw_norms(X, dY, sizes):
    """Scale terms of dW[g] = X_g^T . dY_g, with dW viewed as [E * K, N]."""
    E, K = len(sizes), X.shape[1]
    rn = np.zeros(E * K)
    cn = np.zeros((E, dY.shape[1]))
    o = 0
    for g, n in enumerate(np.asarray(sizes, np.int64)):
        rn[g * K:(g + 1) * K] = vec_norms(X[o:o + n], 0)
        cn[g] = vec_norms(dY[o:o + n], 0)
        o += n
    return rn, cn, np.repeat(np.arange(E), K)


def assert_close(got, ref, fro_tol, elem=None, what="output", norms=None):
    """Relative Frobenius error <= fro_tol, and every element within
    elem[0] |ref| + elem[1] scale, scale = ||a_r|| ||b_n|| from norms (a
    product; see fwd_norms, dx_norms, dw_norms) or rms(ref).  Checked in
    row blocks; a 3-d output is viewed as [d0 * d1, d2]."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    err = rel_fro(got, ref)
    assert err <= fro_tol, f"{what}: relative Frobenius error {err:.3e} > {fro_tol}"
    if ref.size == 0:
        return
    if elem is None:
        elem = GEMM_BF16 if norms is not None else EW_ELEM
    rel, u = elem
    cols = ref.shape[-1] if ref.ndim > 1 else 1
    g2, r2 = got.reshape(-1, cols), ref.reshape(-1, cols)
    rms = 0.0
    if norms is None:
        ss = sum(float(np.sum(np.square(r2[i:i + 4096], dtype=np.float64))) for i in range(0, r2.shape[0], 4096))
        rms = (ss / ref.size) ** 0.5
    else:
        rn, cn, grp = norms
        assert rn.shape[0] == r2.shape[0] and cn.shape[1] == cols and (grp >= 0).all(), f"{what}: norms shape"
    nbad, worst = 0, None
    for i in range(0, r2.shape[0], 4096):
        g = np.asarray(g2[i:i + 4096], np.float64)
        r = np.asarray(r2[i:i + 4096], np.float64)
        scale = rms if norms is None else rn[i:i + 4096, None] * cn[grp[i:i + 4096]]
        excess = np.abs(g - r) - (rel * np.abs(r) + u * scale)
        bad = excess > 0
        if bad.any():
            nbad += int(bad.sum())
            j = np.unravel_index(int(np.argmax(excess)), excess.shape)
            if worst is None or excess[j] > worst[0]:
                sc = scale if np.isscalar(scale) else float(scale[j])
                worst = (float(excess[j]), (i + j[0], j[1]), float(g[j]), float(r[j]), sc)
    assert nbad == 0, (f"{what}: {nbad} of {ref.size} elements outside {rel:.3g}|ref| + {u:.3g} scale; worst at "
                       f"row {worst[1][0]}, column {worst[1][1]}: got {worst[2]!r}, ref {worst[3]!r}, "
                       f"scale {worst[4]:.4g}")
