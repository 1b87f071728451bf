"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module only draws random numbers and lays them out; it holds none of the
grouped-GEMM arithmetic.  Every stream is numpy PCG64 seeded with
``SeedSequence([seed, tensor_id, sub])`` so that a tensor (or one expert's
slice of it) can be regenerated on its own.  fp32 -> bf16 conversion is
round-to-nearest-even on the bit pattern; bf16 tensors are returned as uint16
bit patterns.
"""
import numpy as np

# tensor ids (stable: changing them changes every fixture)
T_X, T_W, T_DY, T_LOGITS, T_W1, T_W2, T_ROUTE, T_PERM, T_SIZES = range(9)


def rng(seed, tensor_id, sub=None):
    key = [int(seed), int(tensor_id)] + ([] if sub is None else [int(sub)])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform_bf16(shape, lo, hi, seed, tensor_id, sub=None):
    g = rng(seed, tensor_id, sub)
    x = g.random(size=shape, dtype=np.float32) * np.float32(hi - lo) + np.float32(lo)
    return f32_to_bf16_bits(x)


def normal_bf16(shape, std, seed, tensor_id, sub=None):
    g = rng(seed, tensor_id, sub)
    x = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(x)


def stacked_normal_bf16(E, shape, std, seed, tensor_id):
    """[E, *shape] with one independent substream per expert."""
    out = np.empty((E,) + tuple(shape), np.uint16)
    for e in range(E):
        out[e] = normal_bf16(shape, std, seed, tensor_id, e)
    return out


# --------------------------------------------------------------------------
# Group sizes
# --------------------------------------------------------------------------

def random_group_sizes(E, total, seed, zero_frac=0.3):
    """Random sizes summing to `total`, with some groups forced empty."""
    g = rng(seed, T_SIZES)
    if E == 1:
        return np.array([total], np.int32)
    active = g.random(E) >= zero_frac
    if not active.any():
        active[g.integers(E)] = True
    cuts = np.sort(g.integers(0, total + 1, size=int(active.sum()) - 1))
    parts = np.diff(np.concatenate([[0], cuts, [total]]))
    sizes = np.zeros(E, np.int64)
    sizes[active] = parts
    return sizes.astype(np.int32)


def jagged_sizes_multiple_of(G, M, multiple, seed):
    """G-1 distinct cut points drawn from the multiples of `multiple` in
    (0, M), sorted, then M appended; returned as sizes."""
    g = rng(seed, T_SIZES)
    cands = np.arange(multiple, M, multiple)
    cuts = np.sort(g.choice(cands, size=G - 1, replace=False))
    ends = np.concatenate([cuts, [M]])
    return np.diff(np.concatenate([[0], ends])).astype(np.int32)


def uniform_expert_rows(total_M, E, seed):
    """Each of total_M rows goes to an expert drawn uniformly from 0..E-1."""
    g = rng(seed, T_ROUTE)
    ids = g.integers(0, E, size=total_M)
    return np.bincount(ids, minlength=E).astype(np.int32)


def zipf_topk_routing(T, E, k, s, seed):
    """Zipf(s) expert popularity over a seeded permutation of the experts;
    each token draws k distinct experts by Gumbel-top-k on log-popularity.
    Returns topk_ids [T, k] int32."""
    g = rng(seed, T_PERM)
    perm = g.permutation(E)
    pop = np.empty(E, np.float64)
    pop[perm] = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    logp = np.log(pop / pop.sum())
    g2 = rng(seed, T_ROUTE)
    keys = logp[None, :] + g2.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return ids.astype(np.int32)


def softmax_topk_routing(T, E, k, seed):
    """Router logits N(0,1) fp32 -> softmax (fp32) -> top-k.  Returns
    (topk_ids [T,k] int32, topk_weights [T,k] fp32); ties broken by the lower
    expert index."""
    g = rng(seed, T_LOGITS)
    logits = g.standard_normal(size=(T, E), dtype=np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = np.take_along_axis(p, ids, axis=1).astype(np.float32)
    return ids, w


# --------------------------------------------------------------------------
# Named workloads (shapes and value distributions of the pages' runs)
# --------------------------------------------------------------------------

def tiny_bf16(seed=0):
    """E=4, K=64, N=48, sizes [0,20,9,8]; X, W uniform[-1,1) bf16."""
    sizes = np.array([0, 20, 9, 8], np.int32)
    X = uniform_bf16((37, 64), -1.0, 1.0, seed, T_X)
    W = uniform_bf16((4, 64, 48), -1.0, 1.0, seed, T_W)
    return dict(sizes=sizes, X=X, W=W, E=4, M=37, K=64, N=48)


def balanced_bf16(seed=0, E=8, M=1024, K=4096, N=6400, with_w=True):
    """M rows split equally over E groups; X, W uniform[0,1) bf16; dY = ones
    (gradient of the sum of the output)."""
    sizes = np.full(E, M // E, np.int32)
    X = uniform_bf16((M, K), 0.0, 1.0, seed, T_X)
    W = None
    if with_w:
        W = np.empty((E, K, N), np.uint16)
        for e in range(E):
            W[e] = uniform_bf16((K, N), 0.0, 1.0, seed, T_W, e)
    dY = np.full((M, N), 0x3F80, np.uint16)  # bf16 1.0
    return dict(sizes=sizes, X=X, W=W, dY=dY, E=E, M=M, K=K, N=N)
