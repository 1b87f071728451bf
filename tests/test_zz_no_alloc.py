"""gmm_fwd_noalloc: the grouped GEMM forward with the library's own fixed
scratch, for callers that cannot allocate.  Through the C ABI it must give
the same bits as gmm_fwd with a caller's workspace, on consecutive calls of
different sizes (the scratch keeps the last call's contents)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_device_amd as mg
import workloads as wl
from gpu_util import bf16_dev, dev, gpu, require_gpu

pytestmark = gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _run_both(E, M, K, N, seed, trans_b, sizes=None):
    if sizes is None:
        sizes = wl.random_group_sizes(E, M, seed, zero_frac=0.25)
    x = bf16_dev(wl.normal_bf16((M, K), 1.0, seed, wl.T_X))
    w = bf16_dev(wl.normal_bf16((E, N, K) if trans_b else (E, K, N), 0.5, seed, wl.T_W))
    gs = dev(sizes)
    y_na = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    mg.gmm_fwd_noalloc(x, w, gs, y_na, trans_b=trans_b)
    y_ws = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    mg.gmm_fwd(x, w, gs, trans_b=trans_b, out=y_ws, ws=mg.workspace(E, M))
    torch.cuda.synchronize()
    return y_na, y_ws, int(sizes.sum())


def test_noalloc_equals_gmm_fwd_on_consecutive_calls():
    """A call whose last round runs stream-K pieces (one group, 4352 x 4096
    at K=256: 544 tiles over the 256-workgroup grid, 2-3 pieces per split
    tile, so the arrival counters and partial tiles are used), then a
    smaller ragged call with empty groups and rows past the groups, then
    the first shape again: each is bit-identical to gmm_fwd."""
    cases = [(1, 4352, 256, 4096, 1, False, np.array([4352], np.int32)),
             (5, 300, 200, 264, 2, True, None),
             (3, 1000, 136, 392, 3, False, np.array([400, 0, 350], np.int32)),
             (1, 4352, 256, 4096, 4, False, np.array([4352], np.int32))]
    for E, M, K, N, seed, trans_b, sizes in cases:
        y_na, y_ws, s = _run_both(E, M, K, N, seed, trans_b, sizes)
        assert torch.equal(y_na, y_ws), (E, M, K, N)
        assert (y_na[s:] == 5.0).all()


def test_noalloc_rejects_before_touching_the_device():
    x = torch.zeros(4, 8, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(2000, 8, 8, dtype=torch.bfloat16, device="cuda")
    gs = torch.zeros(2000, dtype=torch.int32, device="cuda")
    y = torch.zeros(4, 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.MoeGemmError) as e:
        mg.gmm_fwd_noalloc(x, w, gs, y)
    assert e.value.code == mg.MG_EINVAL
