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
