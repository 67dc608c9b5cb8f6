"""Shared helpers for the GPU parity tests: host<->device conversion and error metrics."""
import numpy as np


def to_dev(x, dtype):
    """float32 numpy array (bf16-exact when dtype is bf16) -> contiguous CUDA tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def to_host(t):
    """CUDA tensor -> float64 numpy array."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((got - ref).ravel()) / (den if den > 0 else 1.0))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


# Tolerances: fp32 forward max-abs 1e-5; bf16 relative L2 1e-2 on O and 2e-2 on dQ/dK/dV.
TOL_F32_MAXABS = 1e-5
TOL_O = 1e-2
TOL_GRAD = 2e-2
TOL_LSE_BF16 = 2e-2     # absolute, on natural-log LSE values of size ~1..10
