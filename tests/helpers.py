"""Shared test helpers: device upload and the normwise error metric."""
import numpy as np


def err(a, ref):
    """max|a - ref| / max|ref| (normwise infinity)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(a - ref).max() / (den if den > 0 else 1.0))


def dev(a):
    """numpy array -> CUDA tensor with the same bytes (uint16 travels as int16)."""
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t, dtype=None):
    """CUDA tensor -> numpy (int16 views come back as uint16 when asked)."""
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def bf16_to_f64(bits):
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
