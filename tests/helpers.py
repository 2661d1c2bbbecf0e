"""Shared test utilities: tolerance metrics and device plumbing (no method arithmetic)."""
import numpy as np
import torch

# Tolerances of the parity bar:
#  float32 activations: max_i |y_i - r_i| / max(|r_i|, 1e-2 * max_j |r_j|) <= 1e-4
#  bfloat16 activations: max_i |y_i - r_i| / max_j |r_j| <= 2e-2
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def as_np(t):
    if isinstance(t, torch.Tensor):
        t = t.detach()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def err_f32(got, ref):
    got, ref = as_np(got), as_np(ref)
    scale = np.abs(ref).max()
    floor = np.maximum(np.abs(ref), 1e-2 * scale)
    floor = np.where(floor > 0, floor, 1.0)
    return float((np.abs(got - ref) / floor).max())


def err_bf16(got, ref):
    got, ref = as_np(got), as_np(ref)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def err_for(dtype):
    return err_f32 if dtype in ("f32", torch.float32) else err_bf16


def tol_for(dtype):
    return TOL_F32 if dtype in ("f32", torch.float32) else TOL_BF16


def to_dev(d, device="cuda:0"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def gpu_available():
    return torch.cuda.is_available()
