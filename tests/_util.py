"""Shared test helpers: moving seeded host arrays to the device and comparison metrics."""
import numpy as np


def ndhwc(a):
    """NCDHW host array -> contiguous NDHWC float64 copy."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).transpose(0, 2, 3, 4, 1))


TORCH_DTYPES = {"bf16": "bfloat16", "f32": "float32", "f16": "float16"}


def dev(a, dtype="bf16"):
    """Host NDHWC array (values exact in ``dtype`` for bf16/f16) -> contiguous device tensor."""
    import torch
    t = torch.as_tensor(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(device="cuda", dtype=getattr(torch, TORCH_DTYPES[dtype]))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max_abs(got, ref):
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def psnr(got, ref):
    """10 log10(R^2 / MSE), R = max(ref) - min(ref), in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mse = float(np.mean((got - ref) ** 2))
    rng = float(ref.max() - ref.min())
    return float("inf") if mse == 0 else 10.0 * np.log10(rng * rng / mse)


def bf16_round_bound(ref):
    """Elementwise bound of one round-to-nearest-even bf16 store of ``ref``: half a bf16 ulp."""
    return np.abs(ref) * 2.0 ** -8


def f16_round_bound(ref):
    """Elementwise bound of one round-to-nearest-even fp16 store of ``ref`` (normal range): half
    an fp16 ulp."""
    return np.abs(ref) * 2.0 ** -11


def round_f16(a):
    """Nearest-even fp16 rounding (numpy's conversion), back in float64."""
    return np.asarray(a, np.float64).astype(np.float16).astype(np.float64)
