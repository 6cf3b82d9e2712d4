"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

BF16_TOL = 1e-2   # max |gpu - ref| / max |ref| per output tensor, bf16 inputs
F32_TOL = 1e-4    # same metric for the fp32 path


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a (bf16 or fp32) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(gpu, ref) -> float:
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "non-finite GPU output"
    return float(np.abs(g - r).max() / np.abs(r).max())


def dev(t):
    return t.to("cuda")


def say(msg: str):
    print(msg, flush=True)
