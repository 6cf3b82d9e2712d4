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


def row_err(gpu, ref) -> float:
    """Per-row version of rel_err: the largest over rows (every index but
    the last) of max_j |gpu - ref| / max_j |ref| within the row. Reported
    beside the per-tensor metric; rows whose reference is all zero are
    skipped."""
    g = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    g = g.reshape(-1, g.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    den = np.abs(r).max(axis=1)
    keep = den > 0
    return float((np.abs(g - r).max(axis=1)[keep] / den[keep]).max())


def full_size_rows(L: int, n_random: int = 252, seed: int = 0):
    """Query rows checked at full prefill size: the first three, the last,
    and a seeded sample of the others (all sequences and heads)."""
    fixed = [0, 1, 2, L - 1]
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(L), fixed)
    return sorted(set(fixed) | set(rng.choice(pool, min(n_random, pool.size), replace=False).tolist()))


def dev(t):
    return t.to("cuda")


def say(msg: str):
    print(msg, flush=True)
