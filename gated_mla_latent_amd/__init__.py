"""Gated Multi-head Latent Attention kernels for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library `libgmla.so` (C ABI declared in
include/gmla.h). `gated_mla_latent_amd.ops` is a thin ctypes binding over it
that passes torch device pointers and the current HIP stream; it refuses to run
when the library has not been built.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "ops"]


def __getattr__(name):
    if name == "ops":
        import importlib
        return importlib.import_module(__name__ + ".ops")
    raise AttributeError(name)
