"""Chunkwise Kimi Delta Attention (KDA) for MI355X (gfx950).

The compute lives in ``libkda.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/kda.h``).  This package only marshals arguments:
``chunk_fwd`` (prefill over packed sequences) and ``step_decode`` (one token
per request).  The library is loaded on first use and its absence is an error.
"""
from . import inputs  # noqa: F401  (seeded synthetic inputs; no compute)

__all__ = ["chunk_fwd", "step_decode", "inputs", "library"]


def __getattr__(name):
    if name in ("chunk_fwd", "step_decode", "library", "workspace_size", "KdaError"):
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
