"""Chunkwise Kimi Delta Attention (KDA) for MI355X (gfx950).

The compute lives in ``libkda.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/kda.h``).  This package only marshals arguments:
``chunk_fwd`` (prefill over packed sequences) and ``step_decode`` (one token
per request), ``chunk_fwd_static`` (the prefill on a static device scratch,
for callers that cannot allocate), plus the layer steps around them:
``chunk_fwd_fused`` (prefill with L2Norm and the bounded gate in the kernel),
``step_decode_gated`` (decode with the output gate in the kernel),
``front_end`` (L2Norm and the bounded gate as a pass of their own), ``output_gate``,
``short_conv``, ``state_compose`` and the segment helpers ``kcp_summaries`` /
``kcp_scan``.  The library is loaded on first use and its absence is an error.
"""
from . import inputs  # noqa: F401  (seeded synthetic inputs; no compute)

_API = ("chunk_fwd", "step_decode", "chunk_fwd_fused", "output_gate", "short_conv",
        "state_compose", "kcp_summaries", "kcp_scan", "step_decode_gated", "chunk_fwd_static",
        "front_end", "library", "workspace_size", "KdaError")
__all__ = list(_API[:11]) + ["inputs", "library"]


def __getattr__(name):
    if name in _API:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
