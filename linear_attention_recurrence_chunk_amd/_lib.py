"""ctypes binding of libkda.so (see include/kda.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch on the inputs' device, and the C entry points are called
on torch's current HIP stream.  Every step of the computation runs in the
library's kernels; there is no other code path, and a missing library is an
error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}
_lib = None


class KdaError(RuntimeError):
    """A non-zero status returned by libkda.so."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libkda.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m linear_attention_recurrence_chunk_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd_workspace_size.restype = sz
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                  vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_step_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_step_decode.restype = i32
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = i32
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise KdaError(fn, status, library().kda_status_string(status).decode())


def _ptr(x: Optional[torch.Tensor]):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(x, name, dtype=None, ndim=None, device=None):
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if ndim is not None and x.dim() not in ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {x.dim()}")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, expected {device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_size(num_seqs: int, total_tokens: int, H: int, d: int, chunk_size: int,
                   dtype: torch.dtype) -> int:
    return int(library().kda_chunk_fwd_workspace_size(num_seqs, total_tokens, H, d, d,
                                                      chunk_size, _DTYPES[dtype]))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              output_final_state: bool = True, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill (kda_chunk_fwd).

    q, k [N_tok, H, d_k] or [B, T, H, d_k]; v like q with d_v; g like q (fp32);
    beta [N_tok, H] or [B, T, H] (fp32); initial_state [N, H, d_k, d_v] fp32 or
    None; cu_seqlens int32 [N + 1] on the device or None (one sequence per
    batch row).  Returns (o shaped like v, final_state [N, H, d_k, d_v] fp32 or
    None).  ``out`` / ``final_state`` may be passed preallocated.
    """
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be bf16 or fp32, got {q.dtype}")
    dev = q.device
    _need(q, "q", ndim=(3, 4))
    for name, x in (("k", k), ("v", v)):
        _need(x, name, dtype=q.dtype, ndim=(q.dim(),), device=dev)
    _need(g, "g", dtype=torch.float32, ndim=(q.dim(),), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(q.dim() - 1,), device=dev)
    if q.dim() == 4:
        B, T = q.shape[:2]
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is only accepted with packed 3-D inputs")
        num_seqs, n_tok = B, B * T
    else:
        n_tok = q.shape[0]
        if cu_seqlens is None:
            num_seqs = 1
        else:
            _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=(1,), device=dev)
            num_seqs = cu_seqlens.shape[0] - 1
    H, dk = q.shape[-2:]
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:-1] != q.shape[:-1]:
        raise ValueError("q, k, g must share a shape and v must match it up to d_v")
    if beta.shape != q.shape[:-1]:
        raise ValueError(f"beta must have shape {tuple(q.shape[:-1])}")
    sshape = (num_seqs, H, dk, dv)
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, device=dev)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must have shape {sshape}")
    if out is None:
        out = torch.empty_like(v)
    else:
        _need(out, "out", dtype=v.dtype, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", dtype=torch.float32, device=dev)
    ws_bytes = workspace_size(num_seqs, n_tok, H, dk, chunk_size, q.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    lib = library()
    st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), num_seqs, n_tok, H, dk, dv, chunk_size,
                           _DTYPES[q.dtype], _ptr(out), _ptr(final_state), _ptr(ws), ws_bytes,
                           _stream(dev))
    _check("kda_chunk_fwd", st)
    return out, final_state


def step_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step (kda_step_decode).  q, k, g [N, H, d_k]; v [N, H, d_v];
    beta [N, H]; state [N, H, d_k, d_v] fp32 is updated in place.  Returns o."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be bf16 or fp32, got {q.dtype}")
    dev = q.device
    _need(q, "q", ndim=(3,))
    _need(k, "k", dtype=q.dtype, ndim=(3,), device=dev)
    _need(v, "v", dtype=q.dtype, ndim=(3,), device=dev)
    _need(g, "g", dtype=torch.float32, ndim=(3,), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(2,), device=dev)
    _need(state, "state", dtype=torch.float32, ndim=(4,), device=dev)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:2]) != (N, H):
        raise ValueError("q, k, g must share a shape and v must match it up to d_v")
    if tuple(beta.shape) != (N, H) or tuple(state.shape) != (N, H, dk, dv):
        raise ValueError("beta must be [N, H] and state [N, H, d_k, d_v]")
    if out is None:
        out = torch.empty_like(v)
    st = library().kda_step_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                   _ptr(out), N, H, dk, dv, _DTYPES[q.dtype], _stream(dev))
    _check("kda_step_decode", st)
    return out
