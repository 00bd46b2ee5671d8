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
KDA_FUSE_GATE, KDA_FUSE_L2NORM = 1, 2
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}
# prefill algorithms (kda_algo)
ALGOS = {"auto": 0, "fused": 1, "two_pass": 2}
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
    lib.kda_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                     i32, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_ex.restype = i32
    lib.kda_chunk_fwd_algo_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32]
    lib.kda_chunk_fwd_algo_workspace_size.restype = sz
    lib.kda_chunk_fwd_algo.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                       i32, i32, i32, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_algo.restype = i32
    lib.kda_chunk_fwd_two_pass_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                                  i32, i32, i32, i32, vp, vp, vp]
    lib.kda_chunk_fwd_two_pass_static.restype = i32
    lib.kda_chunk_fwd_static_scratch_bytes.argtypes = []
    lib.kda_chunk_fwd_static_scratch_bytes.restype = sz
    lib.kda_step_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_step_decode.restype = i32
    lib.kda_step_decode_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp,
                                          i32, i32, i32, i32, i32, vp]
    lib.kda_step_decode_gated.restype = i32
    lib.kda_segment_scan.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.kda_segment_scan.restype = i32
    lib.kda_kcp_summaries.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, vp, vp, vp]
    lib.kda_kcp_summaries.restype = i32
    lib.kda_chunk_fwd_fused_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                           i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_fused_ex.restype = i32
    lib.kda_front_end.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.kda_front_end.restype = i32
    lib.kda_short_conv_ex.argtypes = [vp, vp, vp, i32, i64, i32, vp, vp, i32, i32, vp]
    lib.kda_short_conv_ex.restype = i32
    lib.kda_chunk_fwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                        i32, i32, i32, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_fused.restype = i32
    lib.kda_output_gate.argtypes = [vp, vp, vp, ctypes.c_float, vp, i64, i32, i32, vp]
    lib.kda_output_gate.restype = i32
    lib.kda_output_gate_ex.argtypes = [vp, i32, vp, vp, ctypes.c_float, vp, i32, i64, i32, i32, vp]
    lib.kda_output_gate_ex.restype = i32
    lib.kda_short_conv.argtypes = [vp, vp, vp, i32, i64, i32, vp, vp, i32, vp]
    lib.kda_short_conv.restype = i32
    lib.kda_state_compose.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp]
    lib.kda_state_compose.restype = i32
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


def _gpu(dev: torch.device):
    """The kernels take device pointers: refuse tensors that are not on a GPU."""
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {dev}")


def _out(out: Optional[torch.Tensor], shape, dtype, dev, name: str = "out") -> torch.Tensor:
    """A new output tensor, or the caller's after checking it matches exactly
    (the kernels write every element of the expected shape)."""
    if out is None:
        return torch.empty(tuple(shape), dtype=dtype, device=dev)
    _need(out, name, dtype=dtype, device=dev)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    return out


def workspace_size(num_seqs: int, total_tokens: int, H: int, d: int, chunk_size: int,
                   dtype: torch.dtype, algo: str = "auto") -> int:
    if algo not in ALGOS:
        raise ValueError(f"algo must be one of {sorted(ALGOS)}, got {algo!r}")
    return int(library().kda_chunk_fwd_algo_workspace_size(num_seqs, total_tokens, H, d, d,
                                                           chunk_size, _DTYPES[dtype], ALGOS[algo]))


def chunk_fwd(q: Optional[torch.Tensor], k: torch.Tensor, v: Optional[torch.Tensor],
              g: torch.Tensor, beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              output_final_state: bool = True, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, output: bool = True,
              o_dtype: Optional[torch.dtype] = None, algo: str = "auto",
              workspace: Optional[torch.Tensor] = None
              ) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Chunkwise KDA prefill (kda_chunk_fwd_algo).

    q, k [N_tok, H, d_k] or [B, T, H, d_k]; v like q with d_v; g like q (fp32);
    beta [N_tok, H] or [B, T, H] (fp32); initial_state [N, H, d_k, d_v] fp32 or
    None; cu_seqlens int32 [N + 1] on the device or None (one sequence per
    batch row).  Returns (o shaped like v, final_state [N, H, d_k, d_v] fp32 or
    None).  ``out`` / ``final_state`` may be passed preallocated.

    output=False computes only the final states (o is None and q may be None);
    v=None stands for zero values (d_v = d_k).  o_dtype=torch.float32 with bf16
    inputs writes o in fp32 (None: the input dtype).  algo is "auto", "fused"
    or "two_pass" (kda_algo); the two-pass path's workspace is allocated here
    unless a large enough uint8 ``workspace`` tensor is given.
    """
    if not output and not output_final_state and final_state is None:
        raise ValueError("nothing to compute: output=False needs the final state")
    if output and q is None:
        raise ValueError("q is required when the output is computed")
    if algo not in ALGOS:
        raise ValueError(f"algo must be one of {sorted(ALGOS)}, got {algo!r}")
    if k.dtype not in _DTYPES:
        raise ValueError(f"k must be bf16 or fp32, got {k.dtype}")
    dev = k.device
    _gpu(dev)
    _need(k, "k", ndim=(3, 4))
    if q is not None:
        _need(q, "q", dtype=k.dtype, ndim=(k.dim(),), device=dev)
    if v is not None:
        _need(v, "v", dtype=k.dtype, ndim=(k.dim(),), device=dev)
    _need(g, "g", dtype=torch.float32, ndim=(k.dim(),), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(k.dim() - 1,), device=dev)
    if k.dim() == 4:
        B, T = k.shape[:2]
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is only accepted with packed 3-D inputs")
        num_seqs, n_tok = B, B * T
    else:
        n_tok = k.shape[0]
        if cu_seqlens is None:
            num_seqs = 1
        else:
            _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=(1,), device=dev)
            num_seqs = cu_seqlens.shape[0] - 1
    H, dk = k.shape[-2:]
    dv = dk if v is None else v.shape[-1]
    if (q is not None and q.shape != k.shape) or g.shape != k.shape or \
            (v is not None and v.shape[:-1] != k.shape[:-1]):
        raise ValueError("q, k, g must share a shape and v must match it up to d_v")
    if beta.shape != k.shape[:-1]:
        raise ValueError(f"beta must have shape {tuple(k.shape[:-1])}")
    sshape = (num_seqs, H, dk, dv)
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, device=dev)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must have shape {sshape}")
    odt = k.dtype if o_dtype is None else o_dtype
    if odt not in (k.dtype, torch.float32):
        raise ValueError(f"o_dtype must be {k.dtype} or torch.float32, got {o_dtype}")
    out = _out(out, k.shape[:-1] + (dv,), odt, dev) if output else None
    if final_state is not None or output_final_state:
        final_state = _out(final_state, sshape, torch.float32, dev, "final_state")
    ws_bytes = workspace_size(num_seqs, n_tok, H, dk, chunk_size, k.dtype, algo)
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=(1,), device=dev)
        if workspace.numel() < ws_bytes:
            raise ValueError(f"workspace must hold {ws_bytes} bytes, got {workspace.numel()}")
        ws, ws_bytes = workspace, workspace.numel()
    else:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = library().kda_chunk_fwd_algo(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(initial_state), _ptr(cu_seqlens), num_seqs, n_tok, H,
                                      dk, dv, chunk_size, _DTYPES[k.dtype], _DTYPES[odt],
                                      ALGOS[algo], _ptr(out), _ptr(final_state), _ptr(ws),
                                      ws_bytes, _stream(dev))
    _check("kda_chunk_fwd_algo", st)
    return out, final_state


def chunk_fwd_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                     beta: torch.Tensor, initial_state: Optional[torch.Tensor],
                     cu_seqlens: Optional[torch.Tensor], out: torch.Tensor,
                     final_state: torch.Tensor, chunk_size: int = 64) -> None:
    """The two-pass prefill on the library's static scratch
    (kda_chunk_fwd_two_pass_static): no device allocation here or in the
    library.  Packed 3-D inputs as chunk_fwd; ``out`` (o, dtype of the inputs or
    fp32) and ``final_state`` must be preallocated."""
    if k.dtype not in _DTYPES:
        raise ValueError(f"k must be bf16 or fp32, got {k.dtype}")
    dev = k.device
    _gpu(dev)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(x, name, dtype=k.dtype, ndim=(3,), device=dev)
    _need(g, "g", dtype=torch.float32, ndim=(3,), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(2,), device=dev)
    num_seqs, n_tok = _layout(k, cu_seqlens)
    H, dk = k.shape[-2:]
    dv = v.shape[-1]
    if q.shape != k.shape or g.shape != k.shape or v.shape[:-1] != k.shape[:-1] or \
            beta.shape != k.shape[:-1]:
        raise ValueError("q, k, g must share a shape; v and beta must match it")
    sshape = (num_seqs, H, dk, dv)
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, device=dev)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must have shape {sshape}")
    if out.dtype not in (k.dtype, torch.float32):
        raise ValueError(f"out must be {k.dtype} or torch.float32")
    _out(out, v.shape, out.dtype, dev)
    _out(final_state, sshape, torch.float32, dev, "final_state")
    st = library().kda_chunk_fwd_two_pass_static(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
        num_seqs, n_tok, H, dk, dv, chunk_size, _DTYPES[k.dtype], _DTYPES[out.dtype], _ptr(out),
        _ptr(final_state), _stream(dev))
    _check("kda_chunk_fwd_two_pass_static", st)


def step_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step (kda_step_decode).  q, k, g [N, H, d_k]; v [N, H, d_v];
    beta [N, H]; state [N, H, d_k, d_v] fp32 is updated in place.  Returns o."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be bf16 or fp32, got {q.dtype}")
    dev = q.device
    _gpu(dev)
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
    out = _out(out, v.shape, v.dtype, dev)
    st = library().kda_step_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                   _ptr(out), N, H, dk, dv, _DTYPES[q.dtype], _stream(dev))
    _check("kda_step_decode", st)
    return out


def step_decode_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, state: torch.Tensor, gate: torch.Tensor,
                      weight: torch.Tensor, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                      o_raw: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step with the output epilogue fused in (kda_step_decode_gated):
    returns RMSNorm(o) * sigmoid(gate); ``state`` is updated in place and the raw
    o is written to ``o_raw`` when given.  Shapes as step_decode; gate like v;
    weight [d_v] fp32."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q must be bf16 or fp32, got {q.dtype}")
    dev = q.device
    _gpu(dev)
    _need(q, "q", ndim=(3,))
    for name, x in (("k", k), ("v", v), ("gate", gate)):
        _need(x, name, dtype=q.dtype, ndim=(3,), device=dev)
    _need(g, "g", dtype=torch.float32, ndim=(3,), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(2,), device=dev)
    _need(state, "state", dtype=torch.float32, ndim=(4,), device=dev)
    _need(weight, "weight", dtype=torch.float32, ndim=(1,), device=dev)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or tuple(v.shape[:2]) != (N, H) or \
            gate.shape != v.shape or tuple(weight.shape) != (dv,):
        raise ValueError("q, k, g must share a shape; v and gate [N, H, d_v]; weight [d_v]")
    if tuple(beta.shape) != (N, H) or tuple(state.shape) != (N, H, dk, dv):
        raise ValueError("beta must be [N, H] and state [N, H, d_k, d_v]")
    out = _out(out, v.shape, v.dtype, dev)
    if o_raw is not None:
        _out(o_raw, v.shape, v.dtype, dev, "o_raw")
    st = library().kda_step_decode_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                         _ptr(state), _ptr(gate), _ptr(weight), float(eps),
                                         _ptr(out), _ptr(o_raw), N, H, dk, dv, _DTYPES[q.dtype],
                                         _stream(dev))
    _check("kda_step_decode_gated", st)
    return out


def _layout(q: torch.Tensor, cu_seqlens: Optional[torch.Tensor]):
    """(num_seqs, n_tok) of packed 3-D or batched 4-D token-major inputs."""
    if q.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is only accepted with packed 3-D inputs")
        return q.shape[0], q.shape[0] * q.shape[1]
    if cu_seqlens is None:
        return 1, q.shape[0]
    _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=(1,), device=q.device)
    return cu_seqlens.shape[0] - 1, q.shape[0]


def chunk_fwd_fused(q_raw: torch.Tensor, k_raw: torch.Tensor, v: torch.Tensor, z: torch.Tensor,
                    A_log: torch.Tensor, b_alpha: torch.Tensor, beta: torch.Tensor,
                    initial_state: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                    output_final_state: bool = True, l2norm: bool = True,
                    out: Optional[torch.Tensor] = None,
                    final_state: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Prefill with the front end fused in (kda_chunk_fwd_fused_ex):
    g = -5 sigma(e^{A_h} (z + b_alpha^h)) in the kernel, and with l2norm=True
    q, k L2-normalised there too (else q_raw, k_raw must be normalised
    already, e.g. by front_end).  q_raw, k_raw, z like q of chunk_fwd (same
    dtype); A_log [H] fp32; b_alpha [H, d_k] fp32; the rest as chunk_fwd."""
    if q_raw.dtype not in _DTYPES:
        raise ValueError(f"q_raw must be bf16 or fp32, got {q_raw.dtype}")
    dev = q_raw.device
    _gpu(dev)
    _need(q_raw, "q_raw", ndim=(3, 4))
    for name, x in (("k_raw", k_raw), ("v", v), ("z", z)):
        _need(x, name, dtype=q_raw.dtype, ndim=(q_raw.dim(),), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(q_raw.dim() - 1,), device=dev)
    num_seqs, n_tok = _layout(q_raw, cu_seqlens)
    H, dk = q_raw.shape[-2:]
    dv = v.shape[-1]
    if k_raw.shape != q_raw.shape or z.shape != q_raw.shape or v.shape[:-1] != q_raw.shape[:-1]:
        raise ValueError("q_raw, k_raw, z must share a shape and v must match it up to d_v")
    if beta.shape != q_raw.shape[:-1]:
        raise ValueError(f"beta must have shape {tuple(q_raw.shape[:-1])}")
    _need(A_log, "A_log", dtype=torch.float32, ndim=(1,), device=dev)
    _need(b_alpha, "b_alpha", dtype=torch.float32, ndim=(2,), device=dev)
    if tuple(A_log.shape) != (H,) or tuple(b_alpha.shape) != (H, dk):
        raise ValueError("A_log must be [H] and b_alpha [H, d_k]")
    sshape = (num_seqs, H, dk, dv)
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, device=dev)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must have shape {sshape}")
    out = _out(out, v.shape, v.dtype, dev)
    if output_final_state:
        final_state = _out(final_state, sshape, torch.float32, dev, "final_state")
    else:
        final_state = None
    fuse = KDA_FUSE_GATE | (KDA_FUSE_L2NORM if l2norm else 0)
    st = library().kda_chunk_fwd_fused_ex(
        _ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(z), _ptr(A_log), _ptr(b_alpha), _ptr(beta),
        _ptr(initial_state), _ptr(cu_seqlens), num_seqs, n_tok, H, dk, dv, chunk_size,
        _DTYPES[q_raw.dtype], fuse, _ptr(out), _ptr(final_state), None, 0, _stream(dev))
    _check("kda_chunk_fwd_fused_ex", st)
    return out, final_state


def front_end(q_raw: torch.Tensor, k_raw: torch.Tensor, z: Optional[torch.Tensor] = None,
              A_log: Optional[torch.Tensor] = None, b_alpha: Optional[torch.Tensor] = None,
              q: Optional[torch.Tensor] = None, k: Optional[torch.Tensor] = None,
              g: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """The front end as a pass of its own (kda_front_end): q = L2Norm(q_raw),
    k = L2Norm(k_raw) and, when z is given, the fp32 log-decay
    g = -5 sigma(e^{A_h} (z + b_alpha^h)).  q_raw, k_raw, z [..., H, d]."""
    if q_raw.dtype not in _DTYPES:
        raise ValueError(f"q_raw must be bf16 or fp32, got {q_raw.dtype}")
    dev = q_raw.device
    _gpu(dev)
    _need(q_raw, "q_raw", ndim=(3, 4))
    _need(k_raw, "k_raw", dtype=q_raw.dtype, ndim=(q_raw.dim(),), device=dev)
    if k_raw.shape != q_raw.shape:
        raise ValueError("q_raw and k_raw must share a shape")
    H, d = q_raw.shape[-2:]
    n_tok = q_raw.numel() // (H * d)
    if z is not None:
        _need(z, "z", dtype=q_raw.dtype, device=dev)
        _need(A_log, "A_log", dtype=torch.float32, ndim=(1,), device=dev)
        _need(b_alpha, "b_alpha", dtype=torch.float32, ndim=(2,), device=dev)
        if z.shape != q_raw.shape or tuple(A_log.shape) != (H,) or tuple(b_alpha.shape) != (H, d):
            raise ValueError("z like q_raw, A_log [H], b_alpha [H, d]")
        g = _out(g, q_raw.shape, torch.float32, dev, "g")
    else:
        g = None
    q = _out(q, q_raw.shape, q_raw.dtype, dev, "q")
    k = _out(k, q_raw.shape, q_raw.dtype, dev, "k")
    st = library().kda_front_end(_ptr(q_raw), _ptr(k_raw), _ptr(z), _ptr(A_log), _ptr(b_alpha),
                                 n_tok, H, d, _DTYPES[q_raw.dtype], _ptr(q), _ptr(k), _ptr(g),
                                 _stream(dev))
    _check("kda_front_end", st)
    return q, k, g


def output_gate(o_raw: torch.Tensor, gate: torch.Tensor, weight: torch.Tensor,
                eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """RMSNorm(o_raw) * sigmoid(gate) over the last axis (kda_output_gate;
    kda_output_gate_ex when o_raw or the result is fp32 and the gate bf16).

    The gate's dtype is the data type; o_raw may be that or fp32, and the
    result out_dtype (None: o_raw's dtype) that or fp32.
    """
    _need(gate, "gate")
    if gate.dtype not in _DTYPES:
        raise ValueError(f"gate must be bf16 or fp32, got {gate.dtype}")
    dt = gate.dtype
    _need(o_raw, "o_raw")
    if o_raw.dtype not in (dt, torch.float32):
        raise ValueError(f"o_raw must be {dt} or torch.float32, got {o_raw.dtype}")
    odt = o_raw.dtype if out_dtype is None else out_dtype
    if odt not in (dt, torch.float32):
        raise ValueError(f"out_dtype must be {dt} or torch.float32, got {out_dtype}")
    dev = gate.device
    _gpu(dev)
    _need(o_raw, "o_raw", device=dev)
    _need(weight, "weight", dtype=torch.float32, ndim=(1,), device=dev)
    dv = o_raw.shape[-1]
    if gate.shape != o_raw.shape or tuple(weight.shape) != (dv,):
        raise ValueError("gate must match o_raw and weight must be [d_v]")
    out = _out(out, o_raw.shape, odt, dev)
    if o_raw.dtype == dt and odt == dt:
        st = library().kda_output_gate(_ptr(o_raw), _ptr(gate), _ptr(weight), float(eps),
                                       _ptr(out), o_raw.numel() // dv, dv, _DTYPES[dt],
                                       _stream(dev))
        _check("kda_output_gate", st)
    else:
        st = library().kda_output_gate_ex(_ptr(o_raw), _DTYPES[o_raw.dtype], _ptr(gate),
                                          _ptr(weight), float(eps), _ptr(out), _DTYPES[odt],
                                          o_raw.numel() // dv, dv, _DTYPES[dt], _stream(dev))
        _check("kda_output_gate_ex", st)
    return out


def short_conv(x: torch.Tensor, weight: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
               conv_state: Optional[torch.Tensor] = None, num_seqs: Optional[int] = None,
               l2norm_d: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal 4-tap depthwise convolution (kda_short_conv_ex).  x [N_tok, C]
    (packed; one sequence, ``num_seqs`` equal ones, or cu_seqlens); weight
    [C, 4] fp32; conv_state [N, 3, C] fp32 is read and updated in place.
    l2norm_d > 0: each output row of l2norm_d channels (a head) is then
    L2-normalised."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"x must be bf16 or fp32, got {x.dtype}")
    dev = x.device
    _gpu(dev)
    _need(x, "x", ndim=(2,))
    _need(weight, "weight", dtype=torch.float32, ndim=(2,), device=dev)
    n_tok, C = x.shape
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=(1,), device=dev)
        nseq = cu_seqlens.shape[0] - 1
    else:
        nseq = 1 if num_seqs is None else int(num_seqs)
    if tuple(weight.shape) != (C, 4):
        raise ValueError("weight must be [C, 4]")
    if conv_state is not None:
        _need(conv_state, "conv_state", dtype=torch.float32, device=dev)
        if tuple(conv_state.shape) != (nseq, 3, C):
            raise ValueError(f"conv_state must be {(nseq, 3, C)}")
    y = _out(out, x.shape, x.dtype, dev)
    st = library().kda_short_conv_ex(_ptr(x), _ptr(weight), _ptr(cu_seqlens), nseq, n_tok, C,
                                     _ptr(conv_state), _ptr(y), _DTYPES[x.dtype], int(l2norm_d),
                                     _stream(dev))
    _check("kda_short_conv_ex", st)
    return y


def state_compose(M: torch.Tensor, S_in: torch.Tensor, S_tilde: torch.Tensor,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S_out = M @ S_in + S_tilde over a batch of fp32 matrices (kda_state_compose)."""
    dev = M.device
    _gpu(dev)
    for name, x in (("M", M), ("S_in", S_in), ("S_tilde", S_tilde)):
        _need(x, name, dtype=torch.float32, device=dev)
    d = M.shape[-1]
    if M.shape[-2] != d or S_in.shape != S_tilde.shape or S_in.shape[:-2] != M.shape[:-2] \
            or S_in.shape[-2] != d:
        raise ValueError("M must be [..., d, d] and S_in, S_tilde [..., d, d_v]")
    out = _out(out, S_in.shape, torch.float32, dev)
    count = M.numel() // (d * d)
    st = library().kda_state_compose(_ptr(M), _ptr(S_in), _ptr(S_tilde), _ptr(out), count, d,
                                     S_in.shape[-1], _stream(dev))
    _check("kda_state_compose", st)
    return out


def kcp_summaries(q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, cu_seqlens: torch.Tensor
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-segment summaries (M, S~) of packed segments: M from S = I with zero
    values, S~ from S = 0 (d_v = d_k).  One kda_kcp_summaries launch where it
    supports the shape (bf16, or fp32 up to d = 64); fp32 at d = 128 takes two
    state-only kda_chunk_fwd calls instead.  q is not needed.
    Returns ([P, H, d, d], [P, H, d, d_v])."""
    P = cu_seqlens.shape[0] - 1
    dev = k.device
    _gpu(dev)
    _need(k, "k", ndim=(3,))
    H, dk = k.shape[-2:]
    if k.dtype == torch.float32 and dk > 64:
        _, S_t = chunk_fwd(None, k, v, g, beta, cu_seqlens=cu_seqlens, output=False)
        eye = torch.eye(dk, dtype=torch.float32, device=dev).expand(P, H, dk, dk).contiguous()
        _, M = chunk_fwd(None, k, None, g, beta, initial_state=eye, cu_seqlens=cu_seqlens,
                         output=False)
        return M, S_t
    if k.dtype not in _DTYPES:
        raise ValueError(f"k must be bf16 or fp32, got {k.dtype}")
    _need(v, "v", dtype=k.dtype, ndim=(3,), device=dev)
    _need(g, "g", dtype=torch.float32, ndim=(3,), device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=(2,), device=dev)
    _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=(1,), device=dev)
    n = k.shape[0]
    if v.shape != k.shape or g.shape != k.shape or tuple(beta.shape) != (n, H):
        raise ValueError("k, v, g must be [N_tok, H, d] and beta [N_tok, H]")
    M = torch.empty((P, H, dk, dk), dtype=torch.float32, device=dev)
    S_t = torch.empty_like(M)
    st = library().kda_kcp_summaries(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), P, n,
                                     H, dk, 64, _DTYPES[k.dtype], _ptr(M), _ptr(S_t), _stream(dev))
    _check("kda_kcp_summaries", st)
    return M, S_t


def kcp_scan(M: torch.Tensor, S_tilde: torch.Tensor, S0: Optional[torch.Tensor] = None,
             S_in: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor]:
    """States entering each segment and the final state, one kda_segment_scan
    launch: S_in[0] = S0 (or 0), S_in[r + 1] = M[r] S_in[r] + S~[r].
    M, S_tilde [P, H, d, d] fp32; S0 [H, d, d] fp32 or None."""
    _need(M, "M", dtype=torch.float32, ndim=(4,))
    dev = M.device
    _gpu(dev)
    _need(S_tilde, "S_tilde", dtype=torch.float32, ndim=(4,), device=dev)
    P, H, d = M.shape[:3]
    if tuple(M.shape) != (P, H, d, d) or S_tilde.shape != M.shape:
        raise ValueError("M and S_tilde must both be [P, H, d, d]")
    if S0 is not None:
        _need(S0, "S0", dtype=torch.float32, ndim=(3,), device=dev)
        if tuple(S0.shape) != (H, d, d):
            raise ValueError(f"S0 must be [{H}, {d}, {d}]")
    S_in = _out(S_in, M.shape, torch.float32, dev, "S_in")
    S_final = _out(S_final, (H, d, d), torch.float32, dev, "S_final")
    st = library().kda_segment_scan(_ptr(M), _ptr(S_tilde), _ptr(S0), _ptr(S_in), _ptr(S_final),
                                    P, H, d, _stream(dev))
    _check("kda_segment_scan", st)
    return S_in, S_final
