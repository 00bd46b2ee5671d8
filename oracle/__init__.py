"""Oracle for the Kimi Delta Attention (KDA) recurrence: fp64, CPU, sequential.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

Two independent implementations live here:

* ``kda_ref.c`` (built into ``libkda_oracle.so`` with gcc, threaded over
  (sequence, head)) evaluates one token at a time: decay, read, delta
  correction, rank-one write, output.  This is what the parity tests compare
  the GPU against.
* ``numpy_ref.py`` multiplies out the explicit d_k x d_k transition matrix
  M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) of the page "Notations
  mathematiques" (table "Attention et KDA", row M_t).  It is only for tiny
  shapes and serves to cross-check the C code.
* ``layer_ref.py`` holds the steps around the recurrence in a KDA layer, in
  numpy float64: L2Norm of q and k, the bounded gate that turns decay logits
  into g, the causal ShortConv with its streaming state, RMSNorm and the
  sigmoid output gate, and the segment summaries (transition product, state
  from zero) with their composition.

The recurrence (same page and table, rows S_t, alpha_t, g_t, o~_t):
    S_t = M_t S_{t-1} + beta_t k_t v_t^T,   alpha_t = exp(g_t),   o_t = S_t^T q_t.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_ref.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build_oracle(force: bool = True) -> str:
    """Compile kda_ref.c with gcc into libkda_oracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_oracle()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        lib.kda_oracle_forward_f64.argtypes = [dp, dp, dp, dp, dp, dp, lp,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, dp, dp, ctypes.c_int]
        lib.kda_oracle_forward_f64.restype = ctypes.c_int
        lib.kda_oracle_decode_f64.argtypes = [dp, dp, dp, dp, dp, dp,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, dp, ctypes.c_int]
        lib.kda_oracle_decode_f64.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact upcast to a contiguous fp64 numpy array (bf16/fp32 torch or numpy)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: bf16 and fp32 both upcast exactly
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
            nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Run the recurrence over packed sequences.

    Shapes: q, k, g [N_tok, H, dk] (or [B, T, H, dk] for B equal-length
    sequences); v [.., H, dv]; beta [N_tok, H] (or [B, T, H]); initial_state
    [N, H, dk, dv] or None (zeros); cu_seqlens [N + 1] or None (one sequence,
    or B equal ones for 4-D inputs).  Returns (o, final_state) in fp64 with o
    shaped like v.
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    out_shape = v.shape
    if q.ndim == 4:
        B, T = q.shape[:2]
        q, k, v, g = (x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g))
        beta = beta.reshape(B * T, -1)
        if cu_seqlens is None:
            cu_seqlens = np.arange(B + 1, dtype=np.int64) * T
    n_tok, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, n_tok], dtype=np.int64)
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    if cu[-1] != n_tok:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    for name, x, shp in (("k", k, (n_tok, H, dk)), ("g", g, (n_tok, H, dk)),
                         ("v", v, (n_tok, H, dv)), ("beta", beta, (n_tok, H))):
        if x.shape != shp:
            raise ValueError(f"{name} has shape {x.shape}, expected {shp}")
    s0 = _f64(initial_state)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError(f"initial_state has shape {s0.shape}, expected {(N, H, dk, dv)}")
    o = np.zeros((n_tok, H, dv), dtype=np.float64)
    sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_forward_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        N, H, dk, dv, _ptr(o), _ptr(sf), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle forward failed with code {rc}")
    return o.reshape(out_shape), sf


def decode(q, k, v, g, beta, state, nthreads: Optional[int] = None):
    """One token per request.  q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H];
    state [N, H, dk, dv].  Returns (o [N, H, dv], new_state), both fp64; the
    input state is not modified."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    st = np.array(_f64(state), dtype=np.float64, copy=True, order="C")
    N, H, dk = q.shape
    dv = v.shape[-1]
    if st.shape != (N, H, dk, dv):
        raise ValueError(f"state has shape {st.shape}, expected {(N, H, dk, dv)}")
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().kda_oracle_decode_f64(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(st),
        N, H, dk, dv, _ptr(o), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle decode failed with code {rc}")
    return o, st
