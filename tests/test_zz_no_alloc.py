"""The no-allocation prefill (kda_chunk_fwd_two_pass_static) against the
two-pass prefill with a caller workspace (kda_chunk_fwd_algo, KDA_ALGO_TWO_PASS).

The static entry point is for callers that cannot allocate device memory; it
runs the same kernels on the library's static scratch, so its results must equal
the workspace call's bit for bit.  Two calls in a row (the second smaller, the
scratch keeping the first call's contents) and a call too large for the scratch
(refused on the host).
"""
import ctypes

import pytest
import torch

from linear_attention_recurrence_chunk_amd import _lib as kda
from linear_attention_recurrence_chunk_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
KDA_ERR_TOO_LARGE = 7


def _both(w, seed, chunk, o_dtype=None):
    x = inputs.prefill_inputs(w, seed=seed, device=DEV)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    o_ref, s_ref = kda.chunk_fwd(*args, chunk_size=chunk, algo="two_pass", o_dtype=o_dtype)
    out = torch.full_like(o_ref, float("nan"))
    fs = torch.full_like(s_ref, float("nan"))
    kda.chunk_fwd_static(*args, out=out, final_state=fs, chunk_size=chunk)
    torch.cuda.synchronize()
    return (out, fs), (o_ref, s_ref)


def test_static_scratch_equals_workspace_call_twice():
    big = inputs.custom(H=8, dk=128, dv=128, seqlens=[700, 0, 300, 65], state_std=0.05)
    small = inputs.custom(H=2, dk=64, dv=64, seqlens=[70], state_std=0.05)
    for w, seed, chunk in ((big, 1, 64), (small, 2, 64)):
        (o, s), (o_ref, s_ref) = _both(w, seed, chunk)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), (w.H, w.dk)


def test_static_scratch_other_types_and_chunk():
    w128 = inputs.custom(H=4, dk=128, dv=128, seqlens=[300, 129], state_std=0.05)
    (o, s), (o_ref, s_ref) = _both(w128, 3, 128)
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    (o, s), (o_ref, s_ref) = _both(w128, 4, 64, o_dtype=torch.float32)
    assert o.dtype == torch.float32 and torch.equal(o, o_ref) and torch.equal(s, s_ref)
    w32 = inputs.custom(H=3, dk=128, dv=128, seqlens=[190, 1], state_std=0.1, dtype=torch.float32)
    (o, s), (o_ref, s_ref) = _both(w32, 5, 64)
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_static_scratch_refuses_sizes_beyond_it():
    lib = kda.library()
    cap = lib.kda_chunk_fwd_static_scratch_bytes()
    assert cap == 256 << 20
    # one 8K-token sequence of 96 heads needs more than the scratch
    need = kda.workspace_size(1, 8192, 96, 128, 64, torch.bfloat16, "two_pass")
    assert need > cap
    A = ctypes.c_void_p(0x10000)   # never dereferenced: the size check comes first
    st = lib.kda_chunk_fwd_two_pass_static(A, A, A, A, A, None, None, 1, 8192, 96, 128, 128, 64,
                                           1, 1, A, None, None)
    assert st == KDA_ERR_TOO_LARGE
    assert b"static scratch" in lib.kda_status_string(st)
