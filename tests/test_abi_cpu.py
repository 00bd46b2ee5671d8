"""The C ABI library loads without a GPU, exports what include/kda.h declares,
and rejects invalid arguments on the host before any HIP call.

Invalid calls use fake, never-dereferenced device addresses: every call below
must return its status from host-side validation.  They are skipped where a
GPU is visible, so that a validation bug can never launch a kernel on them.
"""
import ctypes
import os
import re

import pytest

from linear_attention_recurrence_chunk_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP = range(7)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.library()
    names = _declared_functions()
    assert names == sorted(["kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_step_decode",
                            "kda_status_string", "kda_version", "kda_chunk_fwd_fused",
                            "kda_output_gate", "kda_short_conv", "kda_state_compose",
                            "kda_chunk_fwd_ex", "kda_output_gate_ex"])
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_version_and_status_strings():
    lib = _lib.library()
    assert lib.kda_version() == 1
    for s in range(7):
        assert lib.kda_status_string(s)
    assert lib.kda_status_string(99) == b"unknown status"


def test_workspace_size_is_zero_for_fused_kernel():
    assert _lib.library().kda_chunk_fwd_workspace_size(16, 100000, 96, 128, 128, 64, 1) == 0


gpu_visible = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="fake-pointer validation tests run only where no GPU is visible")

A = 0x10000        # aligned fake address (never dereferenced)
MIS = 0x10004      # 4-byte aligned only


def _fwd(**kw):
    a = dict(q=A, k=A, v=A, g=A, beta=A, s0=None, cu=None, num_seqs=1, total=128, H=2,
             dk=64, dv=64, chunk=64, dt=1, o=A, sf=None, ws=None, ws_bytes=0)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.library().kda_chunk_fwd(
        p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]), p(a["cu"]),
        a["num_seqs"], a["total"], a["H"], a["dk"], a["dv"], a["chunk"], a["dt"], p(a["o"]),
        p(a["sf"]), p(a["ws"]), a["ws_bytes"], None)


def _dec(**kw):
    a = dict(q=A, k=A, v=A, g=A, beta=A, state=A, o=A, N=4, H=2, dk=64, dv=64, dt=1)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.library().kda_step_decode(
        p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["state"]), p(a["o"]),
        a["N"], a["H"], a["dk"], a["dv"], a["dt"], None)


@gpu_visible
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ENULL), (dict(k=None), ENULL), (dict(g=None), ENULL),
    (dict(beta=None), ENULL),
    (dict(o=None), ENULL),                           # no output and no final state
    (dict(o=None, q=None), ENULL),                   # likewise (v = NULL alone is valid: zero values)
    (dict(total=-1), ESHAPE), (dict(num_seqs=-1), ESHAPE), (dict(H=0), ESHAPE),
    (dict(num_seqs=3, total=128), ESHAPE),           # equal lengths need a multiple
    (dict(num_seqs=0, total=5), ESHAPE),
    (dict(dk=48, dv=48), EUNSUP), (dict(dk=64, dv=128), EUNSUP), (dict(dk=256, dv=256), EUNSUP),
    (dict(chunk=32), EUNSUP), (dict(chunk=96), EUNSUP), (dict(chunk=256), EUNSUP), (dict(dt=7), EUNSUP),
    (dict(dt=0, dk=128, dv=128), EUNSUP),            # fp32 path is for d <= 64
    (dict(H=32768, dk=128, dv=128), ESHAPE),         # a token's g row must stay below 16 MiB
    (dict(q=MIS), EALIGN), (dict(g=MIS), EALIGN), (dict(o=MIS), EALIGN),
    (dict(s0=MIS), EALIGN), (dict(sf=MIS), EALIGN), (dict(cu=MIS), EALIGN),
])
def test_chunk_fwd_rejects(kw, status):
    assert _fwd(**kw) == status


@gpu_visible
def test_chunk_fwd_empty_batch_is_a_no_op():
    assert _fwd(num_seqs=0, total=0) == OK


def _fwd_ex(o_dt, **kw):
    a = dict(q=A, k=A, v=A, g=A, beta=A, s0=None, cu=None, num_seqs=1, total=128, H=2,
             dk=64, dv=64, chunk=64, dt=1, o=A, sf=None, ws=None, ws_bytes=0)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.library().kda_chunk_fwd_ex(
        p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]), p(a["cu"]),
        a["num_seqs"], a["total"], a["H"], a["dk"], a["dv"], a["chunk"], a["dt"], o_dt, p(a["o"]),
        p(a["sf"]), p(a["ws"]), a["ws_bytes"], None)


@gpu_visible
def test_chunk_fwd_ex_rejects():
    # o is the input type or fp32: bf16 o from fp32 inputs, or an unknown type, is refused
    assert _fwd_ex(1, dt=0) == EUNSUP
    assert _fwd_ex(7) == EUNSUP
    assert _fwd_ex(0, q=None) == ENULL              # the common checks still apply
    assert _fwd_ex(0, o=MIS) == EALIGN
    assert _fwd_ex(0, num_seqs=0, total=0) == OK    # bf16 inputs, fp32 o, empty batch


@gpu_visible
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ENULL), (dict(state=None), ENULL), (dict(o=None), ENULL),
    (dict(N=-1), ESHAPE), (dict(H=0), ESHAPE),
    (dict(dk=64, dv=32), EUNSUP), (dict(dk=16, dv=16), EUNSUP), (dict(dt=3), EUNSUP),
    (dict(state=MIS), EALIGN), (dict(v=MIS), EALIGN), (dict(beta=MIS), EALIGN),
])
def test_step_decode_rejects(kw, status):
    assert _dec(**kw) == status


@gpu_visible
def test_step_decode_zero_requests_is_a_no_op():
    assert _dec(N=0) == OK


def test_python_binding_validates_before_the_call():
    import torch
    q = torch.zeros(8, 2, 32)
    with pytest.raises(ValueError):
        _lib.chunk_fwd(q.to(torch.float16), q, q, q, torch.zeros(8, 2))
    with pytest.raises(ValueError):
        _lib.chunk_fwd(q, q, q, q.double(), torch.zeros(8, 2))
    with pytest.raises(ValueError):
        _lib.chunk_fwd(q, q, q, q, torch.zeros(8, 3))
    with pytest.raises(ValueError):
        _lib.step_decode(q, q, q, q, torch.zeros(8, 2), torch.zeros(8, 2, 32, 16))
    # well-formed tensors in host memory are refused: the kernels take device pointers
    with pytest.raises(ValueError, match="GPU device"):
        _lib.chunk_fwd(q, q, q, q, torch.zeros(8, 2))
    with pytest.raises(ValueError, match="GPU device"):
        _lib.step_decode(q, q, q, q, torch.zeros(8, 2), torch.zeros(8, 2, 32, 32))
    with pytest.raises(ValueError, match="GPU device"):
        _lib.output_gate(q, q, torch.ones(32))


def _fused(**kw):
    a = dict(q=A, k=A, v=A, z=A, Al=A, b=A, beta=A, s0=None, cu=None, num_seqs=1, total=128, H=2,
             dk=64, dv=64, chunk=64, dt=1, o=A, sf=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.library().kda_chunk_fwd_fused(
        p(a["q"]), p(a["k"]), p(a["v"]), p(a["z"]), p(a["Al"]), p(a["b"]), p(a["beta"]),
        p(a["s0"]), p(a["cu"]), a["num_seqs"], a["total"], a["H"], a["dk"], a["dv"], a["chunk"],
        a["dt"], p(a["o"]), p(a["sf"]), None, 0, None)


@gpu_visible
@pytest.mark.parametrize("kw,status", [
    (dict(z=None), ENULL), (dict(Al=None), ENULL), (dict(b=None), ENULL), (dict(q=None), ENULL),
    (dict(dk=48, dv=48), EUNSUP), (dict(chunk=32), EUNSUP), (dict(num_seqs=3), ESHAPE),
    (dict(z=MIS), EALIGN), (dict(Al=MIS), EALIGN), (dict(b=MIS), EALIGN),
])
def test_chunk_fwd_fused_rejects(kw, status):
    assert _fused(**kw) == status


@gpu_visible
def test_layer_steps_reject():
    lib = _lib.library()
    p = ctypes.c_void_p
    # output gate: rows, d_v, dtype, pointers, alignment
    assert lib.kda_output_gate(p(A), p(A), p(A), 1e-5, p(A), -1, 128, 1, None) == ESHAPE
    assert lib.kda_output_gate(p(A), p(A), p(A), 1e-5, p(A), 10, 96, 1, None) == EUNSUP
    assert lib.kda_output_gate(p(A), p(A), p(A), -1.0, p(A), 10, 128, 1, None) == ESHAPE
    assert lib.kda_output_gate(p(A), None, p(A), 1e-5, p(A), 10, 128, 1, None) == ENULL
    assert lib.kda_output_gate(p(A), p(A), p(MIS), 1e-5, p(A), 10, 128, 1, None) == EALIGN
    assert lib.kda_output_gate(None, None, None, 1e-5, None, 0, 128, 1, None) == OK
    # output gate with fp32 o~ or result: types, and no in-place call across element sizes
    ex = lib.kda_output_gate_ex
    assert ex(p(A), 7, p(A), p(A), 1e-5, p(A), 1, 10, 128, 1, None) == EUNSUP
    assert ex(p(A), 0, p(A), p(A), 1e-5, p(A), 1, 10, 128, 0, None) == EUNSUP   # bf16 out of fp32 data
    assert ex(p(A), 0, p(A), p(A), 1e-5, p(A), 1, 10, 128, 1, None) == EUNSUP   # out == o_raw, 4 vs 2 bytes
    assert ex(p(A), 0, None, p(A), 1e-5, p(A + 4096), 0, 10, 128, 1, None) == ENULL
    assert ex(None, 0, None, None, 1e-5, None, 0, 0, 128, 1, None) == OK
    # short conv: channels multiple of 4, sequence layout, pointers
    assert lib.kda_short_conv(p(A), p(A), None, 2, 10, 6, None, p(A), 1, None) == EUNSUP
    assert lib.kda_short_conv(p(A), p(A), None, 3, 10, 8, None, p(A), 1, None) == ESHAPE
    assert lib.kda_short_conv(p(A), None, None, 2, 10, 8, None, p(A), 1, None) == ENULL
    assert lib.kda_short_conv(p(A), p(A), None, 2, 10, 8, p(MIS), p(A), 1, None) == EALIGN
    assert lib.kda_short_conv(p(A), p(A), None, 0, 0, 8, None, p(A), 1, None) == OK
    assert lib.kda_short_conv(p(A), p(A), None, 1, 65535 * 64 + 1, 8, None, p(A), 1, None) == ESHAPE
    # state compose: square states of a supported size
    assert lib.kda_state_compose(p(A), p(A), p(A), p(A), 4, 64, 32, None) == EUNSUP
    assert lib.kda_state_compose(p(A), p(A), p(A), p(A), -1, 64, 64, None) == ESHAPE
    assert lib.kda_state_compose(p(A), None, p(A), p(A), 4, 64, 64, None) == ENULL
    assert lib.kda_state_compose(p(A), p(A), p(A), p(MIS), 4, 64, 64, None) == EALIGN
    assert lib.kda_state_compose(None, None, None, None, 0, 64, 64, None) == OK
