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

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP, ETOOLARGE = range(8)


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
                            "kda_chunk_fwd_ex", "kda_output_gate_ex", "kda_chunk_fwd_algo",
                            "kda_chunk_fwd_algo_workspace_size", "kda_chunk_fwd_two_pass_static",
                            "kda_chunk_fwd_static_scratch_bytes", "kda_step_decode_gated", "kda_segment_scan",
                            "kda_kcp_summaries", "kda_chunk_fwd_fused_ex", "kda_front_end",
                            "kda_short_conv_ex"])
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_version_and_status_strings():
    lib = _lib.library()
    assert lib.kda_version() == 1
    for s in range(8):
        assert lib.kda_status_string(s) != b"unknown status"
    assert lib.kda_status_string(99) == b"unknown status"


AUTO, FUSED, TWO_PASS = 0, 1, 2


def _packet_bytes(d, C, esize):
    # Kg, Qg, Kbar^T (C d each), T diag(beta) (two bf16 halves for bf16) and P as
    # C/16 (C/16 + 1) / 2 blocks of 16 x 16, then gamma (d fp32), rounded up to 256 bytes
    nb = C // 16
    nsets = 3 if esize == 2 else 2
    raw = (3 * C * d + nsets * 256 * nb * (nb + 1) // 2) * esize + 4 * d
    return (raw + 255) // 256 * 256


def test_workspace_sizes():
    lib = _lib.library()
    ws = lib.kda_chunk_fwd_workspace_size
    wsa = lib.kda_chunk_fwd_algo_workspace_size
    # the fused kernel keeps every intermediate on chip
    assert ws(16, 100000, 96, 128, 128, 64, 1) == 0
    assert wsa(16, 100000, 96, 128, 128, 64, 1, FUSED) == 0
    # two-pass: one packet per (chunk slot, head), slots < ceil(T / C) + N
    assert _packet_bytes(128, 64, 2) == 65024 and _packet_bytes(128, 128, 2) == 154112
    for (N, T, H, d, C, dt, es) in [(1, 8192, 96, 128, 64, 1, 2), (16, 135168, 96, 128, 64, 1, 2),
                                    (1, 131072, 96, 128, 128, 1, 2), (3, 1000, 2, 32, 128, 0, 4),
                                    (2, 777, 4, 128, 64, 0, 4), (5, 0, 3, 64, 64, 1, 2)]:
        want = ((T + C - 1) // C + N) * H * _packet_bytes(d, C, es)
        assert wsa(N, T, H, d, d, C, dt, TWO_PASS) == want
    # AUTO: the fused kernel where it applies (C = 64, not fp32 at d = 128)
    assert ws(1, 131072, 96, 128, 128, 128, 1) == wsa(1, 131072, 96, 128, 128, 128, 1, TWO_PASS) > 0
    assert ws(2, 777, 4, 128, 128, 64, 0) == wsa(2, 777, 4, 128, 128, 64, 0, TWO_PASS) > 0
    assert ws(2, 777, 4, 64, 64, 64, 0) == 0
    # unsupported: fp32 with C = 128 at d = 128, the fused kernel with C = 128, bad algo
    assert wsa(1, 1000, 2, 128, 128, 128, 0, TWO_PASS) == 0
    assert ws(1, 1000, 2, 128, 128, 128, 0) == 0
    assert wsa(1, 1000, 2, 64, 64, 128, 1, FUSED) == 0
    assert wsa(1, 1000, 2, 64, 64, 64, 1, 9) == 0


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
    (dict(dt=0, dk=128, dv=128, chunk=128), EUNSUP), # fp32 with C = 128 stops at d = 64
    (dict(chunk=128), EWS),                          # the two-pass path needs a workspace
    (dict(chunk=128, ws=A, ws_bytes=1000), EWS),
    (dict(dt=0, dk=128, dv=128), EWS),               # fp32 at d = 128 runs the two-pass path
    (dict(chunk=128, ws=MIS, ws_bytes=1 << 30), EALIGN),
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


def _fwd_algo(algo, **kw):
    a = dict(q=A, k=A, v=A, g=A, beta=A, s0=None, cu=None, num_seqs=1, total=128, H=2,
             dk=64, dv=64, chunk=64, dt=1, odt=1, o=A, sf=None, ws=None, ws_bytes=0)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.library().kda_chunk_fwd_algo(
        p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]), p(a["cu"]),
        a["num_seqs"], a["total"], a["H"], a["dk"], a["dv"], a["chunk"], a["dt"], a["odt"], algo,
        p(a["o"]), p(a["sf"]), p(a["ws"]), a["ws_bytes"], None)


@gpu_visible
def test_chunk_fwd_algo_rejects():
    assert _fwd_algo(FUSED, chunk=128) == EUNSUP            # the fused kernel is C = 64
    assert _fwd_algo(FUSED, dt=0, odt=0, dk=128, dv=128) == EUNSUP
    assert _fwd_algo(9) == EUNSUP
    assert _fwd_algo(TWO_PASS) == EWS                        # no workspace
    assert _fwd_algo(TWO_PASS, ws=A, ws_bytes=10) == EWS
    assert _fwd_algo(TWO_PASS, num_seqs=0, total=0) == OK    # empty batch: nothing to do
    assert _fwd_algo(FUSED, num_seqs=0, total=0) == OK


def _fwd_static(**kw):
    a = dict(q=A, k=A, v=A, g=A, beta=A, s0=None, cu=None, num_seqs=1, total=128, H=2,
             dk=64, dv=64, chunk=64, dt=1, odt=1, o=A, sf=None)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return _lib.library().kda_chunk_fwd_two_pass_static(
        p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]), p(a["s0"]), p(a["cu"]),
        a["num_seqs"], a["total"], a["H"], a["dk"], a["dv"], a["chunk"], a["dt"], a["odt"],
        p(a["o"]), p(a["sf"]), None)


def test_static_scratch_size():
    assert _lib.library().kda_chunk_fwd_static_scratch_bytes() == 256 << 20


@gpu_visible
def test_chunk_fwd_static_rejects():
    # the common checks, then the static scratch's capacity, all before any HIP call
    assert _fwd_static(q=None) == ENULL
    assert _fwd_static(dk=48, dv=48) == EUNSUP
    assert _fwd_static(dt=0, odt=0, dk=128, dv=128, chunk=128) == EUNSUP
    assert _fwd_static(o=MIS) == EALIGN
    assert _fwd_static(odt=7) == EUNSUP
    assert _fwd_static(total=8192, H=96, dk=128, dv=128) == ETOOLARGE   # 8K x 96 heads
    assert _fwd_static(num_seqs=0, total=0) == OK


@gpu_visible
def test_step_decode_gated_rejects():
    lib = _lib.library()
    p = ctypes.c_void_p

    def call(**kw):
        a = dict(q=A, k=A, v=A, g=A, beta=A, state=A, gate=A, w=A, eps=1e-5, out=A, o=None, N=4, H=2,
                 dk=64, dv=64, dt=1)
        a.update(kw)
        q = lambda x: None if x is None else p(x)
        return lib.kda_step_decode_gated(q(a["q"]), q(a["k"]), q(a["v"]), q(a["g"]), q(a["beta"]),
                                         q(a["state"]), q(a["gate"]), q(a["w"]), a["eps"],
                                         q(a["out"]), q(a["o"]), a["N"], a["H"], a["dk"], a["dv"],
                                         a["dt"], None)
    assert call(gate=None) == ENULL and call(w=None) == ENULL and call(out=None) == ENULL
    assert call(eps=-1.0) == ESHAPE and call(N=-1) == ESHAPE
    assert call(dk=48, dv=48) == EUNSUP and call(dt=5) == EUNSUP
    assert call(gate=MIS) == EALIGN and call(o=MIS) == EALIGN
    assert call(N=0) == OK


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
    (dict(chunk=128), EUNSUP),                       # the fused front end runs the C = 64 kernel
    (dict(z=MIS), EALIGN), (dict(Al=MIS), EALIGN), (dict(b=MIS), EALIGN),
])
def test_chunk_fwd_fused_rejects(kw, status):
    assert _fused(**kw) == status


@gpu_visible
@pytest.mark.parametrize("fuse", [0, 2, 4, -1])
def test_chunk_fwd_fused_ex_rejects_unknown_steps(fuse):
    p = ctypes.c_void_p
    assert _lib.library().kda_chunk_fwd_fused_ex(
        p(A), p(A), p(A), p(A), p(A), p(A), p(A), None, None, 1, 128, 2, 64, 64, 64, 1, fuse,
        p(A), None, None, 0, None) == EUNSUP


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
    # ShortConv with the L2Norm of each head's row
    sc = lambda nd, C=256: lib.kda_short_conv_ex(p(A), p(A), None, 1, 16, C, None, p(A), 1, nd, None)
    assert sc(48) == EUNSUP and sc(128, C=192) == EUNSUP and sc(-1) == EUNSUP
    assert lib.kda_short_conv_ex(p(A), p(A), None, 0, 0, 256, None, p(A), 1, 64, None) == OK
    # front end as a pass of its own
    fe = lambda **kw: (lambda a: lib.kda_front_end(
        a["qr"], a["kr"], a["z"], a["A"], a["b"], a["n"], 2, a["d"], a["dt"], a["q"], a["k"], a["g"],
        None))({**dict(qr=p(A), kr=p(A), z=p(A), A=p(A), b=p(A), n=10, d=64, dt=1, q=p(A), k=p(A),
                       g=p(A)), **kw})
    assert fe(d=48) == EUNSUP and fe(dt=7) == EUNSUP and fe(n=-1) == ESHAPE
    assert fe(qr=None) == ENULL and fe(k=None) == ENULL and fe(z=None) == ENULL
    assert fe(g=p(MIS)) == EALIGN and fe(n=0, qr=None) == OK
    # segment summaries in one launch
    ks = lambda **kw: (lambda a: lib.kda_kcp_summaries(
        a["k"], a["v"], p(A), p(A), None, a["P"], a["n"], 2, a["d"], a["C"], a["dt"], a["M"], a["S"],
        None))({**dict(k=p(A), v=p(A), P=2, n=128, d=64, C=64, dt=1, M=p(A), S=p(A)), **kw})
    assert ks(d=128, dt=0) == EUNSUP and ks(C=128) == EUNSUP and ks(d=48) == EUNSUP
    assert ks(M=None) == ENULL and ks(S=None) == ENULL and ks(v=None) == ENULL
    assert ks(k=None) == ENULL and ks(M=p(MIS)) == EALIGN and ks(n=127) == ESHAPE
    assert ks(P=0, n=0) == OK
    # segment scan
    assert lib.kda_segment_scan(p(A), p(A), None, None, p(A), -1, 2, 64, None) == ESHAPE
    assert lib.kda_segment_scan(p(A), p(A), None, None, p(A), 3, 0, 64, None) == ESHAPE
    assert lib.kda_segment_scan(p(A), p(A), None, None, p(A), 3, 2, 48, None) == EUNSUP
    assert lib.kda_segment_scan(p(A), p(A), None, None, None, 3, 2, 64, None) == ENULL
    assert lib.kda_segment_scan(None, p(A), None, None, p(A), 3, 2, 64, None) == ENULL
    assert lib.kda_segment_scan(p(A), p(A), p(MIS), None, p(A), 3, 2, 64, None) == EALIGN
    assert lib.kda_segment_scan(p(A), p(A), None, p(MIS), p(A), 3, 2, 64, None) == EALIGN
