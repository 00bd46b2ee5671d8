"""GPU parity of the layer steps around the recurrence (fused front end, output
gate, ShortConv, segment composition) against the fp64 oracle, through the C
ABI.  The oracle reads the same (bf16-rounded) tensors the GPU receives."""
import numpy as np
import pytest
import torch

import oracle
from oracle import layer_ref as L
import linear_attention_recurrence_chunk_amd as kda

pytestmark = pytest.mark.gpu
dev = "cuda"


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def _np(x):
    return x.detach().to("cpu", torch.float64).numpy()


def _fused_inputs(lens, H, d, dtype, seed, state_std=0.0):
    gen = torch.Generator(device=dev).manual_seed(seed)
    n = sum(lens)
    r = lambda *s: torch.randn(*s, generator=gen, device=dev)
    q_raw = (2.0 * r(n, H, d)).to(dtype)
    k_raw = (0.5 * r(n, H, d)).to(dtype)
    v = r(n, H, d).to(dtype)
    z = (r(n, H, d) + 1.0).to(dtype)
    A_log = 0.3 * r(H)
    b_alpha = 0.5 * r(H, d)
    beta = torch.sigmoid(r(n, H))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    s0 = state_std * r(len(lens), H, d, d) if state_std else None
    return q_raw, k_raw, v, z, A_log, b_alpha, beta, cu, s0


def _fused_oracle(q_raw, k_raw, v, z, A_log, b_alpha, beta, cu, s0, heads=None):
    sel = (slice(None), slice(None) if heads is None else heads)
    q = L.l2norm(_np(q_raw)[sel])
    k = L.l2norm(_np(k_raw)[sel])
    hsel = slice(None) if heads is None else heads
    g = L.bounded_gate(_np(z)[sel], _np(A_log)[hsel], _np(b_alpha)[hsel])
    s0n = None if s0 is None else _np(s0)[:, hsel]
    return oracle.forward(q, k, _np(v)[sel], g, _np(beta)[sel], initial_state=s0n,
                          cu_seqlens=cu.cpu().numpy().astype(np.int64))


@pytest.mark.parametrize("dtype,d,lens,state_std,tol", [
    (torch.bfloat16, 128, [300], 0.0, 2e-2),
    (torch.bfloat16, 128, [64, 1, 0, 129, 200], 0.05, 2e-2),
    (torch.bfloat16, 64, [250, 63], 0.05, 2e-2),
    (torch.bfloat16, 32, [333], 0.0, 2e-2),
    (torch.float32, 32, [100, 0, 77, 256], 0.1, 1e-4),
    (torch.float32, 64, [190], 0.1, 1e-4),
])
def test_fused_prologue_prefill(dtype, d, lens, state_std, tol):
    H = 3
    args = _fused_inputs(lens, H, d, dtype, seed=d + len(lens), state_std=state_std)
    q_raw, k_raw, v, z, A_log, b_alpha, beta, cu, s0 = args
    o, sf = kda.chunk_fwd_fused(q_raw, k_raw, v, z, A_log, b_alpha, beta, initial_state=s0,
                                cu_seqlens=cu)
    torch.cuda.synchronize()
    o_ref, s_ref = _fused_oracle(*args)
    eo, es = _rel(_np(o), o_ref), _rel(_np(sf), s_ref)
    print(f"[parity] fused prologue {dtype} d={d} lens={lens}: o={eo:.3e}, state={es:.3e}")
    assert eo <= tol and es <= tol


def _front_end_paths(mode, q_raw, k_raw, v, z, A_log, b_alpha, beta, cu, s0):
    """The prefill from raw inputs by one of the two other routes: 'split' (a
    front-end pass for L2Norm, the gate fused in the prefill) or 'unfused' (a
    front-end pass for both, then the plain prefill)."""
    if mode == "split":
        q, k, _ = kda.front_end(q_raw, k_raw)
        return kda.chunk_fwd_fused(q, k, v, z, A_log, b_alpha, beta, initial_state=s0,
                                   cu_seqlens=cu, l2norm=False)
    q, k, g = kda.front_end(q_raw, k_raw, z, A_log, b_alpha)
    return kda.chunk_fwd(q, k, v, g, beta, s0, cu)


@pytest.mark.parametrize("mode", ["split", "unfused"])
@pytest.mark.parametrize("dtype,d,lens,state_std,tol", [
    (torch.bfloat16, 128, [300], 0.0, 2e-2),
    (torch.bfloat16, 128, [64, 1, 0, 129, 200], 0.05, 2e-2),
    (torch.bfloat16, 64, [250, 63], 0.05, 2e-2),
    (torch.bfloat16, 32, [333], 0.0, 2e-2),
    (torch.float32, 32, [100, 0, 77, 256], 0.1, 1e-4),
    (torch.float32, 64, [190], 0.1, 1e-4),
])
def test_front_end_routes(mode, dtype, d, lens, state_std, tol):
    H = 3
    args = _fused_inputs(lens, H, d, dtype, seed=d + len(lens), state_std=state_std)
    o, sf = _front_end_paths(mode, *args)
    torch.cuda.synchronize()
    o_ref, s_ref = _fused_oracle(*args)
    eo, es = _rel(_np(o), o_ref), _rel(_np(sf), s_ref)
    print(f"[parity] front end {mode} {dtype} d={d} lens={lens}: o={eo:.3e}, state={es:.3e}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.bfloat16, 32), (torch.float32, 128),
                                     (torch.float32, 64), (torch.float32, 32)])
def test_front_end_pass_against_oracle(dtype, d):
    H, T = 5, 203
    args = _fused_inputs([T], H, d, dtype, seed=60 + d)
    q_raw, k_raw, v, z, A_log, b_alpha = args[:6]
    q_raw[17, 2] = 0                                  # a zero row stays zero
    q, k, g = kda.front_end(q_raw, k_raw, z, A_log, b_alpha)
    q2, k2, g2 = kda.front_end(q_raw, k_raw)
    torch.cuda.synchronize()
    assert torch.count_nonzero(q[17, 2]) == 0
    qr, kr = L.l2norm(_np(q_raw)), L.l2norm(_np(k_raw))
    gr = L.bounded_gate(_np(z), _np(A_log), _np(b_alpha))
    # one rounding of the result: half an ulp of the dtype, relative
    tq = 2 ** -8 if dtype == torch.bfloat16 else 1e-6
    # the L2Norm-only pass: the same rows (the two instances may contract the
    # sums of squares differently, so equal up to the same bound)
    assert g2 is None
    assert np.max(np.abs(_np(q2) - qr)) <= tq and np.max(np.abs(_np(k2) - kr)) <= tq
    assert np.max(np.abs(_np(q) - qr)) <= tq and np.max(np.abs(_np(k) - kr)) <= tq
    assert np.max(np.abs(_np(g) - gr)) <= 5 * 2 ** -20
    print(f"[parity] front end pass {dtype} d={d}", flush=True)


def test_fused_prologue_k3_8k_sampled_heads():
    H, d, T = 96, 128, 8192
    args = _fused_inputs([T], H, d, torch.bfloat16, seed=7)
    q_raw, k_raw, v, z, A_log, b_alpha, beta, cu, s0 = args
    o, sf = kda.chunk_fwd_fused(q_raw, k_raw, v, z, A_log, b_alpha, beta, cu_seqlens=cu)
    torch.cuda.synchronize()
    heads = [0, 95]
    o_ref, s_ref = _fused_oracle(*args, heads=heads)
    eo, es = _rel(_np(o)[:, heads], o_ref), _rel(_np(sf)[:, heads], s_ref)
    print(f"[parity] fused prologue 8k x 96 heads {heads}: o={eo:.3e}, state={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2


def test_front_end_split_k3_8k_sampled_heads():
    H, d, T = 96, 128, 8192
    args = _fused_inputs([T], H, d, torch.bfloat16, seed=7)
    o, sf = _front_end_paths("split", *args)
    torch.cuda.synchronize()
    heads = [0, 95]
    o_ref, s_ref = _fused_oracle(*args, heads=heads)
    eo, es = _rel(_np(o)[:, heads], o_ref), _rel(_np(sf)[:, heads], s_ref)
    print(f"[parity] split front end 8k x 96 heads {heads}: o={eo:.3e}, state={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2


def test_fused_prologue_zero_rows_stay_zero():
    # a zero key row is left at zero (no NaN from 0/0); it then writes nothing
    H, d = 2, 64
    args = list(_fused_inputs([130], H, d, torch.bfloat16, seed=11))
    args[1][5:9] = 0
    args[0][70] = 0
    o, sf = kda.chunk_fwd_fused(*args[:7], cu_seqlens=args[7])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(sf).all()
    o_ref, s_ref = _fused_oracle(*args)
    assert _rel(_np(o), o_ref) <= 2e-2 and _rel(_np(sf), s_ref) <= 2e-2


@pytest.mark.parametrize("dtype,d,tol", [(torch.bfloat16, 128, 1e-2), (torch.bfloat16, 64, 1e-2),
                                         (torch.float32, 128, 1e-5), (torch.float32, 32, 1e-5)])
def test_output_gate(dtype, d, tol):
    gen = torch.Generator(device=dev).manual_seed(d)
    rows = 3 * 1000 + 7
    o_raw = (3.0 * torch.randn(rows, d, generator=gen, device=dev)).to(dtype)
    gate = (2.0 * torch.randn(rows, d, generator=gen, device=dev)).to(dtype)
    w = torch.randn(d, generator=gen, device=dev)
    out = kda.output_gate(o_raw, gate, w)
    ref = L.output_gate(_np(o_raw), _np(gate), _np(w))
    torch.cuda.synchronize()
    e = _rel(_np(out), ref)
    print(f"[parity] output gate {dtype} d={d}: {e:.3e}")
    assert e <= tol
    # in place: out aliases o_raw
    again = kda.output_gate(o_raw, gate, w, out=o_raw)
    torch.cuda.synchronize()
    assert again.data_ptr() == o_raw.data_ptr() and _rel(_np(o_raw), ref) <= tol


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("C", [96, 100])     # 100: bf16 rows not a multiple of 16 bytes
def test_short_conv_prefill(dtype, with_state, C):
    gen = torch.Generator(device=dev).manual_seed(3)
    lens = [5, 0, 1, 2, 300, 64]
    n = sum(lens)
    x = torch.randn(n, C, generator=gen, device=dev).to(dtype)
    w = torch.randn(C, 4, generator=gen, device=dev)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    st = torch.randn(len(lens), 3, C, generator=gen, device=dev) if with_state else None
    st_in = None if st is None else _np(st)
    y = kda.short_conv(x, w, cu_seqlens=cu, conv_state=st)
    torch.cuda.synchronize()
    y_ref, st_ref = L.short_conv(_np(x), _np(w), cu_seqlens=cu.cpu().numpy(), conv_state=st_in)
    e = _rel(_np(y), y_ref)
    print(f"[parity] short conv {dtype} C={C} state={with_state}: {e:.3e}")
    assert e <= (1e-2 if dtype == torch.bfloat16 else 1e-6)
    if with_state:
        np.testing.assert_array_equal(_np(st), st_ref)    # copies of inputs: exact


@pytest.mark.parametrize("dtype,d,H,with_state", [(torch.bfloat16, 128, 3, True),
                                                  (torch.bfloat16, 64, 5, False),
                                                  (torch.bfloat16, 32, 3, True),
                                                  (torch.float32, 128, 2, True),
                                                  (torch.float32, 32, 4, False)])
def test_short_conv_l2norm(dtype, d, H, with_state):
    """ShortConv then L2Norm of each head's row in one pass, against the
    oracle's two steps; the state update is the plain ShortConv's."""
    gen = torch.Generator(device=dev).manual_seed(5 + d)
    lens = [5, 0, 1, 2, 300, 64, 17]
    n, C = sum(lens), H * d
    x = torch.randn(n, C, generator=gen, device=dev).to(dtype)
    x[40, :d] = 0                       # a zero input row of one head ...
    w = torch.randn(C, 4, generator=gen, device=dev)
    w[:d, 3] = 0                        # ... whose three earlier inputs stay
    x[37:40, :d] = 0                    # zero, so its output row is zero
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    st = torch.randn(len(lens), 3, C, generator=gen, device=dev) if with_state else None
    st_in = None if st is None else _np(st)
    st2 = None if st is None else st.clone()
    y = kda.short_conv(x, w, cu_seqlens=cu, conv_state=st, l2norm_d=d)
    kda.short_conv(x, w, cu_seqlens=cu, conv_state=st2)
    torch.cuda.synchronize()
    yc, st_ref = L.short_conv(_np(x), _np(w), cu_seqlens=cu.cpu().numpy(), conv_state=st_in)
    y_ref = L.l2norm(yc.reshape(n, H, d)).reshape(n, C)
    assert torch.count_nonzero(y[40, :d]) == 0
    # one rounding of a unit row's entries
    tol = 2 ** -8 if dtype == torch.bfloat16 else 2e-6
    e = float(np.max(np.abs(_np(y) - y_ref)))
    print(f"[parity] short conv + L2Norm {dtype} d={d} state={with_state}: {e:.3e}", flush=True)
    assert e <= tol
    if with_state:
        assert torch.equal(st, st2)
        np.testing.assert_array_equal(_np(st), st_ref)


def test_short_conv_decode_steps_equal_prefill():
    gen = torch.Generator(device=dev).manual_seed(4)
    N, T, C = 8, 6, 64
    x = torch.randn(N, T, C, generator=gen, device=dev).to(torch.bfloat16)
    w = torch.randn(C, 4, generator=gen, device=dev)
    st0 = torch.randn(N, 3, C, generator=gen, device=dev)
    st = st0.clone()
    ys = [kda.short_conv(x[:, t].contiguous(), w, conv_state=st, num_seqs=N) for t in range(T)]
    st_p = st0.clone()
    yp = kda.short_conv(x.reshape(N * T, C), w, conv_state=st_p, num_seqs=N)
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(ys, 1).reshape(N * T, C), yp)
    assert torch.equal(st, st_p)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_state_compose(d):
    gen = torch.Generator(device=dev).manual_seed(d)
    cnt = 37
    M = torch.randn(cnt, d, d, generator=gen, device=dev) / np.sqrt(d)
    S = torch.randn(cnt, d, d, generator=gen, device=dev)
    St = torch.randn(cnt, d, d, generator=gen, device=dev)
    out = kda.state_compose(M, S, St)
    torch.cuda.synchronize()
    ref = _np(M) @ _np(S) + _np(St)
    e = _rel(_np(out), ref)
    print(f"[parity] state compose d={d}: {e:.3e}")
    assert e <= 1e-5
    # in place on S_in, and on S_tilde: the same result
    S2, St2 = S.clone(), St.clone()
    kda.state_compose(M, S2, St, out=S2)
    kda.state_compose(M, S, St2, out=St2)
    torch.cuda.synchronize()
    assert torch.equal(S2, out) and torch.equal(St2, out)


@pytest.mark.parametrize("d,P,H,with_s0", [(32, 5, 3, True), (64, 1, 2, False), (128, 8, 4, True),
                                           (128, 0, 2, True), (64, 3, 5, False),
                                           (128, 4, 96, True)])
def test_segment_scan_against_oracle(d, P, H, with_s0):
    gen = torch.Generator(device=dev).manual_seed(300 + d + P)
    M = 0.9 * torch.randn(P, H, d, d, generator=gen, device=dev) / np.sqrt(d)
    St = torch.randn(P, H, d, d, generator=gen, device=dev)
    S0 = torch.randn(H, d, d, generator=gen, device=dev) if with_s0 else None
    S_in, S_fin = kda.kcp_scan(M, St, S0)
    torch.cuda.synchronize()
    Mn, Sn = _np(M), _np(St)
    hs = range(H) if H <= 8 else (0, 37, H - 1)
    for h in hs:
        s_in_ref, s_fin_ref = L.kcp_scan(Mn[:, h], Sn[:, h], None if S0 is None else _np(S0[h]))
        e_fin = _rel(_np(S_fin[h]), s_fin_ref)
        e_in = _rel(_np(S_in[:, h]), s_in_ref) if P else 0.0
        assert e_fin <= 2e-5 and e_in <= 2e-5, (h, e_fin, e_in)
    print(f"[parity] segment scan d={d} P={P} H={H}: final {e_fin:.2e}", flush=True)
    # in place on S0, and without the entering states: the same final state
    if S0 is not None:
        S1 = S0.clone()
        lib = kda.library()
        p = lambda x: None if x is None else __import__("ctypes").c_void_p(x.data_ptr())
        assert lib.kda_segment_scan(p(M) if P else None, p(St) if P else None, p(S1), None, p(S1),
                                    P, H, d, None) == 0
        torch.cuda.synchronize()
        assert torch.equal(S1, S_fin)


@pytest.mark.parametrize("dtype,d,cuts", [(torch.bfloat16, 128, [0, 500, 501, 621, 2048]),
                                          (torch.bfloat16, 64, [0, 0, 64, 300]),
                                          (torch.bfloat16, 32, [0, 77, 333]),
                                          (torch.float32, 64, [0, 129, 130, 400]),
                                          (torch.float32, 32, [0, 1, 65])])
def test_kcp_summaries_one_launch(dtype, d, cuts):
    """The one-launch summaries equal the two state-only prefills they replace
    (the same slices run the same arithmetic), and M matches the oracle's
    product of transitions."""
    H = 3
    T = cuts[-1]
    gen = torch.Generator(device=dev).manual_seed(40 + d)
    r = lambda *s: torch.randn(*s, generator=gen, device=dev)
    k = torch.nn.functional.normalize(r(T, H, d), dim=-1).to(dtype)
    v = r(T, H, d).to(dtype)
    g = -5.0 * torch.sigmoid(r(T, H, d) - 6.0)
    beta = torch.sigmoid(r(T, H))
    cu = torch.tensor(cuts, dtype=torch.int32, device=dev)
    P = len(cuts) - 1
    M, St = kda.kcp_summaries(None, k, v, g, beta, cu)
    _, St2 = kda.chunk_fwd(None, k, v, g, beta, cu_seqlens=cu, output=False)
    eye = torch.eye(d, device=dev).expand(P, H, d, d).contiguous()
    _, M2 = kda.chunk_fwd(None, k, None, g, beta, initial_state=eye, cu_seqlens=cu, output=False)
    torch.cuda.synchronize()
    assert torch.equal(M, M2) and torch.equal(St, St2)
    kn, gn, bn = _np(k), _np(g), _np(beta)
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    for s_ in range(P):
        a, b = cuts[s_], cuts[s_ + 1]
        for h in range(H):
            m_ref = L.transition_product(kn[a:b, h], gn[a:b, h], bn[a:b, h])
            assert _rel(_np(M[s_, h]), m_ref) <= tol, (s_, h)
    print(f"[parity] KCP summaries {dtype} d={d}: one launch == two launches", flush=True)


def test_kcp_segments_compose_to_the_whole_sequence():
    H, d = 4, 128
    cuts = [0, 500, 501, 621, 2048]
    T = cuts[-1]
    gen = torch.Generator(device=dev).manual_seed(21)
    r = lambda *s: torch.randn(*s, generator=gen, device=dev)
    q = torch.nn.functional.normalize(r(T, H, d), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(r(T, H, d), dim=-1).to(torch.bfloat16)
    v = r(T, H, d).to(torch.bfloat16)
    # weak decays (long memory), so that a 120-token transition product stays
    # far above the float range's floor and the check of M means something
    g = -5.0 * torch.sigmoid(r(T, H, d) - 6.0)
    beta = torch.sigmoid(r(T, H))
    S0 = 0.05 * r(1, H, d, d)
    cu = torch.tensor(cuts, dtype=torch.int32, device=dev)
    M, St = kda.kcp_summaries(q, k, v, g, beta, cu)
    S_in, S_end = kda.kcp_scan(M, St, S0[0])
    torch.cuda.synchronize()
    qn, kn, vn, gn, bn = (_np(x) for x in (q, k, v, g, beta))
    _, s_ref = oracle.forward(qn, kn, vn, gn, bn, initial_state=_np(S0))
    e_end = _rel(_np(S_end), s_ref[0])
    # the transition of one segment against the oracle's product of transitions
    a, b = cuts[2], cuts[3]
    m_ref = np.stack([L.transition_product(kn[a:b, h], gn[a:b, h], bn[a:b, h]) for h in range(H)])
    assert np.max(np.abs(m_ref)) > 1e-3
    e_m = _rel(_np(M[2]), m_ref)
    # the state entering the third segment against the oracle's prefix
    _, s_pref = oracle.forward(qn[:a], kn[:a], vn[:a], gn[:a], bn[:a], initial_state=_np(S0))
    e_in = _rel(_np(S_in[2]), s_pref[0])
    print(f"[parity] KCP: final={e_end:.3e}, M={e_m:.3e}, entering={e_in:.3e}")
    assert e_end <= 2e-2 and e_m <= 2e-2 and e_in <= 2e-2


# fp32-output option: fp32 o~ (the fp32 attention output) and/or fp32 result,
# bf16 gate logits (kda_output_gate_ex)
@pytest.mark.parametrize("in32,out32", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("d", [128, 64, 32])
def test_output_gate_fp32_variants(in32, out32, d):
    gen = torch.Generator(device=dev).manual_seed(100 + d)
    rows = 2 * 1000 + 3
    o_raw = 3.0 * torch.randn(rows, d, generator=gen, device=dev)
    if not in32:
        o_raw = o_raw.to(torch.bfloat16)
    gate = (2.0 * torch.randn(rows, d, generator=gen, device=dev)).to(torch.bfloat16)
    w = torch.randn(d, generator=gen, device=dev)
    odt = torch.float32 if out32 else torch.bfloat16
    out = kda.output_gate(o_raw, gate, w, out_dtype=odt)
    ref = L.output_gate(_np(o_raw), _np(gate), _np(w))
    torch.cuda.synchronize()
    assert out.dtype == odt
    e = _rel(_np(out), ref)
    print(f"[parity] output gate o~ {o_raw.dtype} -> {odt} d={d}: {e:.3e}")
    # fp32 result: only fp32 rounding and the hardware exp / reciprocal steps
    assert e <= (1e-5 if out32 else 1e-2)
    if in32 == out32:
        # equal element sizes: in place is allowed
        again = kda.output_gate(o_raw, gate, w, out=o_raw, out_dtype=odt)
        torch.cuda.synchronize()
        assert again.data_ptr() == o_raw.data_ptr() and _rel(_np(o_raw), ref) <= 1e-5


def test_output_gate_binding_checks_types():
    o_raw = torch.randn(10, 64, device=dev)
    gate = torch.randn(10, 64, device=dev).to(torch.bfloat16)
    w = torch.ones(64, device=dev)
    with pytest.raises(ValueError):
        kda.output_gate(o_raw, gate, w, out_dtype=torch.float16)        # neither bf16 nor fp32
    with pytest.raises(ValueError):
        kda.output_gate(o_raw, gate, w, out=o_raw, out_dtype=torch.bfloat16)  # out must be bf16
    with pytest.raises(ValueError):
        kda.output_gate(o_raw.to(torch.float16), gate, w)               # o~ neither bf16 nor fp32


# ---------------------------------------------------------------------------
# decode step with the output epilogue fused in (kda_step_decode_gated)
@pytest.mark.parametrize("dtype,d,N,H", [(torch.bfloat16, 128, 7, 3), (torch.bfloat16, 64, 7, 3),
                                         (torch.bfloat16, 32, 7, 3), (torch.float32, 128, 7, 3),
                                         (torch.float32, 64, 5, 2), (torch.bfloat16, 128, 256, 96)])
def test_decode_gated_against_oracle(dtype, d, N, H):
    from linear_attention_recurrence_chunk_amd import inputs
    w = inputs.custom(H=H, dk=d, dv=d, dtype=dtype, decode_requests=N, state_std=0.5)
    x = inputs.decode_inputs(w, seed=200 + d, device=dev)
    gen = torch.Generator(device=dev).manual_seed(201 + d)
    gate = torch.randn(x["v"].shape, generator=gen, device=dev).to(dtype)
    wt = 1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)
    st0 = x["state"].clone()
    st_plain = x["state"].clone()
    o_raw = torch.empty_like(x["v"])
    y = kda.step_decode_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"], gate, wt,
                              1e-5, o_raw=o_raw)
    o_plain = kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], st_plain)
    torch.cuda.synchronize()
    # the step is the plain kernel's, bit for bit
    assert torch.equal(o_raw, o_plain) and torch.equal(x["state"], st_plain)
    o_ref, s_ref = oracle.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], st0)
    y_ref = L.output_gate(o_ref, _np(gate), _np(wt), eps=1e-5)
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    e, es = _rel(_np(y), y_ref), _rel(_np(x["state"]), s_ref)
    print(f"[layer] decode gated {dtype} d={d} N={N} H={H}: out {e:.3e} state {es:.3e}", flush=True)
    assert e <= tol and es <= tol
    # without o_raw the gated output is the same
    st1 = st0.clone()
    y2 = kda.step_decode_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], st1, gate, wt, 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y2, y) and torch.equal(st1, st_plain)
