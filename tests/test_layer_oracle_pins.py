"""Pins of the layer-step oracle (oracle/layer_ref.py) to what the pages and the
mathematics fix: closed forms, special cases and streaming identities.  Each
test would fail under a plausible mistake in the function it pins (named in
the test)."""
import numpy as np
import pytest

import oracle
from oracle import layer_ref as L
from oracle import numpy_ref

rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- L2Norm
def test_l2norm_closed_form_and_unit_length():
    np.testing.assert_array_equal(L.l2norm(np.array([3.0, 4.0])), [0.6, 0.8])
    x = rng.normal(size=(50, 7, 128))
    y = L.l2norm(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    # direction kept: y is a positive multiple of x (a sign or axis mistake breaks it)
    ratio = y / x
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), rtol=1e-12)
    assert np.all(ratio > 0)


def test_l2norm_zero_vector_maps_to_zero():
    assert np.all(L.l2norm(np.zeros((2, 5))) == 0)


# ---------------------------------------------------------------- bounded gate
def test_gate_midpoint_and_limits():
    H, d = 3, 4
    z0 = np.zeros((H, d))
    A0 = np.zeros(H)
    b0 = np.zeros((H, d))
    # sigma(0) = 1/2, so g = g_min / 2 = -2.5 exactly
    np.testing.assert_array_equal(L.bounded_gate(z0, A0, b0), -2.5)
    # the floor g_min and the ceiling 0 of the notation table's domain (g_min, 0)
    np.testing.assert_allclose(L.bounded_gate(z0 + 60.0, A0, b0), -5.0, rtol=1e-15)
    assert np.all(np.abs(L.bounded_gate(z0 - 60.0, A0, b0)) < 1e-24)
    z = rng.normal(scale=3.0, size=(200, H, d))
    g = L.bounded_gate(z, rng.normal(size=H), rng.normal(size=(H, d)))
    assert np.all((g > -5.0) & (g < 0.0))
    # alpha = e^g lies in (e^-5, 1): the notation table's domain of alpha
    a = np.exp(g)
    assert np.all((a > np.exp(-5.0)) & (a < 1.0))


def test_gate_scale_is_exp_of_A_and_bias_inside():
    H, d = 2, 3
    z = np.full((H, d), 1.0)
    b = np.full((H, d), 1.0)
    A = np.full(H, np.log(2.0))
    # e^A (z + b) = 2 * 2 = 4   (a missing exp, or the bias added after the
    # scale, gives 1.39 or 3 instead)
    want = -5.0 / (1.0 + np.exp(-4.0))
    np.testing.assert_allclose(L.bounded_gate(z, A, b), want, rtol=1e-15)
    # larger logits decay faster: g decreases with z
    zs = np.linspace(-4, 4, 9)[:, None, None] * np.ones((1, H, d))
    g = L.bounded_gate(zs, np.zeros(H), np.zeros((H, d)))
    assert np.all(np.diff(g[:, 0, 0]) < 0)


# ---------------------------------------------------------------- RMSNorm and output gate
def test_rmsnorm_closed_forms():
    c = 3.0
    x = np.full(8, c)
    w = np.arange(1, 9, dtype=np.float64)
    np.testing.assert_allclose(L.rmsnorm(x, w), c / np.sqrt(c * c + 1e-5) * w, rtol=1e-15)
    x = rng.normal(size=(10, 128))
    y = L.rmsnorm(x, np.ones(128))
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-5), rtol=1e-13)


def test_output_gate_half_open_gate():
    o = rng.normal(size=(4, 3, 16))
    w = rng.normal(size=16)
    np.testing.assert_allclose(L.output_gate(o, np.zeros_like(o), w), 0.5 * L.rmsnorm(o, w), rtol=1e-15)
    np.testing.assert_allclose(L.output_gate(o, np.full_like(o, 50.0), w), L.rmsnorm(o, w), rtol=1e-15)


# ---------------------------------------------------------------- ShortConv
def test_short_conv_impulse_response_and_convolution():
    T, C = 9, 3
    w = rng.normal(size=(C, 4))
    x = np.zeros((T, C))
    x[2] = 1.0
    y, _ = L.short_conv(x, w)
    # tap i multiplies x_{t-3+i}: an impulse at t=2 gives w[:, 3], w[:, 2], ... at t = 2, 3, ...
    for j in range(4):
        np.testing.assert_array_equal(y[2 + j], w[:, 3 - j])
    assert np.all(y[:2] == 0) and np.all(y[6:] == 0)           # causal, finite support
    x = rng.normal(size=(T, C))
    y, _ = L.short_conv(x, w)
    for c in range(C):
        np.testing.assert_allclose(y[:, c], np.convolve(x[:, c], w[c, ::-1])[:T], rtol=1e-13)


def test_short_conv_state_streams_and_sequences_do_not_leak():
    C = 5
    w = rng.normal(size=(C, 4))
    x = rng.normal(size=(20, C))
    y, st = L.short_conv(x, w)
    for cut in (1, 2, 3, 7):
        y1, s1 = L.short_conv(x[:cut], w)
        y2, s2 = L.short_conv(x[cut:], w, conv_state=s1)
        np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-14)
        np.testing.assert_allclose(s2, st, rtol=0)
    np.testing.assert_array_equal(st[0], x[-3:])
    cu = [0, 6, 6, 20]
    yp, sp = L.short_conv(x, w, cu_seqlens=cu)
    np.testing.assert_allclose(yp[:6], L.short_conv(x[:6], w)[0], rtol=1e-14)
    np.testing.assert_allclose(yp[6:], L.short_conv(x[6:], w)[0], rtol=1e-14)
    assert np.all(sp[1] == 0)                                   # empty sequence keeps its state


# ---------------------------------------------------------------- KCP summaries
def _kqg(T, H, d, seed):
    r = np.random.default_rng(seed)
    k = L.l2norm(r.normal(size=(T, H, d)))
    q = L.l2norm(r.normal(size=(T, H, d)))
    v = r.normal(size=(T, H, d))
    g = -5.0 / (1.0 + np.exp(-r.normal(1.0, 1.0, size=(T, H, d))))
    beta = 1.0 / (1.0 + np.exp(-r.normal(size=(T, H))))
    return q, k, v, g, beta


def test_transition_product_matches_dense_matrices():
    q, k, v, g, beta = _kqg(7, 1, 5, 3)
    M = np.eye(5)
    for t in range(7):
        M = numpy_ref.transition(k[t, 0], g[t, 0], beta[t, 0]) @ M
    np.testing.assert_allclose(L.transition_product(k[:, 0], g[:, 0], beta[:, 0]), M, rtol=1e-13, atol=1e-15)


def test_transition_product_is_the_recurrence_from_identity_with_zero_values():
    q, k, v, g, beta = _kqg(150, 2, 16, 4)
    _, S = oracle.forward(q, k, np.zeros_like(k), g, beta,
                          initial_state=np.broadcast_to(np.eye(16), (1, 2, 16, 16)).copy())
    for h in range(2):
        np.testing.assert_allclose(S[0, h], L.transition_product(k[:, h], g[:, h], beta[:, h]),
                                   rtol=1e-12, atol=1e-14)


def test_kcp_scan_equals_unsplit_sequence():
    T, H, d = 300, 2, 16
    q, k, v, g, beta = _kqg(T, H, d, 5)
    S0 = np.random.default_rng(6).normal(scale=0.1, size=(1, H, d, d))
    cuts = [0, 64, 65, 190, 300]
    _, S_full = oracle.forward(q, k, v, g, beta, initial_state=S0)
    for h in range(H):
        Ms, Ss = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            Ms.append(L.transition_product(k[a:b, h], g[a:b, h], beta[a:b, h]))
            Ss.append(oracle.forward(q[a:b, h:h + 1], k[a:b, h:h + 1], v[a:b, h:h + 1],
                                     g[a:b, h:h + 1], beta[a:b, h:h + 1])[1][0, 0])
        S_in, S_end = L.kcp_scan(Ms, Ss, S0[0, h])
        np.testing.assert_allclose(S_end, S_full[0, h], rtol=1e-11, atol=1e-13)
        for r, a in enumerate(cuts[:-1]):
            _, S_pref = oracle.forward(q[:a, h:h + 1], k[:a, h:h + 1], v[:a, h:h + 1], g[:a, h:h + 1],
                                       beta[:a, h:h + 1], initial_state=S0[:, h:h + 1])
            np.testing.assert_allclose(S_in[r], S_pref[0, 0], rtol=1e-11, atol=1e-13)
        # pairwise composition agrees with the scan (associativity)
        M01, S01 = L.kcp_compose(Ms[1], Ss[1], Ms[0], Ss[0])
        M23, S23 = L.kcp_compose(Ms[3], Ss[3], Ms[2], Ss[2])
        M, S = L.kcp_compose(M23, S23, M01, S01)
        np.testing.assert_allclose(M @ S0[0, h] + S, S_full[0, h], rtol=1e-11, atol=1e-13)
