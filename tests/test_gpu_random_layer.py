"""Seeded random shapes for the layer entry points beside the prefill: the
split front end (kda_front_end for L2Norm, then kda_chunk_fwd_fused_ex with
the gate fused), ShortConv with the L2Norm of each head (kda_short_conv_ex),
and the segment summaries with their scan (kda_kcp_summaries,
kda_segment_scan) against the whole sequence, each against the fp64 oracle.
Lengths mix empty and one-token sequences with the 16- and 64-token edges."""
import numpy as np
import pytest
import torch

import oracle
from oracle import layer_ref as L
import linear_attention_recurrence_chunk_amd as kda

pytestmark = pytest.mark.gpu
dev = "cuda"
EDGES = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129]


def _np(x):
    return x.detach().to("cpu", torch.float64).numpy()


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def _case(seed):
    rng = np.random.default_rng(seed)
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    d = int(rng.choice([32, 64] if dtype == torch.float32 else [32, 64, 128]))
    lens = [int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, 300))
            for _ in range(int(rng.integers(1, 5)))]
    if sum(lens) == 0:
        lens[0] = 1
    return dtype, d, lens, int(rng.integers(1, 6))


@pytest.mark.parametrize("seed", range(500, 510))
def test_split_front_end_random(seed):
    dtype, d, lens, H = _case(seed)
    gen = torch.Generator(device=dev).manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen, device=dev)
    n = sum(lens)
    q_raw, k_raw = (2.0 * r(n, H, d)).to(dtype), (0.5 * r(n, H, d)).to(dtype)
    v, z = r(n, H, d).to(dtype), (r(n, H, d) + 1.0).to(dtype)
    A_log, b_alpha, beta = 0.3 * r(H), 0.5 * r(H, d), torch.sigmoid(r(n, H))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    s0 = 0.05 * r(len(lens), H, d, d)
    q, k, _ = kda.front_end(q_raw, k_raw)
    o, sf = kda.chunk_fwd_fused(q, k, v, z, A_log, b_alpha, beta, initial_state=s0, cu_seqlens=cu,
                                l2norm=False)
    torch.cuda.synchronize()
    g = L.bounded_gate(_np(z), _np(A_log), _np(b_alpha))
    o_ref, s_ref = oracle.forward(L.l2norm(_np(q_raw)), L.l2norm(_np(k_raw)), _np(v), g, _np(beta),
                                  initial_state=_np(s0), cu_seqlens=cu.cpu().numpy().astype(np.int64))
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    eo, es = _rel(_np(o), o_ref), _rel(_np(sf), s_ref)
    print(f"[parity] split front end seed {seed} {dtype} d={d} H={H} lens={lens}: "
          f"o={eo:.2e} state={es:.2e}", flush=True)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("seed", range(600, 610))
def test_short_conv_l2norm_random(seed):
    dtype, d, lens, H = _case(seed)
    gen = torch.Generator(device=dev).manual_seed(seed)
    n, C = sum(lens), H * d
    x = torch.randn(n, C, generator=gen, device=dev).to(dtype)
    w = torch.randn(C, 4, generator=gen, device=dev)
    st = torch.randn(len(lens), 3, C, generator=gen, device=dev)
    st_in = _np(st)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    y = kda.short_conv(x, w, cu_seqlens=cu, conv_state=st, l2norm_d=d)
    torch.cuda.synchronize()
    yc, st_ref = L.short_conv(_np(x), _np(w), cu_seqlens=cu.cpu().numpy(), conv_state=st_in)
    y_ref = L.l2norm(yc.reshape(n, H, d)).reshape(n, C)
    tol = 2 ** -8 if dtype == torch.bfloat16 else 2e-6
    assert float(np.max(np.abs(_np(y) - y_ref))) <= tol
    np.testing.assert_array_equal(_np(st), st_ref)


@pytest.mark.parametrize("seed", range(700, 706))
def test_segments_random(seed):
    """Random cut points of one sequence: summaries, scan, then each segment's
    prefill from its entering state equal the unsplit sequence."""
    rng = np.random.default_rng(seed)
    dtype = torch.bfloat16 if seed % 3 else torch.float32
    d = int(rng.choice([32, 64, 128] if dtype == torch.bfloat16 else [32, 64]))
    H, T = int(rng.integers(1, 5)), int(rng.integers(100, 700))
    cuts = np.sort(rng.choice(np.arange(1, T), size=int(rng.integers(1, 5)), replace=False))
    cuts = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    gen = torch.Generator(device=dev).manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=gen, device=dev)
    q = torch.nn.functional.normalize(r(T, H, d), dim=-1).to(dtype)
    k = torch.nn.functional.normalize(r(T, H, d), dim=-1).to(dtype)
    v = r(T, H, d).to(dtype)
    g = -5.0 * torch.sigmoid(r(T, H, d) - 4.0)
    beta = torch.sigmoid(r(T, H))
    S0 = 0.05 * r(H, d, d)
    cu = torch.tensor(cuts, device=dev)
    M, St = kda.kcp_summaries(None, k, v, g, beta, cu)
    S_in, S_end = kda.kcp_scan(M, St, S0)
    # each segment's outputs from its entering state
    o = torch.empty_like(v)
    for s_ in range(len(cuts) - 1):
        a, b = int(cuts[s_]), int(cuts[s_ + 1])
        # copies: a slice at an arbitrary token need not be 16-byte aligned
        o_s, _ = kda.chunk_fwd(q[a:b].clone(), k[a:b].clone(), v[a:b].clone(), g[a:b].clone(),
                               beta[a:b].clone(), S_in[s_].unsqueeze(0).clone())
        o[a:b] = o_s
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward(_np(q), _np(k), _np(v), _np(g), _np(beta),
                                  initial_state=_np(S0)[None])
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    eo, es = _rel(_np(o), o_ref), _rel(_np(S_end), s_ref[0])
    print(f"[parity] segments seed {seed} {dtype} d={d} H={H} cuts={list(cuts)}: o={eo:.2e} "
          f"state={es:.2e}", flush=True)
    assert eo <= tol and es <= tol
