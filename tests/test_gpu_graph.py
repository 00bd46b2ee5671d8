"""The C-ABI calls captured in a HIP graph (torch.cuda.CUDAGraph on the
current stream, which the binding launches on) and replayed several times,
with eager work and synchronisations between the replays: every replay must
equal the eager call bit for bit.  The library enqueues kernels only (no
memset, no allocation), so its calls can sit in a graph."""
import pytest
import torch

import linear_attention_recurrence_chunk_amd as kda
from linear_attention_recurrence_chunk_amd import inputs

pytestmark = pytest.mark.gpu
dev = "cuda"


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("gated", [False, True])
def test_decode_graph_replays_equal_eager_steps(gated):
    w = inputs.WORKLOADS["nano_k3_decode"]
    x = inputs.decode_inputs(w, seed=9, device=dev)
    gate = torch.randn(x["v"].shape, generator=torch.Generator(device=dev).manual_seed(3),
                       device=dev).to(x["v"].dtype)
    wt = torch.ones(w.dv, device=dev)

    def step(st, out):
        if gated:
            kda.step_decode_gated(x["q"], x["k"], x["v"], x["g"], x["beta"], st, gate, wt, out=out)
        else:
            kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], st, out=out)

    # eager: four successive steps
    st_e, outs = x["state"].clone(), []
    for _ in range(4):
        o = torch.empty_like(x["v"])
        step(st_e, o)
        torch.cuda.synchronize()
        outs.append(o)
    # graph of one step; the warm-up before capture advances the state, so reset it
    st_g, og = x["state"].clone(), torch.empty_like(x["v"])
    g = _capture(lambda: step(st_g, og))
    st_g.copy_(x["state"])
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(og, outs[i]), i
        _ = (og.float() * 2).sum().item()          # eager work between replays
    assert torch.equal(st_g, st_e)


def test_prefill_graph_replays_equal_eager():
    w = inputs.WORKLOADS["nano_k3_prefill"]
    x = inputs.prefill_inputs(w, seed=2, device=dev)
    o_e = torch.empty_like(x["v"])
    sf_e = torch.empty((len(x["seqlens"]), w.H, w.dk, w.dv), device=dev)
    kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None, x["cu_seqlens"], out=o_e,
                  final_state=sf_e)
    torch.cuda.synchronize()
    o_g, sf_g = torch.empty_like(o_e), torch.empty_like(sf_e)
    g = _capture(lambda: kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], None,
                                       x["cu_seqlens"], out=o_g, final_state=sf_g))
    for _ in range(3):
        o_g.zero_()
        sf_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(sf_g, sf_e)
