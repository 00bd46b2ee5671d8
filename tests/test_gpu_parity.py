"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances: bf16 inputs  max|x - x_ref| <= 2e-2 * max|x_ref|, for o and for the
final state; fp32 inputs 1e-4 on the same measure.  Full-size workloads are
checked on every head, every token and every sequence: the GPU runs the whole
workload in the launch configuration the benchmark times, and the oracle
follows it one block of heads at a time (host memory stays bounded).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrence_chunk_amd import inputs
from linear_attention_recurrence_chunk_amd import _lib as kda

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def rel_err(x, ref) -> float:
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.isfinite(x).all(), "non-finite output"
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def report(name, **errs):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)


# prefill algorithms of kda_chunk_fwd_algo: the fused kernel (C = 64) and the
# two-pass path (chunk-parallel intra pass + state pass, C = 64 or 128)
ALGOS = ["fused", "two_pass"]


def algo_ok(algo, dtype, d, chunk):
    if algo == "fused":
        return chunk == 64 and (dtype == torch.bfloat16 or d <= 64)
    return dtype == torch.bfloat16 or chunk == 64 or d <= 64


def run_prefill_streamed(x, chunk, head_block=16, algos=("auto",)):
    """GPU on the whole input (once per algorithm); the oracle over all heads,
    head_block heads at a time.  Returns {algo: (o error, state error)}, whole-
    tensor relative errors."""
    outs = {}
    for a in algos:
        outs[a] = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                                x["cu_seqlens"], chunk_size=chunk, algo=a)
    torch.cuda.synchronize()
    H = x["q"].shape[1]
    cu = x["cu_seqlens"].cpu().numpy()
    num = {(a, k): 0.0 for a in algos for k in "os"}
    den = {"o": 0.0, "s": 0.0}
    for h0 in range(0, H, head_block):
        hs = slice(h0, min(H, h0 + head_block))
        sub = lambda t: None if t is None else t[:, hs].cpu()
        o_ref, sf_ref = oracle.forward(sub(x["q"]), sub(x["k"]), sub(x["v"]), sub(x["g"]),
                                       sub(x["beta"]), sub(x["initial_state"]), cu)
        den["o"] = max(den["o"], float(np.abs(o_ref).max(initial=0.0)))
        den["s"] = max(den["s"], float(np.abs(sf_ref).max(initial=0.0)))
        for a in algos:
            o, sf = outs[a]
            for key, got, ref in (("o", o[:, hs], o_ref), ("s", sf[:, hs], sf_ref)):
                g64 = got.double().cpu().numpy()
                assert np.isfinite(g64).all(), f"non-finite output ({a})"
                num[(a, key)] = max(num[(a, key)], float(np.abs(g64 - ref).max(initial=0.0)))
        del o_ref, sf_ref
    return {a: (num[(a, "o")] / max(den["o"], 1e-30), num[(a, "s")] / max(den["s"], 1e-30))
            for a in algos}


def run_prefill(x, chunk, heads=None, algo="auto"):
    """GPU on the whole input; oracle on `heads` (all when None).  Returns errors."""
    o, sf = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                          x["cu_seqlens"], chunk_size=chunk, algo=algo)
    torch.cuda.synchronize()
    hs = slice(None) if heads is None else list(heads)
    sub = lambda t: None if t is None else t[:, hs].cpu()
    o_ref, sf_ref = oracle.forward(sub(x["q"]), sub(x["k"]), sub(x["v"]), sub(x["g"]),
                                   sub(x["beta"]), sub(x["initial_state"]),
                                   x["cu_seqlens"].cpu().numpy())
    return rel_err(o[:, hs], o_ref), rel_err(sf[:, hs], sf_ref)


# ---------------------------------------------------------------------------
# decode
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_small(dtype, d):
    w = inputs.custom(H=3, dk=d, dv=d, dtype=dtype, decode_requests=5, state_std=0.5)
    x = inputs.decode_inputs(w, seed=d, device=DEV)
    st0 = x["state"].clone()
    o = kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"])
    torch.cuda.synchronize()
    o_ref, st_ref = oracle.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], st0)
    eo, es = rel_err(o, o_ref), rel_err(x["state"], st_ref)
    report(f"decode d={d} {dtype}", o=eo, state=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_k3_256_requests():
    w = inputs.WORKLOADS["k3_decode_256"]
    x = inputs.decode_inputs(w, seed=5, device=DEV)
    st0 = x["state"].cpu()
    o = kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"])
    torch.cuda.synchronize()
    o_ref, st_ref = oracle.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], st0)
    eo, es = rel_err(o, o_ref), rel_err(x["state"], st_ref)
    report("decode k3 N=256", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2


# ---------------------------------------------------------------------------
# prefill, small shapes (whole oracle)
@pytest.mark.parametrize("algo", ALGOS)
def test_prefill_tiny_fp32(algo):
    w = inputs.WORKLOADS["tiny_fp32"]
    x = inputs.prefill_inputs(w, seed=1, device=DEV)
    eo, es = run_prefill(x, w.chunk, algo=algo)
    report(f"prefill tiny fp32 {algo}", o=eo, state=es)
    assert eo <= 1e-4 and es <= 1e-4


CASES = [
    # (dtype, d, seqlens, H, state_std)
    (torch.bfloat16, 128, [300], 4, 0.0),
    (torch.bfloat16, 128, [64, 1, 0, 129, 200], 3, 0.05),
    (torch.bfloat16, 64, [250, 63], 4, 0.05),
    (torch.bfloat16, 32, [333], 2, 0.0),
    (torch.float32, 32, [100, 0, 77, 256], 2, 0.1),
    (torch.float32, 64, [190], 2, 0.1),
    (torch.float32, 128, [190, 64, 1, 0, 129], 3, 0.1),
]


@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype,d,lens,H,std", CASES)
def test_prefill_shapes(dtype, d, lens, H, std, algo, chunk):
    if not algo_ok(algo, dtype, d, chunk):
        pytest.skip(f"{algo} does not take {dtype} d={d} C={chunk}")
    w = inputs.custom(H=H, dk=d, dv=d, seqlens=lens, dtype=dtype, state_std=std)
    x = inputs.prefill_inputs(w, seed=sum(lens) + d, device=DEV)
    eo, es = run_prefill(x, chunk, algo=algo)
    report(f"prefill {algo} C={chunk} {dtype} d={d} lens={lens}", o=eo, state=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("algo,chunk", [("fused", 64), ("two_pass", 64), ("two_pass", 128)])
@pytest.mark.parametrize("gate", ["no_decay", "max_decay"])
@pytest.mark.parametrize("bval", [0.0, 1.0])
def test_prefill_degenerate_gates(gate, bval, algo, chunk):
    """g = 0 (alpha = 1) or g = g_min everywhere; beta all 0 or all 1.  With
    the maximal decay and beta = 0 nothing is written and the prefix state
    decays by e^-5 a token, so the sequences are kept short enough (at most 14
    tokens: e^-70 of the prefix, far from the fp32 subnormal range) that the
    reference state is a normal fp32 number and the comparison can fail."""
    lens = [14, 9, 5] if (gate == "max_decay" and bval == 0.0) else [150, 40]
    w = inputs.custom(H=2, dk=128, dv=128, seqlens=lens, state_std=0.1)
    x = inputs.prefill_inputs(w, seed=7, device=DEV)
    x["g"].fill_(0.0 if gate == "no_decay" else -5.0)
    x["beta"].fill_(bval)
    o, sf = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                          x["cu_seqlens"], chunk_size=chunk, algo=algo)
    torch.cuda.synchronize()
    cpu = lambda t: t.cpu()
    o_ref, sf_ref = oracle.forward(*(cpu(x[n]) for n in ("q", "k", "v", "g", "beta",
                                                         "initial_state")),
                                   x["cu_seqlens"].cpu().numpy())
    assert np.abs(sf_ref).max() > 1e-30 and np.abs(o_ref).max() > 1e-30
    eo, es = rel_err(o, o_ref), rel_err(sf, sf_ref)
    report(f"prefill {algo} C={chunk} gate={gate} beta={bval}", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2


# ---------------------------------------------------------------------------
# full-size workloads
def test_prefill_k3_8k():
    w = inputs.WORKLOADS["k3_prefill_8k"]
    x = inputs.prefill_inputs(w, seed=2, device=DEV)
    errs = run_prefill_streamed(x, w.chunk, head_block=48, algos=ALGOS)
    for a, (eo, es) in errs.items():
        report(f"prefill k3 8k {a}, all 96 heads", o=eo, state=es)
        assert eo <= 2e-2 and es <= 2e-2, a


def test_prefill_nano_k3_full_size():
    # the second workload: 32 sequences x 2048 tokens, 8 heads of 64, every head
    w = inputs.WORKLOADS["nano_k3_prefill"]
    x = inputs.prefill_inputs(w, seed=2, device=DEV)
    eo, es = run_prefill(x, w.chunk)
    report("prefill nano-K3 32 x 2048 x 8 x 64", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2


def test_decode_nano_k3():
    w = inputs.WORKLOADS["nano_k3_decode"]
    x = inputs.decode_inputs(w, seed=5, device=DEV)
    st0 = x["state"].cpu()
    o = kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"])
    torch.cuda.synchronize()
    o_ref, st_ref = oracle.decode(x["q"], x["k"], x["v"], x["g"], x["beta"], st0)
    eo, es = rel_err(o, o_ref), rel_err(x["state"], st_ref)
    report("decode nano-K3 N=256", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2


def test_prefill_chunk_128_and_chunk_64_agree_with_oracle():
    w = inputs.custom(H=3, dk=128, dv=128, seqlens=[300, 129], state_std=0.05)
    x = inputs.prefill_inputs(w, seed=17, device=DEV)
    for chunk in (64, 128):
        eo, es = run_prefill(x, chunk)
        report(f"prefill C={chunk} small", o=eo, state=es)
        assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.slow
def test_prefill_k3_128k():
    w = inputs.WORKLOADS["k3_prefill_128k"]
    x = inputs.prefill_inputs(w, seed=3, device=DEV)
    (eo, es), = run_prefill_streamed(x, w.chunk, head_block=16).values()
    report("prefill k3 128k (C=128, two-pass), all 96 heads", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2


def test_prefill_varlen_prefix():
    w = inputs.WORKLOADS["k3_varlen_prefix"]
    x = inputs.prefill_inputs(w, seed=4, device=DEV)
    print(f"[parity] varlen lengths {x['seqlens']}", flush=True)
    errs = run_prefill_streamed(x, w.chunk, head_block=16, algos=ALGOS)
    for a, (eo, es) in errs.items():
        report(f"prefill varlen+prefix {a}, all 96 heads", o=eo, state=es)
        assert eo <= 2e-2 and es <= 2e-2, a


# ---------------------------------------------------------------------------
# self-consistency of the HIP path
def test_prefill_equals_repeated_decode():
    w = inputs.custom(H=3, dk=128, dv=128, seqlens=[70], state_std=0.1)
    x = inputs.prefill_inputs(w, seed=11, device=DEV)
    o, sf = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                          x["cu_seqlens"])
    st = x["initial_state"].clone()
    outs = []
    for t in range(70):
        one = [x[n][t:t + 1].clone() for n in ("q", "k", "v", "g", "beta")]  # 16-byte aligned
        outs.append(kda.step_decode(*one, st))
    torch.cuda.synchronize()
    od = torch.cat(outs)
    e1 = rel_err(o, od.double().cpu().numpy())
    e2 = rel_err(sf, st.double().cpu().numpy())
    report("prefill vs repeated decode", o=e1, state=e2)
    assert e1 <= 2e-2 and e2 <= 2e-2


def test_prefill_split_resume_equals_whole():
    w = inputs.custom(H=4, dk=128, dv=128, seqlens=[500], state_std=0.05)
    x = inputs.prefill_inputs(w, seed=12, device=DEV)
    o, sf = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"])
    cut = 200
    a = lambda t: t[:cut].contiguous()
    b = lambda t: t[cut:].contiguous()
    o1, s1 = kda.chunk_fwd(a(x["q"]), a(x["k"]), a(x["v"]), a(x["g"]), a(x["beta"]),
                           x["initial_state"])
    o2, s2 = kda.chunk_fwd(b(x["q"]), b(x["k"]), b(x["v"]), b(x["g"]), b(x["beta"]), s1)
    torch.cuda.synchronize()
    e1 = rel_err(torch.cat([o1, o2]), o.double().cpu().numpy())
    e2 = rel_err(s2, sf.double().cpu().numpy())
    report("split/resume", o=e1, state=e2)
    assert e1 <= 2e-2 and e2 <= 2e-2


def test_prefill_is_deterministic_and_final_may_alias_initial():
    w = inputs.custom(H=8, dk=128, dv=128, seqlens=[1000, 333], state_std=0.05)
    x = inputs.prefill_inputs(w, seed=13, device=DEV)
    o1, s1 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                           x["cu_seqlens"])
    o2, s2 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                           x["cu_seqlens"])
    inplace = x["initial_state"].clone()
    o3, s3 = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], inplace,
                           x["cu_seqlens"], final_state=inplace)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, inplace)


def test_decode_is_deterministic():
    w = inputs.WORKLOADS["k3_decode_256"]
    x = inputs.decode_inputs(w, seed=21, device=DEV, requests=8)
    s_a, s_b = x["state"].clone(), x["state"].clone()
    o_a = kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], s_a)
    o_b = kda.step_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], s_b)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)


# ---------------------------------------------------------------------------
# edge cases of the sequence layout
@pytest.mark.parametrize("dtype,d,tol", [(torch.bfloat16, 128, 2e-2), (torch.float32, 64, 1e-4)])
def test_prefill_many_short_and_empty_sequences(dtype, d, tol):
    lens = [1, 2, 3, 0, 0, 5, 63, 64, 65, 1, 16, 17, 0]
    w = inputs.custom(H=2, dk=d, dv=d, seqlens=lens, state_std=0.05, dtype=dtype)
    x = inputs.prefill_inputs(w, seed=41, device=DEV)
    eo, es = run_prefill(x, 64)
    report(f"prefill short/empty sequences {dtype} d={d}", o=eo, state=es)
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("T", [1, 15, 16, 64])
def test_prefill_single_head_tiny_lengths(T):
    # fp32: with one head and a few tokens the whole output can be tiny (a query
    # nearly orthogonal to the keys), and a bound relative to max |o_ref| then
    # measures bf16 rounding of the decayed operands, not the kernel's logic
    w = inputs.custom(H=1, dk=64, dv=64, seqlens=[T], state_std=0.1, dtype=torch.float32)
    x = inputs.prefill_inputs(w, seed=43 + T, device=DEV)
    eo, es = run_prefill(x, 64)
    report(f"prefill H=1 T={T} fp32", o=eo, state=es)
    assert eo <= 1e-4 and es <= 1e-4


def test_prefill_batched_4d_layout_equals_packed():
    # [B, T, H, d] with no cu_seqlens is B equal sequences; same as the packed call
    B, T, H, d = 3, 200, 2, 64
    w = inputs.custom(H=H, dk=d, dv=d, seqlens=[T] * B, state_std=0.05)
    x = inputs.prefill_inputs(w, seed=45, device=DEV)
    o4, s4 = kda.chunk_fwd(*(x[n].view(B, T, H, -1) for n in ("q", "k", "v", "g")),
                           x["beta"].view(B, T, H), x["initial_state"])
    op, sp = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"],
                           x["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o4.view(B * T, H, d), op) and torch.equal(s4, sp)


def test_prefill_many_heads():
    w = inputs.custom(H=256, dk=128, dv=128, seqlens=[130], state_std=0.02)
    x = inputs.prefill_inputs(w, seed=47, device=DEV)
    eo, es = run_prefill(x, 64, heads=[0, 97, 255])
    report("prefill H=256", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2


def _random_cases(n, seed=2024):
    """Seeded random prefill shapes: head count, head size, type, a mix of
    sequence lengths (empty, single tokens, sub-block and chunk edges, long
    ragged ones), prefix states, chunk size and gate distribution."""
    rng = np.random.default_rng(seed)
    edges = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129]
    cases = []
    for i in range(n):
        dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
        d = int(rng.choice([32, 64] if dtype == torch.float32 else [32, 64, 128]))
        nseq = int(rng.integers(1, 6))
        lens = [int(rng.choice(edges)) if rng.random() < 0.5 else int(rng.integers(1, 400))
                for _ in range(nseq)]
        if sum(lens) == 0:
            lens[0] = 1
        cases.append(dict(H=int(rng.integers(1, 7)), dk=d, dv=d, seqlens=lens, dtype=dtype,
                          state_std=float(rng.choice([0.0, 0.05])),
                          chunk=int(rng.choice([64, 128])),
                          extreme_heads=int(rng.integers(0, 2)), seed=100 + i))
    return cases


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("case", _random_cases(16), ids=lambda c: f"seed{c['seed']}")
def test_prefill_random_shapes(case, algo):
    case = dict(case)
    seed = case.pop("seed")
    w = inputs.custom(**case)
    chunk = w.chunk if algo == "two_pass" else 64
    x = inputs.prefill_inputs(w, seed=seed, device=DEV)
    eo, es = run_prefill(x, chunk, algo=algo)
    report(f"prefill random {algo} C={chunk} {case}", o=eo, state=es)
    tol = TOL[w.dtype]
    assert eo <= tol and es <= tol


# ---------------------------------------------------------------------------
# state-only calls (o = NULL) and zero values (v = NULL)
@pytest.mark.parametrize("algo,chunk", [("fused", 64), ("two_pass", 64), ("two_pass", 128)])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 32), (torch.float32, 64),
                                     (torch.float32, 128)])
def test_prefill_state_only(dtype, d, algo, chunk):
    if not algo_ok(algo, dtype, d, chunk):
        pytest.skip(f"{algo} does not take {dtype} d={d} C={chunk}")
    w = inputs.custom(H=3, dk=d, dv=d, seqlens=[100, 0, 64, 1, 200], state_std=0.1, dtype=dtype)
    x = inputs.prefill_inputs(w, seed=60 + d, device=DEV)
    args = (x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    kw = dict(chunk_size=chunk, algo=algo)
    _, sf_full = kda.chunk_fwd(x["q"], *args, **kw)
    o_none, sf = kda.chunk_fwd(None, *args, output=False, **kw)
    torch.cuda.synchronize()
    assert o_none is None
    # the state path is the same arithmetic with or without the output
    es_full = rel_err(sf, sf_full.cpu().double().numpy())
    # zero values: the oracle with v = 0
    _, sz = kda.chunk_fwd(None, x["k"], None, x["g"], x["beta"], x["initial_state"],
                          x["cu_seqlens"], output=False, **kw)
    torch.cuda.synchronize()
    cpu = lambda t: t.cpu()
    _, sz_ref = oracle.forward(cpu(x["q"]), cpu(x["k"]), torch.zeros_like(cpu(x["v"])),
                               cpu(x["g"]), cpu(x["beta"]), cpu(x["initial_state"]),
                               x["cu_seqlens"].cpu().numpy())
    _, sf_ref = oracle.forward(cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), cpu(x["g"]),
                               cpu(x["beta"]), cpu(x["initial_state"]),
                               x["cu_seqlens"].cpu().numpy())
    es, ez = rel_err(sf, sf_ref), rel_err(sz, sz_ref)
    report(f"prefill state only {algo} C={chunk} {dtype} d={d}", vs_full=es_full, state=es,
           zero_v=ez)
    assert es_full <= 1e-6 and es <= TOL[dtype] and ez <= TOL[dtype]


def test_binding_rejects_mismatched_outputs():
    # preallocated outputs must match exactly: the kernels write every element
    w = inputs.custom(H=2, dk=32, dv=32, seqlens=[64], dtype=torch.float32)
    x = inputs.prefill_inputs(w, seed=3, device=DEV)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"])
    with pytest.raises(ValueError, match="out must have shape"):
        kda.chunk_fwd(*args, out=torch.empty(63, 2, 32, device=DEV))
    with pytest.raises(ValueError, match="final_state must have shape"):
        kda.chunk_fwd(*args, final_state=torch.empty(1, 2, 32, 16, device=DEV))
    wd = inputs.custom(H=2, dk=32, dv=32, dtype=torch.float32, decode_requests=3)
    xd = inputs.decode_inputs(wd, seed=3, device=DEV)
    with pytest.raises(ValueError, match="out must have shape"):
        kda.step_decode(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["state"],
                        out=torch.empty(2, 2, 32, device=DEV))
    M = torch.zeros(4, 32, 32, device=DEV)
    with pytest.raises(ValueError, match="out must have shape"):
        kda.state_compose(M, M, M, out=torch.empty(3, 32, 32, device=DEV))


# ---------------------------------------------------------------------------
# fp32 attention output from bf16 inputs (kda_chunk_fwd_ex)
@pytest.mark.parametrize("algo,chunk", [("fused", 64), ("two_pass", 64), ("two_pass", 128)])
@pytest.mark.parametrize("d", [128, 64, 32])
def test_prefill_fp32_output(d, algo, chunk):
    w = inputs.custom(H=3, dk=d, dv=d, seqlens=[130, 0, 64, 7], state_std=0.05,
                      dtype=torch.bfloat16)
    x = inputs.prefill_inputs(w, seed=90 + d, device=DEV)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["initial_state"], x["cu_seqlens"])
    o16, s16 = kda.chunk_fwd(*args, chunk_size=chunk, algo=algo)
    o32, s32 = kda.chunk_fwd(*args, o_dtype=torch.float32, chunk_size=chunk, algo=algo)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32 and o16.dtype == torch.bfloat16
    # the same arithmetic up to the store: the bf16 output is the rounded fp32 one,
    # and the states do not depend on the output type
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(s32, s16)
    cpu = lambda t: t.cpu()
    o_ref, s_ref = oracle.forward(*(cpu(t) for t in args[:6]), x["cu_seqlens"].cpu().numpy())
    eo, es = rel_err(o32, o_ref), rel_err(s32, s_ref)
    report(f"prefill fp32 output {algo} C={chunk} d={d}", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2
