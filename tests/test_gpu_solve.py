"""Parity of the in-chunk solve under correlated keys.

With i.i.d. unit keys the in-chunk matrix A = StrictTril(B (K o e^G)(K o e^-G)^T)
has entries of about 1/sqrt(d_k), and (I + A)^-1 is close to I - A: a mistake in
the higher-order part of the solve (the inverse of a diagonal 16 x 16 block,
the off-diagonal blocks of A, the order of the block forward substitution)
barely moves the output.  Here the keys of each run of tokens share one
direction (k_t = normalise(b + eps n_t), see inputs.Workload), beta is close to
one and the decay is off or small, so A has entries close to beta and its
inverse differs from I - A by terms of order one: every part of the solve
shows in o and in the final state.  The runs are 16 tokens (one diagonal
block), 64 (a whole chunk, so the off-diagonal blocks of A are large too) or a
whole sequence.

The update M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) of page "Notations
mathematiques" (table "Attention et KDA") is what the oracle evaluates token by
token; the chunk algorithm is the UT transform of the "Glossaire" entry "UT".

Tolerances as in the other parity tests: bf16 inputs 2e-2 of max |ref| for o
and the final state, fp32 inputs 1e-4.
"""
import numpy as np
import pytest
import torch

from linear_attention_recurrence_chunk_amd import inputs
from test_gpu_parity import ALGOS, DEV, TOL, algo_ok, report, run_prefill

pytestmark = pytest.mark.gpu

GATES = {"no_decay": dict(gate_const=0.0),
         "k3_gate": dict(gate_mu=1.0, gate_sigma=1.0),
         "extreme_gate": dict(gate_mu=3.0, gate_sigma=0.5)}
BETAS = {"beta_0.99": dict(beta_const=0.99),
         "beta_sigmoid_N(2,1)": dict(beta_mu=2.0, beta_sigma=1.0)}
TYPES = [(torch.bfloat16, 32), (torch.bfloat16, 64), (torch.bfloat16, 128),
         (torch.float32, 32), (torch.float32, 64), (torch.float32, 128)]
# (algorithm, chunk size) pairs of kda_chunk_fwd_algo
PATHS = [("fused", 64), ("two_pass", 64), ("two_pass", 128)]
PATH_IDS = [f"{a}-C{c}" for a, c in PATHS]
LENS = [200, 64, 0, 17, 1, 130]   # chunk and sub-block edges, ragged tails


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("gate", list(GATES))
@pytest.mark.parametrize("beta", list(BETAS))
@pytest.mark.parametrize("eps", [0.05, 0.2])
@pytest.mark.parametrize("dtype,d", TYPES, ids=lambda x: str(x).replace("torch.", ""))
def test_correlated_keys_16_token_runs(dtype, d, eps, beta, gate, path):
    algo, chunk = path
    if not algo_ok(algo, dtype, d, chunk):
        pytest.skip(f"{algo} does not take {dtype} d={d} C={chunk}")
    w = inputs.custom(H=3, dk=d, dv=d, seqlens=LENS, dtype=dtype, state_std=0.05,
                      key_block=16, key_eps=eps, **BETAS[beta], **GATES[gate])
    x = inputs.prefill_inputs(w, seed=1000 + d + int(100 * eps), device=DEV)
    eo, es = run_prefill(x, chunk, algo=algo)
    report(f"correlated keys (16) {algo} C={chunk} {dtype} d={d} eps={eps} {beta} {gate}",
           o=eo, state=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("eps", [0.0, 0.05])
@pytest.mark.parametrize("dtype,d", TYPES, ids=lambda x: str(x).replace("torch.", ""))
def test_correlated_keys_whole_chunk_runs(dtype, d, eps, path):
    # one direction per 64 tokens, beta = 1 (eps = 0: identical keys in a chunk,
    # so A is beta times the strictly lower all-ones matrix), no decay
    algo, chunk = path
    if not algo_ok(algo, dtype, d, chunk):
        pytest.skip(f"{algo} does not take {dtype} d={d} C={chunk}")
    w = inputs.custom(H=2, dk=d, dv=d, seqlens=[256, 100, 65], dtype=dtype, state_std=0.05,
                      key_block=64, key_eps=eps, beta_const=1.0, gate_const=0.0)
    x = inputs.prefill_inputs(w, seed=2000 + d, device=DEV)
    eo, es = run_prefill(x, chunk, algo=algo)
    report(f"correlated keys (64) {algo} C={chunk} {dtype} d={d} eps={eps}", o=eo, state=es)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("d", [32, 64, 128])
def test_correlated_keys_whole_sequence_fp32(d, path):
    # keys close to one direction over the whole sequence with no decay: the
    # hardest conditioning for the solve; the fp32 path holds 1e-4 there
    algo, chunk = path
    if not algo_ok(algo, torch.float32, d, chunk):
        pytest.skip(f"{algo} does not take fp32 d={d} C={chunk}")
    w = inputs.custom(H=2, dk=d, dv=d, seqlens=[512], dtype=torch.float32, state_std=0.05,
                      key_block=512, key_eps=0.01, beta_const=0.99, gate_const=0.0)
    x = inputs.prefill_inputs(w, seed=3000 + d, device=DEV)
    eo, es = run_prefill(x, chunk, algo=algo)
    report(f"correlated keys (512) {algo} C={chunk} fp32 d={d}", o=eo, state=es)
    assert eo <= 1e-4 and es <= 1e-4


@pytest.mark.parametrize("chunk", [64, 128])
def test_correlated_keys_k3_heads(chunk):
    # K3 head count and size (H = 96, d = 128, so every XCD slot of the work
    # mapping is used), half the heads with runs of 16 similar keys
    w = inputs.custom(H=96, dk=128, dv=128, seqlens=[1000, 333], state_std=0.02,
                      key_block=16, key_eps=0.1, beta_mu=2.0, beta_sigma=1.0)
    x = inputs.prefill_inputs(w, seed=4000 + chunk, device=DEV)
    eo, es = run_prefill(x, chunk)
    report(f"correlated keys K3 heads C={chunk}", o=eo, state=es)
    assert eo <= 2e-2 and es <= 2e-2
