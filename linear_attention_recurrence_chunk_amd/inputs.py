"""Seeded synthetic inputs for the KDA recurrence.

This module is shared by the oracle side and the HIP side of every test and of
the benchmark.  It holds no part of the recurrence: it only draws tensors with
the distributions of the workloads below and returns them.  The value recipe
per (token, head):

* q, k ~ N(0, 1) per channel, then divided by their L2 norm in fp32 (the layer
  applies L2Norm to queries and keys before the recurrence: page "Vecteurs,
  embeddings, espaces de representation", section on norms, and page
  "Notations mathematiques", table "Attention et KDA", rows q_t, k_t), then
  cast to the storage dtype (round to nearest even for bf16);
* v ~ N(0, 1);
* beta = sigmoid(z_b), z_b ~ N(0, 1), fp32 (write strength in (0, 1));
* g = -5 * sigmoid(z_g), z_g ~ N(mu, sigma) per channel, fp32, so g lies in
  (g_min, 0) with g_min = -5 (rows g_t and g_min of the same table);
* initial states ~ N(0, std) fp32 when a workload asks for one.

N(mu, s) is read with s the standard deviation.  Every tensor is token-major
and packed: [N_tok, H, d]; B equal sequences of length T are the packed layout
with cu_seqlens = [0, T, 2T, ...].  Draws use one torch.Generator seeded with
the given seed on the target device, in a fixed order (lengths, q, k, v, z_g,
z_b, initial state), so a (workload, seed, device) triple always yields the
same tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import torch

G_MIN = -5.0


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``seqlens`` is None for B equal sequences of T."""
    name: str
    H: int
    dk: int
    dv: int
    chunk: int = 64
    B: int = 1
    T: int = 0
    seqlens: Optional[Sequence[int]] = None
    random_lengths: Optional[tuple] = None      # (count, lo, hi) inclusive
    dtype: torch.dtype = torch.bfloat16          # q, k, v (and o) storage type
    gate_mu: float = 1.0
    gate_sigma: float = 1.0
    extreme_heads: int = 0                       # heads [0, extreme_heads) use the extreme gate
    extreme_mu: float = 3.0
    extreme_sigma: float = 0.5
    state_std: float = 0.0                       # 0 -> no initial state
    decode_requests: int = 0                     # >0 -> a one-token decode workload
    # Correlated keys (stress of the in-chunk solve): with key_block > 0, the
    # keys of each run of key_block tokens from a sequence start share one
    # random unit direction b, k_t = normalise(b + key_eps * n_t), n_t ~
    # N(0, 1/d_k) per channel (|n_t| ~ 1).  key_block = 0: i.i.d. keys.
    key_block: int = 0
    key_eps: float = 0.0
    # beta = beta_const everywhere when given, else sigmoid(N(beta_mu, beta_sigma))
    beta_mu: float = 0.0
    beta_sigma: float = 1.0
    beta_const: Optional[float] = None
    # g = gate_const everywhere when given (0: no decay), else the gate above
    gate_const: Optional[float] = None


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 case the oracle finishes at once.
    "tiny_fp32": Workload("tiny_fp32", H=2, dk=32, dv=32, chunk=64, B=1, T=256,
                          dtype=torch.float32, gate_mu=0.0, gate_sigma=1.0),
    # One 8K-token sequence of a K3 KDA layer (H=96, d=128).
    "k3_prefill_8k": Workload("k3_prefill_8k", H=96, dk=128, dv=128, chunk=64, B=1, T=8192),
    # Long context: one 128K-token sequence, C=128 (1024 chunks).
    "k3_prefill_128k": Workload("k3_prefill_128k", H=96, dk=128, dv=128, chunk=128, B=1,
                                T=131072),
    # 16 packed sequences of 512..16384 tokens with prefix states; half the heads
    # use a gate close to g_min.
    "k3_varlen_prefix": Workload("k3_varlen_prefix", H=96, dk=128, dv=128, chunk=64,
                                 random_lengths=(16, 512, 16384), state_std=0.02,
                                 extreme_heads=48),
    # One decode step for 256 requests with fp32 states ~ N(0, 0.02).
    "k3_decode_256": Workload("k3_decode_256", H=96, dk=128, dv=128, decode_requests=256,
                              state_std=0.02),
    # nano-K3 (the toy model of the pages: 8 heads x 64, context 2048): a batch
    # of 32 full-context sequences, and one decode step for 256 requests.
    "nano_k3_prefill": Workload("nano_k3_prefill", H=8, dk=64, dv=64, chunk=64, B=32, T=2048),
    "nano_k3_decode": Workload("nano_k3_decode", H=8, dk=64, dv=64, decode_requests=256,
                               state_std=0.02),
}


def _gen(seed: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _unit_rows(shape, gen, device, dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.to(dtype)


def _gate(shape, H, w: Workload, gen, device) -> torch.Tensor:
    mu = torch.full((H, 1), w.gate_mu, device=device, dtype=torch.float32)
    sd = torch.full((H, 1), w.gate_sigma, device=device, dtype=torch.float32)
    if w.extreme_heads:
        mu[: w.extreme_heads] = w.extreme_mu
        sd[: w.extreme_heads] = w.extreme_sigma
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * sd + mu
    return G_MIN * torch.sigmoid(z)


def sequence_lengths(w: Workload, seed: int) -> List[int]:
    """Lengths of the packed sequences (drawn on the CPU so every device agrees)."""
    if w.seqlens is not None:
        return [int(x) for x in w.seqlens]
    if w.random_lengths is not None:
        cnt, lo, hi = w.random_lengths
        gen = _gen(seed, "cpu")
        return torch.randint(lo, hi + 1, (cnt,), generator=gen).tolist()
    return [w.T] * w.B


def _correlated_keys(lens, w: Workload, gen, device) -> torch.Tensor:
    """Keys that share a direction within runs of w.key_block tokens of each
    sequence (see Workload)."""
    n_tok, H, dk = int(sum(lens)), w.H, w.dk
    blk_of = []
    nblk = 0
    for L in lens:
        blk_of.append(torch.arange(L) // w.key_block + nblk)
        nblk += (L + w.key_block - 1) // w.key_block
    idx = torch.cat(blk_of).to(device) if blk_of else torch.zeros(0, dtype=torch.int64, device=device)
    base = _unit_rows((max(nblk, 1), H, dk), gen, device, torch.float32)
    noise = torch.randn((n_tok, H, dk), generator=gen, device=device, dtype=torch.float32)
    x = base[idx] + (w.key_eps / dk ** 0.5) * noise
    x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    return x.to(w.dtype)


def prefill_inputs(w: Workload, seed: int, device="cpu") -> dict:
    """q, k [N_tok, H, dk]; v [N_tok, H, dv]; g [N_tok, H, dk] fp32; beta
    [N_tok, H] fp32; initial_state [N, H, dk, dv] fp32 or None; cu_seqlens
    [N + 1] int32 on ``device``; plus ``seqlens`` (host list)."""
    lens = sequence_lengths(w, seed)
    n_tok = int(sum(lens))
    gen = _gen(seed, device)
    H, dk, dv = w.H, w.dk, w.dv
    q = _unit_rows((n_tok, H, dk), gen, device, w.dtype)
    if w.key_block > 0:
        k = _correlated_keys(lens, w, gen, device)
    else:
        k = _unit_rows((n_tok, H, dk), gen, device, w.dtype)
    v = torch.randn((n_tok, H, dv), generator=gen, device=device, dtype=torch.float32).to(w.dtype)
    g = _gate((n_tok, H, dk), H, w, gen, device)
    if w.gate_const is not None:
        g.fill_(w.gate_const)
    beta = torch.sigmoid(torch.randn((n_tok, H), generator=gen, device=device,
                                     dtype=torch.float32) * w.beta_sigma + w.beta_mu)
    if w.beta_const is not None:
        beta.fill_(w.beta_const)
    s0 = None
    if w.state_std > 0:
        s0 = torch.randn((len(lens), H, dk, dv), generator=gen, device=device,
                         dtype=torch.float32) * w.state_std
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0,
                cu_seqlens=cu.to(device), seqlens=lens)


def decode_inputs(w: Workload, seed: int, device="cpu", requests: Optional[int] = None) -> dict:
    """One token per request: q, k [N, H, dk]; v [N, H, dv]; g, beta fp32;
    state [N, H, dk, dv] fp32 ~ N(0, state_std)."""
    N = int(requests if requests is not None else w.decode_requests)
    gen = _gen(seed, device)
    H, dk, dv = w.H, w.dk, w.dv
    q = _unit_rows((N, H, dk), gen, device, w.dtype)
    k = _unit_rows((N, H, dk), gen, device, w.dtype)
    v = torch.randn((N, H, dv), generator=gen, device=device, dtype=torch.float32).to(w.dtype)
    g = _gate((N, H, dk), H, w, gen, device)
    beta = torch.sigmoid(torch.randn((N, H), generator=gen, device=device, dtype=torch.float32))
    state = torch.randn((N, H, dk, dv), generator=gen, device=device,
                        dtype=torch.float32) * (w.state_std if w.state_std > 0 else 1.0)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state=state)


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit fields (tests use it for edge shapes)."""
    return Workload(name=name, **kw)


def layer_inputs(w: Workload, seed: int, device="cuda") -> Dict[str, torch.Tensor]:
    """Raw inputs of the layer steps for a prefill workload (no normalisation,
    no gate applied): q_raw, k_raw ~ N(0, 1) and decay logits z ~ N(gate_mu,
    gate_sigma) in the workload dtype; A_log = 0 and b_alpha = 0 (so that the
    bounded gate reproduces the workload's g distribution); output-gate logits
    ~ N(0, 1); RMSNorm weight ~ N(1, 0.1); ShortConv taps ~ N(0, 0.5) over the
    H * d_k channels of one projection."""
    gen = _gen(seed, device)
    n = sum(sequence_lengths(w, seed))
    r = lambda *s: torch.randn(*s, generator=gen, device=device)
    return {
        "q_raw": r(n, w.H, w.dk).to(w.dtype),
        "k_raw": r(n, w.H, w.dk).to(w.dtype),
        "z": (w.gate_mu + w.gate_sigma * r(n, w.H, w.dk)).to(w.dtype),
        "A_log": torch.zeros(w.H, device=device),
        "b_alpha": torch.zeros(w.H, w.dk, device=device),
        "gate": r(n, w.H, w.dv).to(w.dtype),
        "rms_weight": 1.0 + 0.1 * r(w.dv),
        "conv_w": 0.5 * r(w.H * w.dk, 4),
    }
