"""fp64 oracle for the steps around the KDA recurrence in a KDA layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py; the HIP library never calls it.

Each function is the plain definition the pages give, written out in numpy
float64 with explicit loops where the order matters (the causal convolution,
the segment composition).  Readings of points the pages leave open are stated
where they are taken.

Sources (pages by title, table or entry):
  - "Notations mathematiques", table "Attention et KDA": rows q_t, k_t (L2
    normalised), g_t in (g_min, 0), g_min = -5, A_h (learned per-head log
    scale), b_alpha^h (per-head decay bias in R^{d_k}), z_t (decay logit),
    M_t (transition), S~ (state computed from S = 0), o~_t (raw output before
    the gate).
  - same page, table of functions: L2Norm(x) = x / ||x||_2,
    RMSNorm(x) = x / sqrt(mean(x^2) + eps) (.) g, ShortConv = causal
    convolution with a kernel of size 4, sigma = logistic function.
  - "Glossaire", entry "Decroissance bornee": g = g_min sigma(e^A z).
  - "Glossaire", entry "KCP": a segment is summarised by its transition and by
    the state it reaches from zero; summaries compose associatively.
  - "Glossaire", entry "ShortConv": causal convolution over a short window,
    kernel 4 in K3.
  - "Kimi K3" model tables: RMSNorm epsilon 1e-5; ShortConv kernel 4;
    full-rank KDA output gate; g_min = -5.
"""
from __future__ import annotations

import numpy as np

G_MIN = -5.0
RMS_EPS = 1e-5
CONV_K = 4


def sigmoid(x):
    """Logistic function 1 / (1 + e^-x), written to stay finite for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def l2norm(x):
    """L2Norm over the last axis: x / ||x||_2.  The pages give no epsilon;
    reading: a zero vector maps to zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def bounded_gate(z, A_log, b_alpha, g_min: float = G_MIN):
    """Log-decay of the bounded gate: g = g_min * sigma(e^{A_h} (z + b_alpha^h)).

    z: [..., H, d_k] decay logits; A_log: [H] (the per-head log scale A_h);
    b_alpha: [H, d_k].  The glossary writes g_min sigma(e^A z); the notation
    table adds the per-head bias b_alpha^h.  Reading: the bias is added to the
    logit before the scale."""
    z = np.asarray(z, dtype=np.float64)
    A = np.asarray(A_log, dtype=np.float64)
    b = np.asarray(b_alpha, dtype=np.float64)
    return g_min * sigmoid(np.exp(A)[:, None] * (z + b))


def rmsnorm(x, w, eps: float = RMS_EPS):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * np.asarray(w, dtype=np.float64)


def output_gate(o_raw, gate_logits, w, eps: float = RMS_EPS):
    """Layer output from the raw recurrent output: RMSNorm(o~) (.) sigma(G).

    o_raw, gate_logits: [..., d_v]; w: [d_v] (one RMSNorm weight shared by the
    heads).  Reading of "full-rank gate": one sigmoid gate logit per output
    channel, supplied by the caller."""
    return rmsnorm(o_raw, w, eps) * sigmoid(gate_logits)


def short_conv(x, w, cu_seqlens=None, conv_state=None):
    """Causal depthwise convolution with a kernel of CONV_K taps, per channel.

    x: [N_tok, C] packed sequences (cu_seqlens [N+1], or one sequence);
    w: [C, CONV_K]; tap i multiplies x_{t - (CONV_K - 1) + i}, so tap
    CONV_K - 1 is the current token.  Inputs before a sequence start come from
    conv_state [N, CONV_K - 1, C] (oldest first) or are zero.  No activation
    (the pages name none).  Returns (y [N_tok, C], final conv state
    [N, CONV_K - 1, C]: the last CONV_K - 1 inputs of each sequence, with the
    entering state in front when the sequence is shorter)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n_tok, C = x.shape
    cu = np.array([0, n_tok] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    state = (np.zeros((N, CONV_K - 1, C)) if conv_state is None
             else np.array(conv_state, dtype=np.float64))
    y = np.zeros_like(x)
    new_state = np.zeros((N, CONV_K - 1, C))
    for n in range(N):
        hist = [state[n, j] for j in range(CONV_K - 1)]   # oldest first
        for t in range(cu[n], cu[n + 1]):
            window = hist[-(CONV_K - 1):] + [x[t]]
            acc = np.zeros(C)
            for i in range(CONV_K):
                acc += w[:, i] * window[i]
            y[t] = acc
            hist.append(x[t])
        for j in range(CONV_K - 1):
            new_state[n, j] = hist[len(hist) - (CONV_K - 1) + j]
    return y, new_state


def transition_product(k, g, beta):
    """M = M_T ... M_1 for one segment of one head, M_t = (I - b k k^T) Diag(e^g).

    k, g: [T, d_k]; beta: [T].  Applied one token at a time from the left as
    M <- Diag(alpha) M, then M <- M - beta k (k^T M)."""
    k = np.asarray(k, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    d = k.shape[1]
    M = np.eye(d)
    for t in range(k.shape[0]):
        M = np.exp(g[t])[:, None] * M
        M = M - beta[t] * np.outer(k[t], k[t] @ M)
    return M


def kcp_compose(M2, S2, M1, S1):
    """Summary of segment 1 followed by segment 2: (M2 M1, M2 S1 + S2)."""
    M1, S1, M2, S2 = (np.asarray(a, dtype=np.float64) for a in (M1, S1, M2, S2))
    return M2 @ M1, M2 @ S1 + S2


def kcp_scan(Ms, Ss, S0=None):
    """States entering each segment and the final state, from the per-segment
    summaries (M_r, S~_r), r = 0..P-1, in order: S_in[0] = S0 (or zero),
    S_in[r + 1] = M_r S_in[r] + S~_r.  Returns (S_in [P, d_k, d_v], S_final)."""
    Ms = np.asarray(Ms, dtype=np.float64)
    Ss = np.asarray(Ss, dtype=np.float64)
    P, dk, dv = Ss.shape
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    S_in = np.zeros((P, dk, dv))
    for r in range(P):
        S_in[r] = S
        S = Ms[r] @ S + Ss[r]
    return S_in, S
