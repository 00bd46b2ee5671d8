"""Second oracle for tiny shapes: the recurrence with the explicit transition matrix.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Page "Notations mathematiques", table "Attention et KDA": the transition of a
token is the d_k x d_k matrix M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), the
state is S_t = M_t S_{t-1} + beta_t k_t v_t^T, alpha_t = exp(g_t) (rows
"alpha_t" and "g_t"), and the output read after the write is o_t = S_t^T q_t.
This module forms M_t as a dense matrix and multiplies, which is O(d_k^2 d_v)
per token: use it for d <= 16 and short sequences only.
"""
from __future__ import annotations

import numpy as np


def transition(k_t: np.ndarray, g_t: np.ndarray, beta_t: float) -> np.ndarray:
    """M_t = (I - beta k k^T) Diag(exp(g))."""
    k_t = np.asarray(k_t, dtype=np.float64)
    d = k_t.shape[0]
    return (np.eye(d) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.exp(np.asarray(g_t, np.float64)))


def forward_single(q, k, v, g, beta, s0=None):
    """One sequence, one head.  q, k, g [T, dk]; v [T, dv]; beta [T]; s0 [dk, dv].
    Returns (o [T, dv], S_T [dk, dv])."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S = transition(k[t], g[t], beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def forward(q, k, v, g, beta, initial_state=None, cu_seqlens=None):
    """Packed layout like the C oracle: q, k, g [N_tok, H, dk] ... ."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    n_tok, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.array([0, n_tok]) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((n_tok, H, dv))
    sf = np.zeros((N, H, dk, dv))
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            s0 = None if initial_state is None else np.asarray(initial_state, np.float64)[n, h]
            o[a:b, h], sf[n, h] = forward_single(q[a:b, h], k[a:b, h], v[a:b, h],
                                                 g[a:b, h], beta[a:b, h], s0)
    return o, sf
