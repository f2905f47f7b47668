"""Gradients of exact attention in float64 (test infrastructure only).

For phi = <dO, O> with O = softmax(S) V and S = scale * Q K^T (masked), the
chain rule through the row softmax gives, row by row:

    dV = P^T dO,        dP = dO V^T,
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
    dQ = scale * dS K,  dK = scale * dS^T Q.

This is the backward pass that the Triton article's section on the core
idea (核心思想) asks to run by recomputing the score matrix instead of
storing it; here S and P are simply materialised from the definition (the
forward oracle's own steps), which is what a recomputation must reproduce.
Hidden scores have P = 0, so they get no gradient; a row with no visible key
contributes nothing.  Arrays are [B, H, N, d]; returns (dQ, dK, dV) float64.
"""

import numpy as np

from .exact_attention import _causal_mask, _f64


def attention_backward(q, k, v, do, scale, causal=False):
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h].T)
            if causal:
                S[_causal_mask(N, 0, k.shape[2])] = -np.inf
            m = S.max(axis=1)
            dead = ~np.isfinite(m)
            E = np.exp(S - np.where(dead, 0.0, m)[:, None])
            l = E.sum(axis=1)
            P = np.where(dead[:, None], 0.0, E / np.where(dead, 1.0, l)[:, None])
            dv[b, h] = P.T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ k[b, h])
            dk[b, h] = scale * (dS.T @ q[b, h])
    return dq, dk, dv
