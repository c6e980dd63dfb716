"""Quadratic (masked-matrix) forms of the Lightning Attention layer, numpy fp64.

TEST INFRASTRUCTURE ONLY.  Tiny sizes: memory is O(N^2) per head.

With the decay matrix D[t, s] = lambda^(t-s) for s <= t (0 above the diagonal),
lambda = exp(-slope), these are the textbook masked-attention expressions of
the same definition the recurrent oracle evaluates token by token:

    O   = ((Q K^T) * D) V + diag(lambda^(t+1)) Q S0
    S_N = K^T diag(lambda^(N-1-s)) V + lambda^N S0
    dQ  = ((dO V^T) * D) K + diag(lambda^(t+1)) dO S0^T
    dK  = ((dO V^T) * D)^T Q
    dV  = ((Q K^T) * D)^T dO

(* is the elementwise product.)  The backward lines follow from
L = sum(O * dO) by differentiating the first line.
"""
from __future__ import annotations

import numpy as np


def decay_matrix(slope: float, N: int) -> np.ndarray:
    s = float(np.float32(slope))
    t = np.arange(N, dtype=np.float64)
    diff = t[:, None] - t[None, :]
    D = np.exp(-s * np.where(diff >= 0, diff, 0.0))
    return np.where(diff >= 0, D, 0.0)


def fwd(q, k, v, slope, S0=None):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, N, d = q.shape
    o = np.zeros_like(q)
    S = np.zeros((B, H, d, d))
    t = np.arange(N, dtype=np.float64)
    for h in range(H):
        s = float(np.float32(slope[h]))
        D = decay_matrix(s, N)
        for b in range(B):
            Q, K, V = q[b, h], k[b, h], v[b, h]
            o[b, h] = ((Q @ K.T) * D) @ V
            S[b, h] = K.T @ (np.exp(-s * (N - 1 - t))[:, None] * V)
            if S0 is not None:
                S0bh = np.asarray(S0[b, h], dtype=np.float64)
                o[b, h] += np.exp(-s * (t + 1))[:, None] * (Q @ S0bh)
                S[b, h] += np.exp(-s * N) * S0bh
    return o, S


def bwd(q, k, v, dout, slope, S0=None):
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, H, N, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    t = np.arange(N, dtype=np.float64)
    for h in range(H):
        s = float(np.float32(slope[h]))
        D = decay_matrix(s, N)
        for b in range(B):
            Q, K, V, G = q[b, h], k[b, h], v[b, h], g[b, h]
            A = (G @ V.T) * D
            P = (Q @ K.T) * D
            dq[b, h] = A @ K
            dk[b, h] = A.T @ Q
            dv[b, h] = P.T @ G
            if S0 is not None:
                S0bh = np.asarray(S0[b, h], dtype=np.float64)
                dq[b, h] += np.exp(-s * (t + 1))[:, None] * (G @ S0bh.T)
    return dq, dk, dv
