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
L = sum(O * dO) by differentiating the first line.  For a packed (varlen)
batch the same forms hold with D made block-diagonal over the sequences and
each sequence's own initial state and token positions.
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


def _seq_ids(cu, T):
    ids = np.empty(T, dtype=np.int64)
    pos = np.empty(T, dtype=np.float64)
    for s in range(len(cu) - 1):
        ids[cu[s]:cu[s + 1]] = s
        pos[cu[s]:cu[s + 1]] = np.arange(cu[s + 1] - cu[s])
    return ids, pos


def packed_decay_matrix(slope: float, cu) -> np.ndarray:
    """D[t, u] = lambda^(t-u) when u <= t and both tokens belong to the same
    packed sequence, else 0: the block-diagonal mask of a varlen batch."""
    T = int(cu[-1])
    ids, _ = _seq_ids(cu, T)
    return decay_matrix(slope, T) * (ids[:, None] == ids[None, :])


def fwd_varlen(q, k, v, slope, cu, S0=None):
    """Packed forward, q, k, v: [H,T,d], S0: [nseq,H,d,d] or None:

        O   = ((Q K^T) * Dp) V + diag(lambda^(pos_t+1)) Q S0[seq(t)]
        S_s = K_s^T diag(lambda^(n_s-1-pos)) V_s + lambda^(n_s) S0[s]

    with Dp the block-diagonal decay mask and pos_t the position of token t
    inside its own sequence."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    H, T, d = q.shape
    cu = [int(x) for x in cu]
    nseq = len(cu) - 1
    ids, pos = _seq_ids(cu, T)
    o = np.zeros_like(q)
    S = np.zeros((nseq, H, d, d))
    for h in range(H):
        s = float(np.float32(slope[h]))
        Dp = packed_decay_matrix(s, cu)
        Q, K, V = q[h], k[h], v[h]
        o[h] = ((Q @ K.T) * Dp) @ V
        for j in range(nseq):
            a, b = cu[j], cu[j + 1]
            n = b - a
            w = np.exp(-s * (n - 1 - np.arange(n, dtype=np.float64)))
            S[j, h] = K[a:b].T @ (w[:, None] * V[a:b])
            if S0 is not None:
                S0j = np.asarray(S0[j, h], dtype=np.float64)
                o[h, a:b] += np.exp(-s * (pos[a:b] + 1))[:, None] * (Q[a:b] @ S0j)
                S[j, h] += np.exp(-s * n) * S0j
    return o, S


def bwd_varlen(q, k, v, dout, slope, cu):
    """Packed backward with zero initial states:
    dQ = ((dO V^T) * Dp) K,  dK = ((dO V^T) * Dp)^T Q,  dV = ((Q K^T) * Dp)^T dO."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    H, T, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for h in range(H):
        s = float(np.float32(slope[h]))
        Dp = packed_decay_matrix(s, cu)
        Q, K, V, G = q[h], k[h], v[h], g[h]
        A = (G @ V.T) * Dp
        P = (Q @ K.T) * Dp
        dq[h] = A @ K
        dk[h] = A.T @ Q
        dv[h] = P.T @ G
    return dq, dk, dv
