"""ctypes wrapper around the C recurrent oracle (la_oracle.c).

TEST INFRASTRUCTURE ONLY (see the package docstring).  All arrays are converted
to contiguous float64 before the call; the slope stays fp32, the exact values
handed to the GPU, and the decay is exp(-(double)slope) inside the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(force: bool = False) -> str:
    """Compile la_oracle.c with gcc (-O2, OpenMP).  Plain C, no GPU code."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.lao_fwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P]
        lib.lao_fwd_chunked.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.lao_decode.argtypes = [I, I, I, P, P, P, P, P, P]
        lib.lao_bwd.argtypes = [I, I, I, I, P, P, P, P, P, P, P, P, P]
        lib.lao_num_threads.restype = I
        for f in (lib.lao_fwd, lib.lao_fwd_chunked, lib.lao_decode, lib.lao_bwd):
            f.restype = None
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _slope(s):
    return np.ascontiguousarray(s, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def num_threads() -> int:
    return _load().lao_num_threads()


def fwd(q, k, v, slope, S0=None):
    """Recurrent forward.  q, k, v: [B,H,N,d]; slope: [H]; S0: [B,H,d,d] or None.

    Returns (o [B,H,N,d], S_N [B,H,d,d]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    s = _slope(slope)
    assert s.shape == (H,)
    S0 = None if S0 is None else _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, d, d)
    o = np.empty_like(q)
    S = np.empty((B, H, d, d), dtype=np.float64)
    _load().lao_fwd(B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(S0), _ptr(o), _ptr(S))
    return o, S


def fwd_chunked(q, k, v, slope, C, S0=None):
    """Chunked-order forward (same definition, different evaluation order)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    s = _slope(slope)
    S0 = None if S0 is None else _f64(S0)
    o = np.empty_like(q)
    S = np.empty((B, H, d, d), dtype=np.float64)
    _load().lao_fwd_chunked(
        B, H, N, d, int(C), _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(S0), _ptr(o), _ptr(S)
    )
    return o, S


def decode(q, k, v, slope, state):
    """One decode step.  q, k, v: [B,H,d]; state: [B,H,d,d] (not modified).

    Returns (o [B,H,d], new_state [B,H,d,d])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, d = q.shape
    s = _slope(slope)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    o = np.empty_like(q)
    _load().lao_decode(B, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(s), _ptr(st), _ptr(o))
    return o, st


def bwd(q, k, v, dout, slope, S0=None):
    """Gradients (dq, dk, dv) of L = sum(o * dout)."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    s = _slope(slope)
    S0 = None if S0 is None else _f64(S0)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    _load().lao_bwd(
        B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s), _ptr(S0), _ptr(dq), _ptr(dk), _ptr(dv)
    )
    return dq, dk, dv


def _check_cu(cu, T):
    cu = [int(x) for x in cu]
    assert len(cu) >= 2 and cu[0] == 0 and cu[-1] == T, "cu_seqlens must run from 0 to T"
    assert all(a <= b for a, b in zip(cu, cu[1:])), "cu_seqlens must be non-decreasing"
    return cu


def fwd_varlen(q, k, v, slope, cu_seqlens, S0=None):
    """Packed sequences.  q, k, v: [H,T,d]; sequence s holds tokens
    cu_seqlens[s] .. cu_seqlens[s+1]-1 of every head; S0: [nseq,H,d,d] or None.

    Every sequence is its own recurrence from its own initial state (the
    varlen batches of the "Context Parallel for Lightning Attention" section,
    and prefix caching on the "linghe" section: a cached state continues a
    sequence).  Returns (o [H,T,d], S [nseq,H,d,d]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, T, d = q.shape
    cu = _check_cu(cu_seqlens, T)
    nseq = len(cu) - 1
    o = np.empty_like(q)
    S = np.empty((nseq, H, d, d), dtype=np.float64)
    for s in range(nseq):
        a, b = cu[s], cu[s + 1]
        init = None if S0 is None else _f64(S0)[s][None]
        o_s, S_s = fwd(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], slope, init)
        o[:, a:b] = o_s[0]
        S[s] = S_s[0]
    return o, S


def bwd_varlen(q, k, v, dout, slope, cu_seqlens):
    """Gradients (dq, dk, dv) [H,T,d] of L = sum(o * dout) for packed
    sequences with zero initial states."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    H, T, d = q.shape
    cu = _check_cu(cu_seqlens, T)
    dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        r = bwd(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], g[None, :, a:b], slope)
        dq[:, a:b], dk[:, a:b], dv[:, a:b] = (x[0] for x in r)
    return dq, dk, dv


def gated_group_rmsnorm(o, gate, weight, eps):
    """The output epilogue of the "linghe" section (Group RMSNorm + Sigmoid
    Gate), one group per head:

        y[..., h, t, j] = o[..., h, t, j] / sqrt(mean_j' o[..., h, t, j']^2 + eps)
                          * weight[h, j] * sigmoid(gate[..., h, t, j])

    o, gate: [..., H, N, d]; weight: [H, d]; all in float64."""
    o, g = _f64(o), _f64(gate)
    w = np.asarray(weight, dtype=np.float64)
    assert g.shape == o.shape and w.shape == o.shape[-3:-2] + o.shape[-1:]
    ms = np.mean(o * o, axis=-1, keepdims=True)
    sig = 1.0 / (1.0 + np.exp(-g))
    return o / np.sqrt(ms + float(eps)) * w[:, None, :] * sig


def fwd_gated(q, k, v, slope, gate, weight, eps, S0=None):
    """Forward followed by the gated group RMSNorm of its output.  Returns
    (y [B,H,N,d], S_N [B,H,d,d])."""
    o, S = fwd(q, k, v, slope, S0)
    return gated_group_rmsnorm(o, gate, weight, eps), S
