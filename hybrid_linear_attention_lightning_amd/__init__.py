"""Lightning Attention for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in include/lightning_la.h: argument marshalling
only.  Every step of the computation runs in the HIP kernels of
liblightning_la.so; there is no CPU or PyTorch fallback, and importing this
module fails loudly if the library cannot be built or loaded.  PyTorch is used
for device memory (tensors) and streams.

    o, S = prefill(q, k, v, slope, chunk=128)        # q, k, v: [B, H, N, d] cuda tensors
    o    = decode_step(q1, k1, v1, slope, S)          # S updated in place
    o    = decode_tokens(qK, kK, vK, slope, S)         # K tokens at once: [B, H, K, d]
    dq, dk, dv = prefill_bwd(q, k, v, dout, slope, chunk=64)
    o, S = prefill_varlen(q, k, v, slope, cu_seqlens, chunk=128)   # q: [H, T, d] packed

The operation (Ling & Ring 2.6 Technical Report pages, "Hybrid Linear
Attention" section): per head, lambda = exp(-slope[h]),
S_t = lambda S_{t-1} + k_t v_t^T and o_t = q_t^T S_t.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime this library links against

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblightning_la.so")

LA_F32, LA_BF16 = 0, 1
STATUS = {
    0: "LA_OK",
    1: "LA_ERR_NULL_POINTER",
    2: "LA_ERR_BAD_SHAPE",
    3: "LA_ERR_BAD_DTYPE",
    4: "LA_ERR_UNSUPPORTED",
    5: "LA_ERR_WORKSPACE",
    6: "LA_ERR_HIP",
    7: "LA_ERR_ALIGNMENT",
    8: "LA_ERR_ALIAS",
}

# every symbol the header declares, with its ctypes signature
_P, _I, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "la_prefill": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "la_prefill_prepass": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "la_prefill_gated": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                              _P, _P, _P, _Z, _P]),
    "la_prefill_main": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "la_decode_step": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "la_decode_tokens": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "la_prefill_bwd": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "la_prefill_bwd_reuse": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                                  _P]),
    "la_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "la_prefill_varlen": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "la_prefill_bwd_varlen": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "la_prefill_bwd_varlen_reuse": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "la_workspace_bytes_varlen": (_Z, [_I, _I, _I, _I, _I, _I, _P]),
    "la_status_string": (ctypes.c_char_p, [_I]),
    "la_abi_version": (_I, []),
}

_lib = None


class LightningError(RuntimeError):
    def __init__(self, fn, code, lib):
        msg = lib.la_status_string(code).decode() if lib is not None else ""
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(code, code), msg))
        self.code = code


def lib():
    """The loaded liblightning_la.so (built in-tree first if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build

            _build.build()
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _check(fn, code):
    if code != 0:
        raise LightningError(fn, code, _lib)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError("expected bfloat16 or float32 tensors, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_bytes(op: int, dtype: int, B: int, H: int, N: int, d: int, C: int) -> int:
    n = lib().la_workspace_bytes(op, dtype, B, H, N, d, C)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("arguments rejected by la_workspace_bytes")
    return n


def _workspace(nbytes: int, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None or ws.numel() * ws.element_size() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def prefill(q, k, v, slope, chunk=64, state_in=None, out=None, state_out=None,
            return_state=True, workspace=None, stream=None):
    """Chunked forward.  q, k, v: [B,H,N,d] bf16 or fp32; slope: [H] fp32.

    Returns (o, state_out) where state_out is [B,H,d,d] fp32 (None when
    return_state is False and no state_out tensor is given)."""
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("%s must match q in shape and dtype" % name)
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    nbytes = workspace_bytes(0, dt, B, H, N, d, chunk)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    code = lib().la_prefill(
        dt, B, H, N, d, chunk,
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(slope, "slope", torch.float32),
        None if state_in is None else _dev(state_in, "state_in", torch.float32),
        _dev(out, "out", q.dtype),
        None if state_out is None else _dev(state_out, "state_out", torch.float32),
        None if ws is None else ws.data_ptr(), wsb, _stream(stream),
    )
    _check("la_prefill", code)
    return out, state_out


def prefill_gated(q, k, v, slope, gate, norm_weight, eps=1e-6, chunk=64, state_in=None,
                  out=None, state_out=None, return_state=True, workspace=None, stream=None):
    """prefill with the fused output epilogue: y = RMSNorm_head(o) * norm_weight[h]
    * sigmoid(gate), gate like q, norm_weight [H, d] fp32.  Returns (y, state_out)."""
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("gate", gate)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("%s must match q in shape and dtype" % name)
    if tuple(norm_weight.shape) != (H, d):
        raise ValueError("norm_weight must be [H, d]")
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    nbytes = workspace_bytes(0, dt, B, H, N, d, chunk)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    code = lib().la_prefill_gated(
        dt, B, H, N, d, chunk,
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(slope, "slope", torch.float32),
        None if state_in is None else _dev(state_in, "state_in", torch.float32),
        _dev(gate, "gate", q.dtype), _dev(norm_weight, "norm_weight", torch.float32), float(eps),
        _dev(out, "out", q.dtype),
        None if state_out is None else _dev(state_out, "state_out", torch.float32),
        None if ws is None else ws.data_ptr(), wsb, _stream(stream),
    )
    _check("la_prefill_gated", code)
    return out, state_out


def prefill_prepass(k, v, slope, chunk, workspace, state_in=None, stream=None):
    """First half of `prefill`: segment start states into `workspace`
    (a uint8 cuda tensor of at least workspace_bytes(0, ...) bytes)."""
    B, H, N, d = k.shape
    dt = _dtype_code(k)
    nbytes = workspace_bytes(0, dt, B, H, N, d, chunk)
    code = lib().la_prefill_prepass(
        dt, B, H, N, d, chunk, _dev(k, "k"), _dev(v, "v", k.dtype),
        _dev(slope, "slope", torch.float32),
        None if state_in is None else _dev(state_in, "state_in", torch.float32),
        None if nbytes == 0 else _dev(workspace, "workspace"),
        0 if nbytes == 0 else workspace.numel() * workspace.element_size(), _stream(stream),
    )
    _check("la_prefill_prepass", code)


def prefill_main(q, k, v, slope, chunk, workspace, out, state_out=None, state_in=None,
                 stream=None):
    """Second half of `prefill`: all segments from the states prefill_prepass
    left in `workspace`."""
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    nbytes = workspace_bytes(0, dt, B, H, N, d, chunk)
    code = lib().la_prefill_main(
        dt, B, H, N, d, chunk, _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(slope, "slope", torch.float32),
        None if state_in is None else _dev(state_in, "state_in", torch.float32),
        _dev(out, "out", q.dtype),
        None if state_out is None else _dev(state_out, "state_out", torch.float32),
        None if nbytes == 0 else _dev(workspace, "workspace"),
        0 if nbytes == 0 else workspace.numel() * workspace.element_size(), _stream(stream),
    )
    _check("la_prefill_main", code)
    return out


def decode_step(q, k, v, slope, state, out=None, stream=None):
    """One decode step.  q, k, v: [B,H,d]; state: [B,H,d,d] fp32 updated in place."""
    B, H, d = q.shape
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    code = lib().la_decode_step(
        dt, B, H, d, _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(slope, "slope", torch.float32), _dev(state, "state", torch.float32),
        _dev(out, "out", q.dtype), _stream(stream),
    )
    _check("la_decode_step", code)
    return out


def decode_tokens(q, k, v, slope, state, out=None, stream=None):
    """K tokens per (b, h) on a carried state in one call.  q, k, v:
    [B,H,K,d]; state: [B,H,d,d] fp32 updated in place.  Equals K decode_step
    calls."""
    B, H, K, d = q.shape
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    code = lib().la_decode_tokens(
        dt, B, H, K, d, _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
        _dev(slope, "slope", torch.float32), _dev(state, "state", torch.float32),
        _dev(out, "out", q.dtype), _stream(stream),
    )
    _check("la_decode_tokens", code)
    return out


def prefill_bwd(q, k, v, dout, slope, chunk=64, dq=None, dk=None, dv=None,
                workspace=None, stream=None, reuse_forward_workspace=False):
    """Gradients (dq, dk, dv) of sum(o * dout) for o = prefill(q, k, v, slope).

    With reuse_forward_workspace, workspace must be the one the forward
    prefill call (same k, v, slope, chunk, no state_in) used, unmodified since:
    the dq pass then takes the forward's segment start states from it
    (la_prefill_bwd_reuse)."""
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    nbytes = workspace_bytes(1, dt, B, H, N, d, chunk)
    if reuse_forward_workspace and nbytes > 0 and workspace is None:
        raise ValueError("reuse_forward_workspace needs the forward's workspace")
    ws, wsb = _workspace(nbytes, q.device, workspace)
    fn = "la_prefill_bwd_reuse" if reuse_forward_workspace else "la_prefill_bwd"
    code = getattr(lib(), fn)(
        dt, B, H, N, d, chunk,
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(dout, "dout", q.dtype),
        _dev(slope, "slope", torch.float32), None,
        _dev(dq, "dq", q.dtype), _dev(dk, "dk", q.dtype), _dev(dv, "dv", q.dtype),
        None if ws is None else ws.data_ptr(), wsb, _stream(stream),
    )
    _check(fn, code)
    return dq, dk, dv


def _cu_array(cu_seqlens):
    """cu_seqlens (a list, numpy array or CPU tensor of nseq + 1 ints) as a
    host int32 ctypes array, the form the library reads."""
    if isinstance(cu_seqlens, torch.Tensor):
        if cu_seqlens.is_cuda:
            raise TypeError("cu_seqlens must be host data (list, numpy array or CPU tensor)")
        cu_seqlens = cu_seqlens.tolist()
    vals = [int(x) for x in cu_seqlens]
    return len(vals) - 1, (ctypes.c_int * len(vals))(*vals)


def workspace_bytes_varlen(op: int, dtype: int, H: int, d: int, C: int, cu_seqlens) -> int:
    nseq, cu = _cu_array(cu_seqlens)
    n = lib().la_workspace_bytes_varlen(op, dtype, H, d, C, nseq, cu)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("arguments rejected by la_workspace_bytes_varlen")
    return n


def prefill_varlen(q, k, v, slope, cu_seqlens, chunk=64, state_in=None, out=None,
                   state_out=None, return_state=True, workspace=None, stream=None):
    """Packed batch: q, k, v [H,T,d]; sequence s is tokens
    cu_seqlens[s] .. cu_seqlens[s+1]-1 (host ints).  Returns (o, state_out)
    with state_out [nseq,H,d,d] fp32 (None when return_state is False and no
    state_out tensor is given)."""
    H, T, d = q.shape
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("%s must match q in shape and dtype" % name)
    nseq, cu = _cu_array(cu_seqlens)
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((nseq, H, d, d), dtype=torch.float32, device=q.device)
    nbytes = workspace_bytes_varlen(0, dt, H, d, chunk, cu_seqlens)
    ws, wsb = _workspace(nbytes, q.device, workspace)
    code = lib().la_prefill_varlen(
        dt, H, d, chunk, nseq, cu,
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(slope, "slope", torch.float32),
        None if state_in is None else _dev(state_in, "state_in", torch.float32),
        _dev(out, "out", q.dtype),
        None if state_out is None else _dev(state_out, "state_out", torch.float32),
        None if ws is None else ws.data_ptr(), wsb, _stream(stream),
    )
    _check("la_prefill_varlen", code)
    return out, state_out


def prefill_bwd_varlen(q, k, v, dout, slope, cu_seqlens, chunk=64, dq=None, dk=None, dv=None,
                       workspace=None, stream=None, reuse_forward_workspace=False):
    """Gradients (dq, dk, dv) [H,T,d] of sum(o * dout) for o = prefill_varlen(...)
    with zero initial states.  reuse_forward_workspace as for prefill_bwd
    (la_prefill_bwd_varlen_reuse)."""
    H, T, d = q.shape
    dt = _dtype_code(q)
    nseq, cu = _cu_array(cu_seqlens)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    nbytes = workspace_bytes_varlen(1, dt, H, d, chunk, cu_seqlens)
    if reuse_forward_workspace and nbytes > 0 and workspace is None:
        raise ValueError("reuse_forward_workspace needs the forward's workspace")
    ws, wsb = _workspace(nbytes, q.device, workspace)
    fn = "la_prefill_bwd_varlen_reuse" if reuse_forward_workspace else "la_prefill_bwd_varlen"
    code = getattr(lib(), fn)(
        dt, H, d, chunk, nseq, cu,
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(dout, "dout", q.dtype),
        _dev(slope, "slope", torch.float32),
        _dev(dq, "dq", q.dtype), _dev(dk, "dk", q.dtype), _dev(dv, "dv", q.dtype),
        None if ws is None else ws.data_ptr(), wsb, _stream(stream),
    )
    _check(fn, code)
    return dq, dk, dv


def abi_version() -> int:
    return lib().la_abi_version()
