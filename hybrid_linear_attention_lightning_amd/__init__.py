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
    "la_prefill_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
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
    "la_probe_stream_rmw": (_I, [_P, _Z, ctypes.c_float, _I, _I, _P]),
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


def _dtype_code(t) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor, got %s" % type(t).__name__)
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError("expected bfloat16 or float32 tensors, got %s" % t.dtype)


def _ptrs(device, *specs):
    """Device addresses of the tensors in `specs`, each (tensor or None, name,
    shape, dtype), after checking all of them: a torch tensor of exactly that
    shape and dtype, contiguous, then (in a second round, so that a wrongly
    sized tensor reports its shape wherever it stands) on the GPU `device`.
    None stays None.  Every tensor is checked before any launch: the library
    takes plain pointers and sizes and cannot see a tensor that is too small."""
    for t, name, shape, dtype in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
        if t.shape != shape:
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
        if t.dtype is not dtype:
            raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    index = device.index
    out = []
    for t, name, _, _ in specs:
        if t is None:
            out.append(None)
            continue
        if not t.is_cuda:
            raise TypeError("%s must be a GPU tensor" % name)
        if t.get_device() != index:
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
        out.append(t.data_ptr())
    return out


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_bytes(op: int, dtype: int, B: int, H: int, N: int, d: int, C: int) -> int:
    n = lib().la_workspace_bytes(op, dtype, B, H, N, d, C)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("arguments rejected by la_workspace_bytes")
    return n


def _workspace(nbytes: int, device, ws, required=False):
    """(pointer, size) of the workspace: the caller's tensor, checked, or a
    fresh one when the caller passes none (unless `required`: the call reads
    states an earlier call left there).  A caller's workspace that is too
    small is an error, never replaced behind the caller's back."""
    if nbytes == 0:
        return None, 0
    if ws is None:
        if required:
            raise ValueError("this call needs the workspace of the earlier call whose "
                             "segment start states it reads")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous torch tensor")
    size = ws.numel() * ws.element_size()
    if size < nbytes:
        raise ValueError("workspace holds %d bytes, %d needed" % (size, nbytes))
    if not ws.is_cuda or ws.device != device:
        raise ValueError("workspace must be a GPU tensor on %s" % device)
    return ws.data_ptr(), size


def _same(ref, others):
    """k, v (and the like) must match q in shape and dtype."""
    for name, t in others:
        if not isinstance(t, torch.Tensor) or t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("%s must match q in shape and dtype" % name)


def _shape(t, name, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    return tuple(t.shape)


def prefill(q, k, v, slope, chunk=64, state_in=None, out=None, state_out=None,
            return_state=True, workspace=None, stream=None):
    """Chunked forward.  q, k, v: [B,H,N,d] bf16 or fp32; slope: [H] fp32.

    Returns (o, state_out) where state_out is [B,H,d,d] fp32 (None when
    return_state is False and no state_out tensor is given)."""
    B, H, N, d = _shape(q, "q", 4)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v)))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    sd = (B, H, d, d)
    args = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
                 (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
                 (state_in, "state_in", sd, torch.float32), (out, "out", q.shape, q.dtype),
                 (state_out, "state_out", sd, torch.float32))
    ws, wsb = _workspace(workspace_bytes(0, dt, B, H, N, d, chunk), dev, workspace)
    code = lib().la_prefill(dt, B, H, N, d, chunk, *args, ws, wsb, _stream(stream))
    _check("la_prefill", code)
    return out, state_out


def prefill_noalloc(q, k, v, slope, chunk=64, state_in=None, out=None, state_out=None,
                    return_state=True, stream=None):
    """`prefill` without a workspace (la_prefill_noalloc): the library's static
    per-GPU scratch buffer holds the segment states, so the call allocates no
    device memory when `out` (and `state_out`, or return_state=False) are
    given.  Calls that overlap on one GPU race."""
    B, H, N, d = _shape(q, "q", 4)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v)))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    sd = (B, H, d, d)
    args = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
                 (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
                 (state_in, "state_in", sd, torch.float32), (out, "out", q.shape, q.dtype),
                 (state_out, "state_out", sd, torch.float32))
    code = lib().la_prefill_noalloc(dt, B, H, N, d, chunk, *args, _stream(stream))
    _check("la_prefill_noalloc", code)
    return out, state_out


def prefill_gated(q, k, v, slope, gate, norm_weight, eps=1e-6, chunk=64, state_in=None,
                  out=None, state_out=None, return_state=True, workspace=None, stream=None):
    """prefill with the fused output epilogue: y = RMSNorm_head(o) * norm_weight[h]
    * sigmoid(gate), gate like q, norm_weight [H, d] fp32.  Returns (y, state_out)."""
    B, H, N, d = _shape(q, "q", 4)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v), ("gate", gate)))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    sd = (B, H, d, d)
    p = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
              (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
              (state_in, "state_in", sd, torch.float32), (gate, "gate", q.shape, q.dtype),
              (norm_weight, "norm_weight", (H, d), torch.float32), (out, "out", q.shape, q.dtype),
              (state_out, "state_out", sd, torch.float32))
    args = p[:7] + [float(eps)] + p[7:]
    ws, wsb = _workspace(workspace_bytes(0, dt, B, H, N, d, chunk), dev, workspace)
    code = lib().la_prefill_gated(dt, B, H, N, d, chunk, *args, ws, wsb, _stream(stream))
    _check("la_prefill_gated", code)
    return out, state_out


def prefill_prepass(k, v, slope, chunk, workspace, state_in=None, stream=None):
    """First half of `prefill`: segment start states into `workspace`
    (a uint8 cuda tensor of at least workspace_bytes(0, ...) bytes)."""
    B, H, N, d = _shape(k, "k", 4)
    dt = _dtype_code(k)
    dev = k.device
    args = _ptrs(dev, (k, "k", k.shape, k.dtype), (v, "v", k.shape, k.dtype),
                 (slope, "slope", (H,), torch.float32),
                 (state_in, "state_in", (B, H, d, d), torch.float32))
    nbytes = workspace_bytes(0, dt, B, H, N, d, chunk)
    ws, wsb = _workspace(nbytes, dev, workspace, required=True)
    code = lib().la_prefill_prepass(dt, B, H, N, d, chunk, *args, ws, wsb, _stream(stream))
    _check("la_prefill_prepass", code)


def prefill_main(q, k, v, slope, chunk, workspace, out, state_out=None, state_in=None,
                 stream=None):
    """Second half of `prefill`: all segments from the states prefill_prepass
    left in `workspace` (all-NaN outputs if the workspace does not hold the
    states of a prepass with the same arguments)."""
    B, H, N, d = _shape(q, "q", 4)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v)))
    dev = q.device
    sd = (B, H, d, d)
    if out is None:
        raise ValueError("prefill_main needs the output tensor")
    args = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
                 (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
                 (state_in, "state_in", sd, torch.float32), (out, "out", q.shape, q.dtype),
                 (state_out, "state_out", sd, torch.float32))
    nbytes = workspace_bytes(0, dt, B, H, N, d, chunk)
    ws, wsb = _workspace(nbytes, dev, workspace, required=True)
    code = lib().la_prefill_main(dt, B, H, N, d, chunk, *args, ws, wsb, _stream(stream))
    _check("la_prefill_main", code)
    return out


def decode_step(q, k, v, slope, state, out=None, stream=None):
    """One decode step.  q, k, v: [B,H,d]; state: [B,H,d,d] fp32 updated in place."""
    B, H, d = _shape(q, "q", 3)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v)))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    args = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
                 (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
                 (state, "state", (B, H, d, d), torch.float32), (out, "out", q.shape, q.dtype))
    code = lib().la_decode_step(dt, B, H, d, *args, _stream(stream))
    _check("la_decode_step", code)
    return out


def decode_tokens(q, k, v, slope, state, out=None, stream=None):
    """K tokens per (b, h) on a carried state in one call.  q, k, v:
    [B,H,K,d]; state: [B,H,d,d] fp32 updated in place.  Equals K decode_step
    calls."""
    B, H, K, d = _shape(q, "q", 4)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v)))
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    args = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
                 (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
                 (state, "state", (B, H, d, d), torch.float32), (out, "out", q.shape, q.dtype))
    code = lib().la_decode_tokens(dt, B, H, K, d, *args, _stream(stream))
    _check("la_decode_tokens", code)
    return out


def prefill_bwd(q, k, v, dout, slope, chunk=64, dq=None, dk=None, dv=None,
                workspace=None, stream=None, reuse_forward_workspace=False):
    """Gradients (dq, dk, dv) of sum(o * dout) for o = prefill(q, k, v, slope).

    With reuse_forward_workspace, workspace must be the one the forward
    prefill call (same k, v, slope, chunk, no state_in) used, unmodified since:
    the dq pass then takes the forward's segment start states from it
    (la_prefill_bwd_reuse; dq is all NaN if the workspace holds other
    states)."""
    B, H, N, d = _shape(q, "q", 4)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v), ("dout", dout)))
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    p = _ptrs(dev, *((t, n, q.shape, q.dtype) for n, t in (("q", q), ("k", k), ("v", v),
                                                           ("dout", dout))),
              (slope, "slope", (H,), torch.float32),
              *((t, n, q.shape, q.dtype) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))))
    args = p[:5] + [None] + p[5:]
    nbytes = workspace_bytes(1, dt, B, H, N, d, chunk)
    ws, wsb = _workspace(nbytes, dev, workspace, required=reuse_forward_workspace)
    fn = "la_prefill_bwd_reuse" if reuse_forward_workspace else "la_prefill_bwd"
    code = getattr(lib(), fn)(dt, B, H, N, d, chunk, *args, ws, wsb, _stream(stream))
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
    if len(vals) < 2:
        raise ValueError("cu_seqlens needs at least two entries (one sequence)")
    return len(vals) - 1, (ctypes.c_int * len(vals))(*vals)


def _packed_T(cu, T, name="q"):
    """The packed tensors must hold exactly cu_seqlens[-1] tokens: the library
    takes T = cu_seqlens[nseq] and would address past a shorter tensor."""
    if cu[len(cu) - 1] != T:
        raise ValueError("cu_seqlens[-1] = %d but %s holds %d tokens" % (cu[len(cu) - 1], name, T))


def workspace_bytes_varlen(op: int, dtype: int, H: int, d: int, C: int, cu_seqlens) -> int:
    nseq, cu = _cu_array(cu_seqlens)
    n = lib().la_workspace_bytes_varlen(op, dtype, H, d, C, nseq, cu)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("arguments rejected by la_workspace_bytes_varlen")
    return n


def prefill_varlen(q, k, v, slope, cu_seqlens, chunk=64, state_in=None, out=None,
                   state_out=None, return_state=True, workspace=None, stream=None):
    """Packed batch: q, k, v [H,T,d]; sequence s is tokens
    cu_seqlens[s] .. cu_seqlens[s+1]-1 (host ints, cu_seqlens[-1] == T).
    Returns (o, state_out) with state_out [nseq,H,d,d] fp32 (None when
    return_state is False and no state_out tensor is given)."""
    H, T, d = _shape(q, "q", 3)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v)))
    nseq, cu = _cu_array(cu_seqlens)
    _packed_T(cu, T)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    if state_out is None and return_state:
        state_out = torch.empty((nseq, H, d, d), dtype=torch.float32, device=dev)
    sd = (nseq, H, d, d)
    args = _ptrs(dev, (q, "q", q.shape, q.dtype), (k, "k", q.shape, q.dtype),
                 (v, "v", q.shape, q.dtype), (slope, "slope", (H,), torch.float32),
                 (state_in, "state_in", sd, torch.float32), (out, "out", q.shape, q.dtype),
                 (state_out, "state_out", sd, torch.float32))
    ws, wsb = _workspace(workspace_bytes_varlen(0, dt, H, d, chunk, cu_seqlens), dev, workspace)
    code = lib().la_prefill_varlen(dt, H, d, chunk, nseq, cu, *args, ws, wsb, _stream(stream))
    _check("la_prefill_varlen", code)
    return out, state_out


def prefill_bwd_varlen(q, k, v, dout, slope, cu_seqlens, chunk=64, dq=None, dk=None, dv=None,
                       workspace=None, stream=None, reuse_forward_workspace=False):
    """Gradients (dq, dk, dv) [H,T,d] of sum(o * dout) for o = prefill_varlen(...)
    with zero initial states.  reuse_forward_workspace as for prefill_bwd
    (la_prefill_bwd_varlen_reuse)."""
    H, T, d = _shape(q, "q", 3)
    dt = _dtype_code(q)
    _same(q, (("k", k), ("v", v), ("dout", dout)))
    nseq, cu = _cu_array(cu_seqlens)
    _packed_T(cu, T)
    dev = q.device
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    args = _ptrs(dev, *((t, n, q.shape, q.dtype) for n, t in (("q", q), ("k", k), ("v", v),
                                                              ("dout", dout))),
                 (slope, "slope", (H,), torch.float32),
                 *((t, n, q.shape, q.dtype) for n, t in (("dq", dq), ("dk", dk), ("dv", dv))))
    nbytes = workspace_bytes_varlen(1, dt, H, d, chunk, cu_seqlens)
    ws, wsb = _workspace(nbytes, dev, workspace, required=reuse_forward_workspace)
    fn = "la_prefill_bwd_varlen_reuse" if reuse_forward_workspace else "la_prefill_bwd_varlen"
    code = getattr(lib(), fn)(dt, H, d, chunk, nseq, cu, *args, ws, wsb, _stream(stream))
    _check(fn, code)
    return dq, dk, dv


CPOL_NT, CPOL_SC1 = 2, 16  # cache-policy bits accepted by probe_stream_rmw


def probe_stream_rmw(x, a=1.0, load_policy=CPOL_NT, store_policy=CPOL_SC1, stream=None):
    """Measurement helper: x <- a x in place over a contiguous fp32 GPU
    tensor (the decode step's state traffic without its arithmetic), with
    the given cache-policy bits on the loads and on the stores."""
    (ptr,) = _ptrs(x.device, (x, "x", x.shape, torch.float32))
    code = lib().la_probe_stream_rmw(ptr, x.numel(), float(a), int(load_policy),
                                     int(store_policy), _stream(stream))
    _check("la_probe_stream_rmw", code)
    return x


def abi_version() -> int:
    return lib().la_abi_version()
