"""The C-ABI library: it loads, exports every declared symbol, and rejects bad
arguments before any HIP call (so these run without a GPU).

Every call below is built to fail validation; none reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

import hybrid_linear_attention_lightning_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_la.h")

F32, BF16 = la.LA_F32, la.LA_BF16
OK, NULLP, SHAPE, DTYPE, UNSUP, WS, HIP, ALIGN, ALIAS = range(9)

# fake, aligned, non-overlapping device addresses (never dereferenced: every
# call here fails validation first)
Q, K, V, O, S_IN, S_OUT, SLOPE, WSP, DO, DQ, DK, DV = (0x10_0000_0000 * (i + 1) for i in range(12))


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(la_[a-z_]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = la.lib()
    syms = declared_symbols()
    assert set(syms) == set(la.SIGNATURES), syms
    for s in syms:
        assert hasattr(lib, s), s


def test_abi_version_and_status_strings():
    lib = la.lib()
    assert lib.la_abi_version() == 4
    for code in range(9):
        assert lib.la_status_string(code)
    assert lib.la_status_string(123) == b"unknown status"


def prefill(dt=BF16, B=1, H=2, N=256, d=128, C=64, q=Q, k=K, v=V, slope=SLOPE, s_in=None,
            o=O, s_out=None, ws=None, wsb=0):
    return la.lib().la_prefill(dt, B, H, N, d, C, q, k, v, slope, s_in, o, s_out, ws, wsb, None)


def test_prefill_validation():
    nws = la.workspace_bytes(0, BF16, 1, 2, 256, 128, 64)
    assert nws > 0  # few heads: the sequence is split into segments
    assert prefill(dt=7) == DTYPE
    assert prefill(B=0) == SHAPE and prefill(H=0) == SHAPE and prefill(N=0) == SHAPE
    assert prefill(d=96) == SHAPE and prefill(dt=BF16, d=32) == SHAPE
    assert prefill(C=48) == SHAPE and prefill(C=256) == SHAPE
    # size limits: B*H*N above 2^30, or B*H above 2^19 (32-bit work-item counts)
    assert prefill(B=1 << 12, H=1 << 10, N=1 << 9) == UNSUP
    assert prefill(dt=F32, B=1 << 10, H=(1 << 9) + 1, N=1, d=64) == UNSUP
    # bf16 C = 16 is accepted and runs 32-token chunks: same plan, same workspace
    assert prefill(dt=BF16, C=16) == WS
    assert la.workspace_bytes(0, BF16, 1, 2, 256, 128, 16) == la.workspace_bytes(0, BF16, 1, 2, 256, 128, 32)
    assert prefill(q=None) == NULLP and prefill(slope=None) == NULLP and prefill(o=None) == NULLP
    assert prefill(q=Q + 8) == ALIGN and prefill(o=O + 2) == ALIGN and prefill(slope=SLOPE + 1) == ALIGN
    assert prefill(s_in=S_IN + 4) == ALIGN
    assert prefill(o=Q) == ALIAS and prefill(o=V + 64) == ALIAS
    assert prefill(s_in=S_IN, s_out=S_IN + 16) == ALIAS
    assert prefill(s_out=O) == ALIAS
    assert prefill() == WS  # needs a workspace
    assert prefill(ws=WSP, wsb=nws - 1) == WS
    assert prefill(ws=WSP + 8, wsb=nws) == ALIGN


def test_piece_launch_limit():
    # B*H*N within 2^30, but 131071 (a prime) chunks of 32 tokens per segment
    # leave one-chunk pieces: 255 * 131071 piece workgroups of 256 threads
    # exceed the dispatch's 32-bit count of work-items
    N = 256 * 32 * 131071
    assert N <= 2**30
    far = [0x1000_0000_0000 * (i + 1) for i in range(5)]  # 16 TiB apart: no overlap
    big = dict(B=1, H=1, N=N, d=128, C=32, q=far[0], k=far[1], v=far[2], o=far[3])
    assert prefill(ws=far[4], wsb=2**62, **big) == UNSUP
    bwd = la.lib().la_prefill_bwd(BF16, 1, 1, N, 128, 32, far[0], far[1], far[2], far[3], SLOPE,
                                  None, far[4] + far[0], far[4] + far[1], far[4] + far[2],
                                  far[4] + far[3], 2**62, None)
    assert bwd == UNSUP
    # with a segment of 2^17 chunks the pieces are 1024 tokens long: accepted
    # (and then it needs a workspace)
    assert prefill(**dict(big, N=2**30)) == WS


def test_decode_validation():
    f = la.lib().la_decode_step

    def call(dt=BF16, B=2, H=2, d=128, q=Q, k=K, v=V, slope=SLOPE, st=S_IN, o=O):
        return f(dt, B, H, d, q, k, v, slope, st, o, None)

    assert call(dt=3) == DTYPE
    assert call(B=0) == SHAPE and call(d=100) == SHAPE
    assert call(st=None) == NULLP and call(k=None) == NULLP
    assert call(st=S_IN + 4) == ALIGN
    assert call(o=S_IN + 64) == ALIAS and call(st=Q) == ALIAS
    assert call(B=1 << 11, H=(1 << 10) + 1) == UNSUP  # B*H above 2^21


@pytest.mark.parametrize("entry", ["la_prefill_bwd", "la_prefill_bwd_reuse"])
def test_backward_validation(entry):
    f = getattr(la.lib(), entry)

    def call(dt=BF16, N=256, C=64, s_in=None, dq=DQ, dk=DK, dv=DV, ws=None, wsb=0):
        return f(dt, 1, 2, N, 128, C, Q, K, V, DO, SLOPE, s_in, dq, dk, dv, ws, wsb, None)

    assert call(C=16) == WS
    assert call(dq=None) == NULLP
    assert call(s_in=S_IN) == UNSUP
    assert call(dk=DQ) == ALIAS and call(dv=DO) == ALIAS
    assert call() == WS


def test_workspace_plan():
    # fp32 path and many heads: single segment, no workspace
    assert la.workspace_bytes(0, F32, 1, 2, 256, 64, 64) == 0
    assert la.workspace_bytes(0, BF16, 16, 16, 4096, 128, 64) == 0
    # 128K-token prefill with 32 heads: segments and piece states
    n = la.workspace_bytes(0, BF16, 1, 32, 131072, 128, 128)
    assert 0 < n < 2**30
    assert la.workspace_bytes(1, BF16, 1, 32, 131072, 128, 128) == n
    with pytest.raises(ValueError):
        la.workspace_bytes(0, BF16, 1, 32, 131072, 100, 128)
    assert la.lib().la_workspace_bytes(2, BF16, 1, 1, 1, 64, 64) == ctypes.c_size_t(-1).value


def test_varlen_validation():
    f = la.lib().la_prefill_varlen

    def call(dt=BF16, H=2, d=128, C=64, cu=(0, 100, 5000), q=Q, o=O, s_in=None, s_out=None,
             ws=None, wsb=0, nseq=None):
        n = (len(cu) - 1 if cu is not None else 1) if nseq is None else nseq
        arr = (ctypes.c_int * len(cu))(*cu) if cu is not None else None
        return f(dt, H, d, C, n, arr, q, K, V, SLOPE, s_in, o, s_out, ws, wsb, None)

    assert call(dt=5) == DTYPE
    assert call(H=0) == SHAPE and call(d=96) == SHAPE and call(C=48) == SHAPE
    assert call(nseq=0) == SHAPE
    assert call(dt=BF16, C=16) == WS
    assert call(cu=None) == NULLP
    assert call(cu=(1, 100)) == SHAPE  # must start at 0
    assert call(cu=(0, 100, 50)) == SHAPE  # must not decrease
    assert call(cu=tuple(range(258))) == UNSUP  # 257 sequences
    assert call(H=4097) == UNSUP
    assert call(q=None) == NULLP and call(o=None) == NULLP
    assert call(q=Q + 8) == ALIGN and call(s_out=S_OUT + 4) == ALIGN
    assert call(o=K) == ALIAS and call(s_in=S_IN, s_out=S_IN + 16) == ALIAS
    nws = la.workspace_bytes_varlen(0, BF16, 2, 128, 64, (0, 100, 5000))
    assert nws > 0  # the long sequence is cut into segments
    assert call() == WS and call(ws=WSP, wsb=nws - 1) == WS and call(ws=WSP + 8, wsb=nws) == ALIGN


@pytest.mark.parametrize("entry", ["la_prefill_bwd_varlen", "la_prefill_bwd_varlen_reuse"])
def test_varlen_backward_validation(entry):
    f = getattr(la.lib(), entry)
    cu = (ctypes.c_int * 3)(0, 100, 5000)

    def call(dq=DQ, dk=DK, dv=DV, C=64):
        return f(BF16, 2, 128, C, 2, cu, Q, K, V, DO, SLOPE, dq, dk, dv, None, 0, None)

    assert call(C=16) == WS and call(dq=None) == NULLP
    assert call(dk=DQ) == ALIAS and call(dv=DO) == ALIAS
    assert call() == WS


def test_varlen_workspace_plan():
    # enough (sequence, head) rows to fill the GPU: one segment each, no
    # workspace; the fp32 path never segments
    assert la.workspace_bytes_varlen(0, BF16, 32, 128, 128, list(range(0, 8001, 1000))) == 0
    # few rows: sequences are cut into segments
    assert la.workspace_bytes_varlen(0, BF16, 32, 128, 128, [0, 1000, 2000, 2048]) > 0
    assert la.workspace_bytes_varlen(0, F32, 2, 64, 64, [0, 100000]) == 0
    # one 128K-token sequence of 32 heads: the same cut as the uniform plan
    assert (la.workspace_bytes_varlen(0, BF16, 32, 128, 128, [0, 131072])
            == la.workspace_bytes(0, BF16, 1, 32, 131072, 128, 128) + 32 * 16 * 64 * 1024)
    assert la.workspace_bytes_varlen(1, BF16, 2, 64, 64, [0, 0, 0]) == 0
    cu = (ctypes.c_int * 2)(0, 10)
    assert la.lib().la_workspace_bytes_varlen(2, BF16, 1, 64, 64, 1, cu) == ctypes.c_size_t(-1).value


def test_decode_tokens_validation():
    f = la.lib().la_decode_tokens

    def call(dt=BF16, B=2, H=2, nk=4, d=128, q=Q, st=S_IN, o=O):
        return f(dt, B, H, nk, d, q, K, V, SLOPE, st, o, None)

    assert call(dt=3) == DTYPE
    assert call(nk=0) == SHAPE and call(B=0) == SHAPE and call(d=100) == SHAPE
    assert call(nk=129) == UNSUP
    assert call(B=1 << 10, H=(1 << 9) + 1, nk=1) == UNSUP  # B*H above 2^19
    assert call(st=None) == NULLP and call(q=None) == NULLP
    assert call(st=S_IN + 4) == ALIGN
    assert call(o=S_IN + 64) == ALIAS and call(st=Q) == ALIAS
    assert call(B=1 << 11, H=(1 << 10) + 1) == UNSUP  # B*H above 2^21


def test_gated_prefill_validation():
    f = la.lib().la_prefill_gated
    G, W = 0x10_0000_0000 * 20, 0x10_0000_0000 * 21
    nws = la.workspace_bytes(0, BF16, 1, 2, 256, 128, 64)

    def call(gate=G, w=W, eps=1e-6, y=O, ws=WSP, wsb=nws):
        return f(BF16, 1, 2, 256, 128, 64, Q, K, V, SLOPE, None, gate, w, eps, y, None, ws, wsb,
                 None)

    assert call(gate=None) == NULLP and call(w=None) == NULLP
    assert call(gate=G + 8) == ALIGN and call(w=W + 2) == ALIGN
    assert call(eps=-1.0) == SHAPE and call(eps=float("nan")) == SHAPE
    assert call(eps=float("inf")) == SHAPE
    assert call(y=G) == ALIAS and call(y=W) == ALIAS
    assert call(ws=None, wsb=0) == WS


def test_noalloc_validation():
    f = la.lib().la_prefill_noalloc

    def call(dt=BF16, B=1, N=256, C=64, q=Q, o=O, s_in=None, s_out=None):
        return f(dt, B, 2, N, 128, C, q, K, V, SLOPE, s_in, o, s_out, None)

    assert call(dt=7) == DTYPE and call(B=0) == SHAPE and call(C=48) == SHAPE
    assert call(q=None) == NULLP and call(q=Q + 8) == ALIGN
    assert call(o=K) == ALIAS and call(s_in=S_IN, s_out=S_IN + 16) == ALIAS


def test_probe_validation():
    f = la.lib().la_probe_stream_rmw
    assert f(None, 16, 1.0, 2, 16, None) == NULLP
    assert f(Q, 0, 1.0, 2, 16, None) == SHAPE and f(Q, 6, 1.0, 2, 16, None) == SHAPE
    assert f(Q, 4 * 1024 * (1 << 24), 1.0, 2, 16, None) == UNSUP  # grid above 2^24 - 1
    assert f(Q + 8, 16, 1.0, 2, 16, None) == ALIGN
    assert f(Q, 16, 1.0, 1, 16, None) == UNSUP  # sc0 loads are not offered
    assert f(Q, 16, 1.0, 2, 18, None) == UNSUP  # nor nt|sc1 stores
