"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronizations in between,
reproduces the eager result bit for bit.

Covered: the bf16 prefill with its segment pre-pass (three kernels on a
caller's workspace), the allocation-free prefill (the entry point for callers
under graph capture), the decode step (state updated in place), a training
step (forward, then the backward reusing the forward's workspace), the gated
prefill followed by multi-token decode, and a packed batch's forward and
backward.  Outputs are
set to NaN before each replay, so a replay that skipped a kernel would show.
"""
import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _other_work(dev):
    """Eager work between replays: another prefill on other buffers."""
    q, k, v = la_inputs.qkv_device(77, 1, 4, 1024, 128, dev, torch.bfloat16)
    sl = torch.from_numpy(la_inputs.slopes(4)).to(dev)
    o, S = la.prefill(q, k, v, sl, chunk=64)
    torch.cuda.synchronize()
    return float(o.float().abs().sum()) + float(S.abs().sum())


def _replay_and_check(g, outs, refs, reset=None):
    dev = outs[0].device
    for _ in range(REPLAYS):
        _other_work(dev)
        for t in outs:
            t.fill_(float("nan"))
        if reset is not None:
            reset()  # in-place inputs (the decode state) back to their start
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r)


def _prefill_inputs(dev, seed=5, B=1, H=8, N=4096, d=128):
    q, k, v = la_inputs.qkv_device(seed, B, H, N, d, dev, torch.bfloat16)
    sl = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    return q, k, v, sl


def test_prefill_with_prepass_replays():
    dev = device()
    q, k, v, sl = _prefill_inputs(dev)
    B, H, N, d = q.shape
    C = 64
    nws = la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C)
    assert nws > 0  # 8 heads: segments, so the pre-pass runs
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)

    def fn():
        la.prefill(q, k, v, sl, chunk=C, out=o, state_out=S, workspace=ws)

    fn()
    torch.cuda.synchronize()
    refs = (o.clone(), S.clone())
    g = _capture(fn)
    _replay_and_check(g, (o, S), refs)


def test_noalloc_prefill_replays():
    dev = device()
    q, k, v, sl = _prefill_inputs(dev, seed=6, H=16, N=8192)
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)

    def fn():
        la.prefill_noalloc(q, k, v, sl, chunk=128, out=o, state_out=S)

    fn()  # the first call on the device also looks up the scratch buffer
    torch.cuda.synchronize()
    refs = (o.clone(), S.clone())
    g = _capture(fn)
    _replay_and_check(g, (o, S), refs)


def test_decode_step_replays():
    dev = device()
    B, H, d = 8, 16, 128
    S0 = torch.from_numpy(la_inputs.decode_state(14, B, H, d)).to(dev)
    sl = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    q, k, v = ((torch.randn((B, H, d), generator=gen, device=dev) / d ** 0.5).to(torch.bfloat16)
               for _ in range(3))
    state = S0.clone()
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)

    def fn():
        la.decode_step(q, k, v, sl, state, out=o)

    fn()
    torch.cuda.synchronize()
    refs = (o.clone(), state.clone())

    def reset():
        state.copy_(S0)

    reset()
    g = _capture(fn)  # the capture's warm-up steps advance the state: reset each replay
    _replay_and_check(g, (o, state), refs, reset=reset)


def test_training_step_replays():
    dev = device()
    q, k, v, sl = _prefill_inputs(dev, seed=7, B=2, H=4, N=2048)
    B, H, N, d = q.shape
    C = 64
    g_out = la_inputs.upstream_grad_device(7, B, H, N, d, dev, torch.bfloat16)
    nws = max(la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C),
              la.workspace_bytes(1, la.LA_BF16, B, H, N, d, C))
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def fn():
        la.prefill(q, k, v, sl, chunk=C, out=o, return_state=False, workspace=ws)
        la.prefill_bwd(q, k, v, g_out, sl, chunk=C, dq=dq, dk=dk, dv=dv, workspace=ws,
                       reuse_forward_workspace=True)

    fn()
    torch.cuda.synchronize()
    assert not torch.isnan(dq.float()).any()  # the reused states matched
    refs = (o.clone(), dq.clone(), dk.clone(), dv.clone())
    g = _capture(fn)
    _replay_and_check(g, (o, dq, dk, dv), refs)


def test_gated_prefill_and_decode_tokens_replay():
    dev = device()
    q, k, v, sl = _prefill_inputs(dev, seed=8, H=8, N=4096)
    B, H, N, d = q.shape
    C = 128
    gate = la_inputs.gate_device(8, B, H, N, d, dev, torch.bfloat16)
    w = torch.from_numpy(la_inputs.norm_weight(8, H, d)).to(dev)
    ws = torch.empty(la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    # four new tokens per row on the final state of the prefill
    K = 4
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    qt, kt, vt = ((torch.randn((B, H, K, d), generator=gen, device=dev) / d ** 0.5)
                  .to(torch.bfloat16) for _ in range(3))
    ot = torch.empty((B, H, K, d), dtype=torch.bfloat16, device=dev)

    def fn():
        la.prefill_gated(q, k, v, sl, gate, w, chunk=C, out=y, state_out=S, workspace=ws)
        la.decode_tokens(qt, kt, vt, sl, S, out=ot)

    fn()
    torch.cuda.synchronize()
    refs = (y.clone(), S.clone(), ot.clone())
    g = _capture(fn)
    _replay_and_check(g, (y, S, ot), refs)


def test_packed_batch_forward_and_backward_replay():
    dev = device()
    H, d, C, T, nseq = 8, 128, 64, 6000, 7
    cu = la_inputs.packed_cu_seqlens(9, nseq, T)
    q, k, v = (x[0] for x in la_inputs.qkv_device(9, 1, H, T, d, dev, torch.bfloat16))
    q, k, v = (x.contiguous() for x in (q, k, v))
    gout = la_inputs.upstream_grad_device(9, 1, H, T, d, dev, torch.bfloat16)[0].contiguous()
    sl = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    nws = max(la.workspace_bytes_varlen(0, la.LA_BF16, H, d, C, cu),
              la.workspace_bytes_varlen(1, la.LA_BF16, H, d, C, cu))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    S = torch.empty((nseq, H, d, d), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def fn():
        la.prefill_varlen(q, k, v, sl, cu, chunk=C, out=o, state_out=S, workspace=ws)
        la.prefill_bwd_varlen(q, k, v, gout, sl, cu, chunk=C, dq=dq, dk=dk, dv=dv, workspace=ws,
                              reuse_forward_workspace=True)

    fn()
    torch.cuda.synchronize()
    assert not torch.isnan(dq.float()).any()
    refs = (o.clone(), S.clone(), dq.clone(), dk.clone(), dv.clone())
    g = _capture(fn)
    _replay_and_check(g, (o, S, dq, dk, dv), refs)
