"""Parity at the full workload sizes, in the launch configuration bench.py times.

Heads (and decode rows) are independent, so the fp64 oracle checks whole
heads exactly: every head of the 8K and 128K prefills, sampled heads or rows
of the other workloads.
"""
import numpy as np
import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import assert_close, device, to_host

pytestmark = pytest.mark.gpu


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def test_prefill_8k_full(oracle_mod):
    c = la_inputs.CONFIGS["prefill_8k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    q, k, v = la_inputs.qkv(c["seed"], B, H, N, d, dtype="bf16")
    s = la_inputs.slopes(H)
    dev = device()
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
    o, S = la.prefill(tq, tk, tv, torch.from_numpy(s).to(dev), chunk=C)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.fwd(q, k, v, s)
    assert_close(_host(o), ro, "bf16", "o")
    assert_close(_host(S), rS, "bf16", "S", stored_bf16=False)


def test_prefill_128k_every_head(oracle_mod):
    c = la_inputs.CONFIGS["prefill_128k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = device()
    tq, tk, tv = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    s = la_inputs.slopes(H)
    o, S = la.prefill(tq, tk, tv, torch.from_numpy(s).to(dev), chunk=C)
    torch.cuda.synchronize()
    # all 32 heads, eight at a time (host memory), each against its own bar
    for h0 in range(0, H, 8):
        heads = list(range(h0, min(H, h0 + 8)))
        q, k, v = (_host(t[:, heads]) for t in (tq, tk, tv))
        ro, rS = oracle_mod.fwd(q, k, v, s[heads])
        go, gS = _host(o[:, heads]), _host(S[:, heads])
        for i, h in enumerate(heads):
            assert_close(go[:, i], ro[:, i], "bf16", "o head %d" % h)
            assert_close(gS[:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
        del q, k, v, ro, rS, go, gS


def test_decode_b64_1000_steps(oracle_mod):
    """1000 consecutive decode steps on the B=64, H=32 state: every output of
    every step and the final state of every row, against the oracle's
    recurrent forward over the 1000 tokens (decode steps are that recurrence)."""
    c = la_inputs.CONFIGS["decode_b64"]
    B, H, d, steps = c["B"], c["H"], c["d"], c["steps"]
    dev = device()
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(c["seed"], B, H, d)
    tS = torch.from_numpy(S0).to(dev)
    ts = torch.from_numpy(s).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(c["seed"])
    qs, ks, vs = ((torch.randn((steps, B, H, d), generator=g, device=dev) / d**0.5).to(torch.bfloat16)
                  for _ in range(3))
    outs = torch.empty((steps, B, H, d), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        la.decode_step(qs[t], ks[t], vs[t], ts, tS, out=outs[t])
    torch.cuda.synchronize()
    # [steps][B][H][d] -> [B][H][steps][d]: each (b, h) row is a 1000-token sequence
    q, k, v = (_host(t.permute(1, 2, 0, 3).contiguous()) for t in (qs, ks, vs))
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    go = _host(outs.permute(1, 2, 0, 3).contiguous())
    gS = _host(tS)
    for h in range(H):
        assert_close(go[:, h], ro[:, h], "bf16", "o head %d" % h)
        assert_close(gS[:, h], rS[:, h], "bf16", "state head %d" % h, stored_bf16=False)


def test_train_32k_every_row(oracle_mod):
    """The training workload as the benchmark runs it (forward, then the
    backward on the forward's workspace), every (b, h) row against the oracle."""
    c = la_inputs.CONFIGS["train_32k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = device()
    tq, tk, tv = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    tg = la_inputs.upstream_grad_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    s = la_inputs.slopes(H)
    ts = torch.from_numpy(s).to(dev)
    ws = torch.empty(max(la.workspace_bytes(1, la.LA_BF16, B, H, N, d, C), 16),
                     dtype=torch.uint8, device=dev)
    o, _ = la.prefill(tq, tk, tv, ts, chunk=C, return_state=False, workspace=ws)
    dq, dk, dv = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C, workspace=ws,
                                reuse_forward_workspace=True)
    torch.cuda.synchronize()
    for b in range(B):
        q, k, v, g = (_host(t[b:b + 1]) for t in (tq, tk, tv, tg))
        ro, _ = oracle_mod.fwd(q, k, v, s)
        rq, rk, rv = oracle_mod.bwd(q, k, v, g, s)
        go, gq, gk, gv = (_host(t[b:b + 1]) for t in (o, dq, dk, dv))
        for h in range(H):
            what = "(b=%d,h=%d)" % (b, h)
            assert_close(go[:, h], ro[:, h], "bf16", "o " + what)
            assert_close(gq[:, h], rq[:, h], "bf16", "dq " + what)
            assert_close(gk[:, h], rk[:, h], "bf16", "dk " + what)
            assert_close(gv[:, h], rv[:, h], "bf16", "dv " + what)


def test_varlen_128k_every_head(oracle_mod):
    """The benchmark's packed batch (64 ragged sequences, 131072 tokens,
    H=32, d=128, C=128): the forward with per-sequence initial states, then
    the backward (zero initial states), every head against the oracle."""
    c = la_inputs.CONFIGS["varlen_128k"]
    H, d, C, nseq, T, seed = c["H"], c["d"], c["C"], c["nseq"], c["T"], c["seed"]
    dev = device()
    cu = la_inputs.packed_cu_seqlens(seed, nseq, T)
    tq, tk, tv = (x[0] for x in la_inputs.qkv_device(seed, 1, H, T, d, dev, torch.bfloat16))
    tg = la_inputs.upstream_grad_device(seed, 1, H, T, d, dev, torch.bfloat16)[0]
    s = la_inputs.slopes(H)
    ts = torch.from_numpy(s).to(dev)
    S0 = la_inputs.decode_state(seed, nseq, H, d)
    o, S = la.prefill_varlen(tq, tk, tv, ts, cu, chunk=C, state_in=torch.from_numpy(S0).to(dev))
    dq, dk, dv = la.prefill_bwd_varlen(tq, tk, tv, tg, ts, cu, chunk=C)
    torch.cuda.synchronize()
    for h0 in range(0, H, 8):
        heads = list(range(h0, min(H, h0 + 8)))
        q, k, v, g = (_host(t[heads]) for t in (tq, tk, tv, tg))
        ro, rS = oracle_mod.fwd_varlen(q, k, v, s[heads], cu, S0[:, heads])
        rq, rk, rv = oracle_mod.bwd_varlen(q, k, v, g, s[heads], cu)
        go, gS = _host(o[heads]), _host(S[:, heads])
        gq, gk, gv = (_host(t[heads]) for t in (dq, dk, dv))
        for i, h in enumerate(heads):
            assert_close(go[i], ro[i], "bf16", "o head %d" % h)
            assert_close(gS[:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
            assert_close(gq[i], rq[i], "bf16", "dq head %d" % h)
            assert_close(gk[i], rk[i], "bf16", "dk head %d" % h)
            assert_close(gv[i], rv[i], "bf16", "dv head %d" % h)


def test_prefill_gated_128k_every_head(oracle_mod):
    """The 128K prefill with the fused output epilogue, as the benchmark runs it."""
    c = la_inputs.CONFIGS["prefill_128k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = device()
    tq, tk, tv = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    tg = la_inputs.gate_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    w = la_inputs.norm_weight(c["seed"], H, d)
    s = la_inputs.slopes(H)
    y, S = la.prefill_gated(tq, tk, tv, torch.from_numpy(s).to(dev), tg,
                            torch.from_numpy(w).to(dev), eps=1e-6, chunk=C)
    torch.cuda.synchronize()
    for h0 in range(0, H, 8):
        heads = list(range(h0, min(H, h0 + 8)))
        q, k, v, g = (_host(t[:, heads]) for t in (tq, tk, tv, tg))
        ry, rS = oracle_mod.fwd_gated(q, k, v, s[heads], g, w[heads], 1e-6)
        gy, gS = _host(y[:, heads]), _host(S[:, heads])
        for i, h in enumerate(heads):
            assert_close(gy[:, i], ry[:, i], "bf16", "y head %d" % h)
            assert_close(gS[:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
