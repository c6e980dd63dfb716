"""Parity at the full workload sizes, in the launch configuration bench.py times.

Heads (and decode rows) are independent, so the fp64 oracle checks whole
sampled heads exactly; the 8K prefill is checked in full.
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


def test_prefill_128k_sampled_heads(oracle_mod):
    c = la_inputs.CONFIGS["prefill_128k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = device()
    tq, tk, tv = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    s = la_inputs.slopes(H)
    o, S = la.prefill(tq, tk, tv, torch.from_numpy(s).to(dev), chunk=C)
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    q, k, v = (_host(t[:, heads]) for t in (tq, tk, tv))
    ro, rS = oracle_mod.fwd(q, k, v, s[heads])
    go, gS = _host(o[:, heads]), _host(S[:, heads])
    for i, h in enumerate(heads):
        assert_close(go[:, i], ro[:, i], "bf16", "o head %d" % h)
        assert_close(gS[:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
    # the whole tensor is finite
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_decode_b64_1000_steps(oracle_mod):
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
    pairs = [(0, 0), (17, 5), (40, 16), (63, 31)]
    bi = torch.tensor([p[0] for p in pairs], device=dev)
    hi = torch.tensor([p[1] for p in pairs], device=dev)
    outs = torch.empty((steps, len(pairs), d), dtype=torch.bfloat16, device=dev)
    first = []
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    for t in range(steps):
        la.decode_step(qs[t], ks[t], vs[t], ts, tS, out=o)
        outs[t] = o[bi, hi]
        if t < 2:
            first.append(_host(o))
    torch.cuda.synchronize()
    # every row for the first two steps
    ref_state = S0.astype(np.float64)
    for t in range(2):
        ro, ref_state = oracle_mod.decode(_host(qs[t]), _host(ks[t]), _host(vs[t]), s, ref_state)
        assert_close(first[t], ro, "bf16", "o step %d" % t)
    # sampled rows over all steps: decode steps are the recurrent forward
    for j, (b, h) in enumerate(pairs):
        q = _host(qs[:, b, h])[None, None]
        k = _host(ks[:, b, h])[None, None]
        v = _host(vs[:, b, h])[None, None]
        ro, rS = oracle_mod.fwd(q, k, v, s[h:h + 1], S0[b:b + 1, h:h + 1])
        assert_close(_host(outs[:, j]), ro[0, 0], "bf16", "o (b=%d,h=%d)" % (b, h))
        assert_close(_host(tS[b, h]), rS[0, 0], "bf16", "state (b=%d,h=%d)" % (b, h), stored_bf16=False)


def test_train_32k_sampled_heads(oracle_mod):
    c = la_inputs.CONFIGS["train_32k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = device()
    tq, tk, tv = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    tg = la_inputs.upstream_grad_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    s = la_inputs.slopes(H)
    ts = torch.from_numpy(s).to(dev)
    o, _ = la.prefill(tq, tk, tv, ts, chunk=C, return_state=False)
    dq, dk, dv = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (3, 15)]:
        q, k, v, g = (_host(t[b:b + 1, h:h + 1]) for t in (tq, tk, tv, tg))
        sh = s[h:h + 1]
        ro, _ = oracle_mod.fwd(q, k, v, sh)
        rq, rk, rv = oracle_mod.bwd(q, k, v, g, sh)
        assert_close(_host(o[b:b + 1, h:h + 1]), ro, "bf16", "o (b=%d,h=%d)" % (b, h))
        assert_close(_host(dq[b:b + 1, h:h + 1]), rq, "bf16", "dq (b=%d,h=%d)" % (b, h))
        assert_close(_host(dk[b:b + 1, h:h + 1]), rk, "bf16", "dk (b=%d,h=%d)" % (b, h))
        assert_close(_host(dv[b:b + 1, h:h + 1]), rv, "bf16", "dv (b=%d,h=%d)" % (b, h))


def test_varlen_128k_sampled_heads(oracle_mod):
    """The benchmark's packed batch (64 ragged sequences, 131072 tokens,
    H=32, d=128, C=128, per-sequence initial states): every sequence of
    sampled heads against the oracle."""
    c = la_inputs.CONFIGS["varlen_128k"]
    H, d, C, nseq, T, seed = c["H"], c["d"], c["C"], c["nseq"], c["T"], c["seed"]
    dev = device()
    cu = la_inputs.packed_cu_seqlens(seed, nseq, T)
    tq, tk, tv = (x[0] for x in la_inputs.qkv_device(seed, 1, H, T, d, dev, torch.bfloat16))
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(seed, nseq, H, d)
    o, S = la.prefill_varlen(tq, tk, tv, torch.from_numpy(s).to(dev), cu, chunk=C,
                             state_in=torch.from_numpy(S0).to(dev))
    torch.cuda.synchronize()
    heads = [0, 31]
    q, k, v = (_host(t[heads]) for t in (tq, tk, tv))
    ro, rS = oracle_mod.fwd_varlen(q, k, v, s[heads], cu, S0[:, heads])
    go, gS = _host(o[heads]), _host(S[:, heads])
    for i, h in enumerate(heads):
        assert_close(go[i], ro[i], "bf16", "o head %d" % h)
        assert_close(gS[:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()


def test_prefill_gated_128k_sampled_heads(oracle_mod):
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
    heads = [0, 31]
    q, k, v, g = (_host(t[:, heads]) for t in (tq, tk, tv, tg))
    ry, rS = oracle_mod.fwd_gated(q, k, v, s[heads], g, w[heads], 1e-6)
    gy, gS = _host(y[:, heads]), _host(S[:, heads])
    for i, h in enumerate(heads):
        assert_close(gy[:, i], ry[:, i], "bf16", "y head %d" % h)
        assert_close(gS[:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
    assert torch.isfinite(y.float()).all()
