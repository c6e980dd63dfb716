"""la_prefill_noalloc (no workspace: the library's static scratch buffer)
against la_prefill, through the C ABI: two calls in a row on the same GPU,
the second smaller, each checked against la_prefill's output (and the
oracle) to the bf16 bar."""
import ctypes

import numpy as np
import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import assert_close, device, to_dev, to_host

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, s, C, S0=None):
    """la_prefill_noalloc called through ctypes with preallocated outputs."""
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    code = la.lib().la_prefill_noalloc(
        la.LA_BF16, B, H, N, d, C, q.data_ptr(), k.data_ptr(), v.data_ptr(), s.data_ptr(),
        None if S0 is None else S0.data_ptr(), o.data_ptr(), S.data_ptr(), stream)
    assert code == 0, la.lib().la_status_string(code)
    return o, S


def test_noalloc_two_calls_match_prefill(oracle_mod):
    dev = device()
    # call 1: 64K tokens, 32 heads, C = 128: la_prefill's workspace (128 MiB)
    # exceeds the 64 MiB buffer, so the pieces are lengthened
    B, H, N, d, C = 1, 32, 65536, 128, 128
    assert la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C) > 64 << 20
    tq, tk, tv = la_inputs.qkv_device(31, B, H, N, d, dev, torch.bfloat16)
    s = la_inputs.slopes(H)
    ts = torch.from_numpy(s).to(dev)
    o1, S1 = _noalloc(tq, tk, tv, ts, C)
    r1, rS1 = la.prefill(tq, tk, tv, ts, chunk=C)
    torch.cuda.synchronize()
    go1, gS1 = to_host(o1), to_host(S1)
    assert_close(go1, to_host(r1), "bf16", "o (vs la_prefill)")
    assert_close(gS1, to_host(rS1), "bf16", "S (vs la_prefill)", stored_bf16=False)
    heads = [0, 15, 31]  # fastest, middle and slowest decay against the oracle
    q, k, v = (to_host(t[:, heads]) for t in (tq, tk, tv))
    ro, rS = oracle_mod.fwd(q, k, v, s[heads])
    for i, h in enumerate(heads):
        assert_close(go1[:, heads][:, i], ro[:, i], "bf16", "o head %d" % h)
        assert_close(gS1[:, heads][:, i], rS[:, i], "bf16", "S head %d" % h, stored_bf16=False)
    del tq, tk, tv, o1, S1, r1, rS1
    # call 2, smaller, with an initial state: la_prefill's plan fits, so the
    # results are la_prefill's bit for bit
    B, H, N, d, C = 2, 3, 1500, 64, 64
    q, k, v = la_inputs.qkv(32, B, H, N, d, dtype="bf16")
    s2 = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(32, B, H, d)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    ts2 = torch.from_numpy(s2).to(dev)
    tS0 = torch.from_numpy(S0).to(dev)
    o2, S2 = _noalloc(tq, tk, tv, ts2, C, tS0)
    r2, rS2 = la.prefill(tq, tk, tv, ts2, chunk=C, state_in=tS0)
    torch.cuda.synchronize()
    assert torch.equal(o2, r2) and torch.equal(S2, rS2)
    ro, rS = oracle_mod.fwd(q, k, v, s2, S0)
    assert_close(to_host(o2), ro, "bf16", "o")
    assert_close(to_host(S2), rS, "bf16", "S", stored_bf16=False)
