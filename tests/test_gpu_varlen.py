"""GPU parity of packed variable-length batches (la_prefill_varlen,
la_prefill_bwd_varlen) against the fp64 oracle, through the C ABI.

The cases mix empty, one-token, sub-chunk, ragged and multi-segment
sequences, so that the per-sequence segment plan, the piece pre-pass (one and
several pieces per segment), the skip rule and the state pass-through of an
empty sequence all run; 256 sequences is the largest batch the ABI takes.
"""
import numpy as np
import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import assert_close, device, to_dev, to_host

pytestmark = pytest.mark.gpu


def _packed_inputs(seed, H, T, d, dtype):
    q, k, v = la_inputs.qkv(seed, 1, H, T, d, dtype=dtype)
    return q[0], k[0], v[0]


def _ragged_cu(seed, nseq, max_len):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=nseq)
    return [0] + np.cumsum(lens).tolist()


def _run(q, k, v, s, cu, C, dtype, S0=None, S_out=None):
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    ts = torch.from_numpy(s).to(device())
    tS0 = None
    if S0 is not None:
        tS0 = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(device())
    o, S = la.prefill_varlen(tq, tk, tv, ts, cu, chunk=C, state_in=tS0,
                             state_out=tS0 if S_out == "in_place" else None)
    torch.cuda.synchronize()
    return to_host(o), to_host(S)


VARLEN_CASES = [
    # dtype, H, d, C, cu, with_state
    ("bf16", 2, 128, 64, [0, 1, 64, 64, 200, 1500], True),
    ("bf16", 4, 128, 128, [0, 3000, 3001, 7000], False),
    ("bf16", 1, 64, 32, [0, 17, 500, 2100], True),
    ("bf16", 3, 64, 128, [0, 0, 0, 50], True),
    ("bf16", 2, 128, 64, _ragged_cu(11, 256, 40), True),
    ("bf16", 8, 64, 64, [0, 40000], False),  # segments of 1280 tokens, 2 pieces each
    ("f32", 2, 32, 32, [0, 5, 5, 70, 300], True),
    ("f32", 1, 128, 64, [0, 100, 101], False),
    ("f32", 2, 64, 16, _ragged_cu(12, 40, 30), True),
]


@pytest.mark.parametrize("dtype,H,d,C,cu,with_state", VARLEN_CASES)
def test_varlen_prefill(oracle_mod, dtype, H, d, C, cu, with_state):
    T = cu[-1]
    q, k, v = _packed_inputs(600 + T, H, T, d, dtype)
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(9, len(cu) - 1, H, d) if with_state else None
    o, S = _run(q, k, v, s, cu, C, dtype, S0)
    ro, rS = oracle_mod.fwd_varlen(q, k, v, s, cu, S0)
    assert_close(o, ro, dtype, "o")
    assert_close(S, rS, dtype, "S", stored_bf16=False)


def test_varlen_prefix_caching_and_in_place_state(oracle_mod):
    """Continue every sequence from its cached prefix state, the state updated
    in place, and compare with the oracle over the whole sequences."""
    H, d, C = 4, 128, 64
    full = [0, 900, 1000, 3500]
    lens = np.diff(full)
    pre = np.array([300, 1, 1200])
    assert np.all(pre <= lens)
    T = full[-1]
    q, k, v = _packed_inputs(700, H, T, d, "bf16")
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(10, 3, H, d)
    ro, rS = oracle_mod.fwd_varlen(q, k, v, s, full, S0)
    # split every sequence into its prefix and the rest
    idx_a = np.concatenate([np.arange(full[j], full[j] + pre[j]) for j in range(3)])
    idx_b = np.concatenate([np.arange(full[j] + pre[j], full[j + 1]) for j in range(3)])
    cu_a = [0] + np.cumsum(pre).tolist()
    cu_b = [0] + np.cumsum(lens - pre).tolist()
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    ts = torch.from_numpy(s).to(device())
    state = torch.from_numpy(S0.astype(np.float32)).to(device())
    ia, ib = (torch.from_numpy(x).to(device()) for x in (idx_a, idx_b))
    oa, _ = la.prefill_varlen(tq[:, ia].contiguous(), tk[:, ia].contiguous(), tv[:, ia].contiguous(),
                              ts, cu_a, chunk=C, state_in=state, state_out=state)
    ob, _ = la.prefill_varlen(tq[:, ib].contiguous(), tk[:, ib].contiguous(), tv[:, ib].contiguous(),
                              ts, cu_b, chunk=C, state_in=state, state_out=state)
    torch.cuda.synchronize()
    o = np.empty_like(ro)
    o[:, idx_a] = to_host(oa)
    o[:, idx_b] = to_host(ob)
    assert_close(o, ro, "bf16", "o (prefix + continuation)")
    assert_close(to_host(state), rS, "bf16", "S (in place)", stored_bf16=False)


BWD_VARLEN_CASES = [
    ("bf16", 2, 128, 64, [0, 1, 64, 64, 200, 1500]),
    ("bf16", 3, 64, 32, [0, 0, 333, 2000]),
    # C = 128: the fused reverse pass runs 64-token chunks in 128-token-multiple segments
    ("bf16", 2, 128, 128, [0, 70, 70, 1100, 1300]),
    ("f32", 2, 64, 32, [0, 5, 5, 70, 300]),
]


@pytest.mark.parametrize("dtype,H,d,C,cu", BWD_VARLEN_CASES)
def test_varlen_backward(oracle_mod, dtype, H, d, C, cu):
    T = cu[-1]
    q, k, v = _packed_inputs(800 + T, H, T, d, dtype)
    g = la_inputs.upstream_grad(800 + T, 1, H, T, d, dtype=dtype)[0]
    s = la_inputs.slopes(H)
    tq, tk, tv, tg = (to_dev(x, dtype) for x in (q, k, v, g))
    dq, dk, dv = la.prefill_bwd_varlen(tq, tk, tv, tg, torch.from_numpy(s).to(device()), cu, chunk=C)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_mod.bwd_varlen(q, k, v, g, s, cu)
    assert_close(to_host(dq), rq, dtype, "dq")
    assert_close(to_host(dk), rk, dtype, "dk")
    assert_close(to_host(dv), rv, dtype, "dv")


@pytest.mark.parametrize("dtype,H,d,C,cu", [
    ("bf16", 2, 128, 64, [0, 1, 64, 64, 200, 1500]),
    ("bf16", 2, 128, 128, [0, 70, 70, 1100, 1300]),
    ("f32", 2, 64, 32, [0, 5, 5, 70, 300]),
])
def test_varlen_backward_reusing_forward_workspace(oracle_mod, dtype, H, d, C, cu):
    """la_prefill_bwd_varlen_reuse after la_prefill_varlen (no initial states)
    on the same workspace."""
    T = cu[-1]
    q, k, v = _packed_inputs(900 + T, H, T, d, dtype)
    g = la_inputs.upstream_grad(900 + T, 1, H, T, d, dtype=dtype)[0]
    s = la_inputs.slopes(H)
    tq, tk, tv, tg = (to_dev(x, dtype) for x in (q, k, v, g))
    ts = torch.from_numpy(s).to(device())
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    ws = torch.empty(max(la.workspace_bytes_varlen(0, code, H, d, C, cu), 16),
                     dtype=torch.uint8, device=device())
    la.prefill_varlen(tq, tk, tv, ts, cu, chunk=C, workspace=ws)
    dq, dk, dv = la.prefill_bwd_varlen(tq, tk, tv, tg, ts, cu, chunk=C, workspace=ws,
                                       reuse_forward_workspace=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_mod.bwd_varlen(q, k, v, g, s, cu)
    assert_close(to_host(dq), rq, dtype, "dq")
    assert_close(to_host(dk), rk, dtype, "dk")
    assert_close(to_host(dv), rv, dtype, "dv")
    dq2, dk2, dv2 = la.prefill_bwd_varlen(tq, tk, tv, tg, ts, cu, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    if dtype == "bf16" and la.workspace_bytes_varlen(0, code, H, d, C, cu) > 0:
        # a workspace without the states, or with the states of another cut of
        # the same tokens, gives NaN (the sequence table is part of the tag)
        ws.zero_()
        dq3, _, _ = la.prefill_bwd_varlen(tq, tk, tv, tg, ts, cu, chunk=C, workspace=ws,
                                          reuse_forward_workspace=True)
        torch.cuda.synchronize()
        assert torch.isnan(dq3.float()).all()
        cu2 = list(cu[:-2]) + [cu[-2] + 1, cu[-1]]
        ws2 = torch.empty(max(la.workspace_bytes_varlen(0, code, H, d, C, cu),
                              la.workspace_bytes_varlen(0, code, H, d, C, cu2)),
                          dtype=torch.uint8, device=device())
        la.prefill_varlen(tq, tk, tv, ts, cu2, chunk=C, workspace=ws2)
        dq4, _, _ = la.prefill_bwd_varlen(tq, tk, tv, tg, ts, cu, chunk=C, workspace=ws2,
                                          reuse_forward_workspace=True)
        torch.cuda.synchronize()
        assert torch.isnan(dq4.float()).all()
