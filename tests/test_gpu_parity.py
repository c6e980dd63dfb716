"""GPU parity of the HIP path against the fp64 CPU oracle, through the C ABI.

Small shapes cover several chunks, ragged tails, every chunk length, both head
dims, both dtypes, the segmented and single-segment plans and the degenerate
decays.  The full-size workloads run in the same launch configuration the
benchmark uses and are checked on sampled heads (heads are independent, so
the oracle computes those heads exactly).
"""
import numpy as np
import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import assert_close, device, to_dev, to_host

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, N, d, dtype):
    q, k, v = la_inputs.qkv(seed, B, H, N, d, dtype=dtype)
    return q, k, v


def _run_prefill(q, k, v, s, C, dtype, S0=None):
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    ts = torch.from_numpy(s).to(device())
    tS0 = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(device())
    o, S = la.prefill(tq, tk, tv, ts, chunk=C, state_in=tS0)
    torch.cuda.synchronize()
    return to_host(o), to_host(S)


def test_tiny_f32_workload(oracle_mod):
    c = la_inputs.CONFIGS["tiny_f32"]
    q, k, v = _inputs(c["seed"], c["B"], c["H"], c["N"], c["d"], "f32")
    s = la_inputs.slopes(c["H"])
    o, S = _run_prefill(q, k, v, s, c["C"], "f32")
    ro, rS = oracle_mod.fwd(q, k, v, s)
    assert_close(o, ro, "f32", "o")
    assert_close(S, rS, "f32", "S", stored_bf16=False)


BF16_CASES = [
    # B, H, N, d, C, with_state
    (1, 2, 1, 128, 64, False),
    (1, 2, 37, 128, 64, True),
    (2, 3, 200, 128, 64, False),
    (1, 4, 513, 128, 128, True),
    (2, 2, 300, 128, 32, False),
    (1, 3, 777, 64, 64, True),
    (2, 2, 129, 64, 128, False),
    (1, 1, 1000, 64, 32, False),
    (16, 16, 100, 64, 64, False),  # 256 heads: single segment
    (1, 3, 301, 128, 16, True),    # C = 16 runs 32-token chunks
    (2, 2, 77, 64, 16, False),
]


@pytest.mark.parametrize("B,H,N,d,C,with_state", BF16_CASES)
def test_bf16_prefill(oracle_mod, B, H, N, d, C, with_state):
    q, k, v = _inputs(100 + N, B, H, N, d, "bf16")
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(7, B, H, d) if with_state else None
    o, S = _run_prefill(q, k, v, s, C, "bf16", S0)
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(o, ro, "bf16", "o")
    assert_close(S, rS, "bf16", "S", stored_bf16=False)


F32_CASES = [
    (1, 2, 1, 16, 16, False),
    (2, 2, 70, 32, 32, True),
    (1, 3, 300, 64, 128, True),
    (1, 2, 100, 128, 64, False),
]


@pytest.mark.parametrize("B,H,N,d,C,with_state", F32_CASES)
def test_f32_prefill(oracle_mod, B, H, N, d, C, with_state):
    q, k, v = _inputs(200 + N, B, H, N, d, "f32")
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(8, B, H, d) if with_state else None
    o, S = _run_prefill(q, k, v, s, C, "f32", S0)
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(o, ro, "f32", "o")
    assert_close(S, rS, "f32", "S", stored_bf16=False)


# fp32 rows of at most 256 tokens take the parallel form (one workgroup per
# 16 query rows and per 16 state rows), longer rows the chunked kernel: the
# cases straddle the 16-row blocks, the 64-key steps and the 256-token switch.
F32_SHORT_CASES = [(N, d) for d in (16, 64, 128) for N in (15, 17, 64, 65, 256, 257)] + [
    (1, 32), (200, 32)]


@pytest.mark.parametrize("N,d", F32_SHORT_CASES)
def test_f32_short_rows(oracle_mod, N, d):
    B, H, C = 2, 2, 64
    q, k, v = _inputs(500 + N + d, B, H, N, d, "f32")
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(9, B, H, d)
    o, S = _run_prefill(q, k, v, s, C, "f32", S0)
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(o, ro, "f32", "o")
    assert_close(S, rS, "f32", "S", stored_bf16=False)


def test_f32_short_rows_without_state_and_in_place(oracle_mod):
    B, H, N, d, C = 1, 4, 100, 64, 32
    q, k, v = _inputs(531, B, H, N, d, "f32")
    s = np.array([0.0, 1.0e4, 2.0**-8, 0.9], dtype=np.float32)  # degenerate decays too
    tq, tk, tv = (to_dev(x, "f32") for x in (q, k, v))
    ts = torch.from_numpy(s).to(device())
    # no state in or out: only the query-block workgroups run
    o, none = la.prefill(tq, tk, tv, ts, chunk=C, return_state=False)
    torch.cuda.synchronize()
    assert none is None
    ro, rS = oracle_mod.fwd(q, k, v, s)
    assert_close(to_host(o), ro, "f32", "o")
    # an in-place continuation (state_in is state_out) keeps the chunked kernel
    S0 = la_inputs.decode_state(10, B, H, d)
    tS = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(device())
    o2, S2 = la.prefill(tq, tk, tv, ts, chunk=C, state_in=tS, state_out=tS)
    torch.cuda.synchronize()
    ro2, rS2 = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(to_host(o2), ro2, "f32", "o in place")
    assert_close(to_host(S2), rS2, "f32", "S in place", stored_bf16=False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_degenerate_decays(oracle_mod, dtype):
    # slope 0 (no decay: every earlier token counts, no piece may be skipped),
    # a huge slope (only the current token counts) and ordinary slopes
    B, H, N, d = 1, 4, 700, 64
    q, k, v = _inputs(301, B, H, N, d, dtype)
    s = np.array([0.0, 1.0e4, 2.0**-8, 0.9], dtype=np.float32)
    o, S = _run_prefill(q, k, v, s, 64, dtype)
    ro, rS = oracle_mod.fwd(q, k, v, s)
    for h in range(H):
        assert_close(o[:, h], ro[:, h], dtype, "o head %d" % h)
        assert_close(S[:, h], rS[:, h], dtype, "S head %d" % h, stored_bf16=False)


def test_state_continuation_and_in_place(oracle_mod):
    B, H, N1, N2, d, C = 1, 4, 300, 200, 128, 64
    q, k, v = _inputs(302, B, H, N1 + N2, d, "bf16")
    s = la_inputs.slopes(H)
    dev = device()
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    ts = torch.from_numpy(s).to(dev)
    o1, S1 = la.prefill(tq[:, :, :N1].contiguous(), tk[:, :, :N1].contiguous(), tv[:, :, :N1].contiguous(), ts, chunk=C)
    # continue in place: state_in and state_out are the same buffer
    o2, S2 = la.prefill(tq[:, :, N1:].contiguous(), tk[:, :, N1:].contiguous(), tv[:, :, N1:].contiguous(), ts,
                        chunk=C, state_in=S1, state_out=S1)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.fwd(q, k, v, s)
    assert_close(np.concatenate([to_host(o1), to_host(o2)], axis=2), ro, "bf16", "o")
    assert_close(to_host(S2), rS, "bf16", "S", stored_bf16=False)


def test_pieces_truncated_by_decay(oracle_mod):
    """64 rows of 8192 tokens: four segments of 2048 tokens per row, cut into
    two pieces of 1024 for the pre-pass.  For the faster heads only the last
    tokens of the piece before a segment start carry a decay above 2^-32
    (32 tokens for head 0 at H = 16), so the piece pass starts near the end
    of its piece; the slowest heads use whole pieces.  Every row against the
    oracle, from an initial state."""
    B, H, N, d, C = 4, 16, 8192, 64, 64
    assert la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C) > 0  # a segmented plan
    q, k, v = _inputs(808, B, H, N, d, "bf16")
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(808, B, H, d)
    o, S = _run_prefill(q, k, v, s, C, "bf16", S0)
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(o, ro, "bf16", "o")
    assert_close(S, rS, "bf16", "S", stored_bf16=False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps(oracle_mod, dtype):
    B, H, d, steps = 3, 4, 128 if dtype == "bf16" else 64, 5
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(9, B, H, d)
    dev = device()
    tS = torch.from_numpy(S0).to(dev)
    ts = torch.from_numpy(s).to(dev)
    ref = S0.astype(np.float64)
    for t in range(steps):
        q, k, v = (x[:, :, 0] for x in la_inputs.qkv(9, B, H, 1, d, dtype=dtype, step=t))
        o = la.decode_step(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), ts, tS)
        torch.cuda.synchronize()
        ro, ref = oracle_mod.decode(q, k, v, s, ref)
        assert_close(to_host(o), ro, dtype, "o step %d" % t)
    assert_close(to_host(tS), ref, dtype, "state", stored_bf16=False)


def test_prefill_then_decode_equals_longer_prefill(oracle_mod):
    B, H, N, d, C = 2, 2, 130, 128, 64
    q, k, v = _inputs(303, B, H, N + 1, d, "bf16")
    s = la_inputs.slopes(H)
    dev = device()
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    ts = torch.from_numpy(s).to(dev)
    _, S = la.prefill(tq[:, :, :N].contiguous(), tk[:, :, :N].contiguous(), tv[:, :, :N].contiguous(), ts, chunk=C)
    o = la.decode_step(tq[:, :, N].contiguous(), tk[:, :, N].contiguous(), tv[:, :, N].contiguous(), ts, S)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.fwd(q, k, v, s)
    assert_close(to_host(o), ro[:, :, N], "bf16", "o")
    assert_close(to_host(S), rS, "bf16", "S", stored_bf16=False)


BWD_CASES = [
    # bf16 runs the fused dk/dv pass (with C = 128 in 64-token chunks inside
    # the 128-token-multiple segments), f32 the separate passes
    ("bf16", 1, 2, 200, 128, 64),
    ("bf16", 2, 2, 333, 64, 128),
    ("bf16", 1, 2, 300, 128, 128),
    ("bf16", 1, 3, 97, 128, 32),
    ("bf16", 1, 2, 500, 64, 64),
    ("bf16", 2, 3, 300, 64, 32),
    ("bf16", 16, 16, 70, 128, 64),  # 256 heads: one segment, no pre-pass
    ("bf16", 1, 2, 250, 128, 16),   # C = 16 runs 32-token chunks
    ("f32", 1, 2, 150, 64, 64),
    ("f32", 1, 2, 64, 16, 16),
]


@pytest.mark.parametrize("dtype,B,H,N,d,C", BWD_CASES)
def test_backward(oracle_mod, dtype, B, H, N, d, C):
    q, k, v = _inputs(400 + N, B, H, N, d, dtype)
    g = la_inputs.upstream_grad(400 + N, B, H, N, d, dtype=dtype)
    s = la_inputs.slopes(H)
    tq, tk, tv, tg = (to_dev(x, dtype) for x in (q, k, v, g))
    dq, dk, dv = la.prefill_bwd(tq, tk, tv, tg, torch.from_numpy(s).to(device()), chunk=C)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_mod.bwd(q, k, v, g, s)
    assert_close(to_host(dq), rq, dtype, "dq")
    assert_close(to_host(dk), rk, dtype, "dk")
    assert_close(to_host(dv), rv, dtype, "dv")


SPLIT_CASES = [
    ("bf16", 1, 4, 1000, 128, 128, True),  # several segments per row, with an initial state
    ("bf16", 2, 2, 300, 64, 64, False),
    ("f32", 1, 2, 100, 64, 64, True),      # fp32: no segments, no workspace
]


@pytest.mark.parametrize("dtype,B,H,N,d,C,with_state", SPLIT_CASES)
def test_prefill_in_two_calls_equals_prefill(dtype, B, H, N, d, C, with_state):
    """la_prefill_prepass then la_prefill_main (the two halves the benchmark
    times separately) give la_prefill's results bit for bit."""
    q, k, v = _inputs(600 + N, B, H, N, d, dtype)
    s = la_inputs.slopes(H)
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    ts = torch.from_numpy(s).to(device())
    tS0 = (torch.from_numpy(la_inputs.decode_state(10, B, H, d)).to(device())
           if with_state else None)
    o1, S1 = la.prefill(tq, tk, tv, ts, chunk=C, state_in=tS0)
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    ws = torch.empty(max(la.workspace_bytes(0, code, B, H, N, d, C), 16), dtype=torch.uint8,
                     device=device())
    o2 = torch.empty_like(tq)
    S2 = torch.empty_like(S1)
    la.prefill_prepass(tk, tv, ts, C, ws, state_in=tS0)
    la.prefill_main(tq, tk, tv, ts, C, ws, o2, state_out=S2, state_in=tS0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


REUSE_CASES = [
    ("bf16", 1, 2, 300, 128, 64),   # segments of one 64-token chunk
    ("bf16", 2, 2, 333, 64, 128),
    ("bf16", 1, 3, 500, 128, 32),
    ("bf16", 16, 16, 70, 128, 64),  # one segment per row: no states to reuse
    ("f32", 1, 2, 150, 64, 64),
]


@pytest.mark.parametrize("dtype,B,H,N,d,C", REUSE_CASES)
def test_backward_reusing_forward_workspace(oracle_mod, dtype, B, H, N, d, C):
    """la_prefill_bwd_reuse after la_prefill on the same workspace: the dq
    pass takes the forward's segment start states, transposed."""
    q, k, v = _inputs(500 + N, B, H, N, d, dtype)
    g = la_inputs.upstream_grad(500 + N, B, H, N, d, dtype=dtype)
    s = la_inputs.slopes(H)
    tq, tk, tv, tg = (to_dev(x, dtype) for x in (q, k, v, g))
    ts = torch.from_numpy(s).to(device())
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    ws = torch.empty(max(la.workspace_bytes(0, code, B, H, N, d, C), 16), dtype=torch.uint8,
                     device=device())
    la.prefill(tq, tk, tv, ts, chunk=C, workspace=ws)
    dq, dk, dv = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C, workspace=ws,
                                reuse_forward_workspace=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle_mod.bwd(q, k, v, g, s)
    assert_close(to_host(dq), rq, dtype, "dq")
    assert_close(to_host(dk), rk, dtype, "dk")
    assert_close(to_host(dv), rv, dtype, "dv")
    # dk and dv come from the same passes as in la_prefill_bwd
    dq2, dk2, dv2 = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert_close(to_host(dq2), rq, dtype, "dq (own pre-pass)")
    if dtype == "bf16" and la.workspace_bytes(0, code, B, H, N, d, C) > 0:
        # the states are really read from the workspace, and checked: a
        # workspace without them gives NaN
        ws.zero_()
        dq3, _, _ = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C, workspace=ws,
                                   reuse_forward_workspace=True)
        torch.cuda.synchronize()
        assert torch.isnan(dq3.float()).all()


def test_foreign_workspace_gives_nan(oracle_mod):
    """The workspace tag: a reuse backward, or la_prefill_main, on a
    workspace that does not hold the states it expects writes NaN outputs;
    the right workspace gives the oracle's result."""
    B, H, N, d, C = 1, 2, 300, 128, 64
    q, k, v = _inputs(520, B, H, N, d, "bf16")
    g = la_inputs.upstream_grad(520, B, H, N, d, dtype="bf16")
    s = la_inputs.slopes(H)
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, g))
    ts = torch.from_numpy(s).to(device())
    nws = la.workspace_bytes(1, la.LA_BF16, B, H, N, d, C)
    assert nws > 0
    ws = torch.empty(nws, dtype=torch.uint8, device=device())
    # forward over a copy of k (same values, another buffer): not this k's states
    la.prefill(tq, tk.clone(), tv, ts, chunk=C, workspace=ws)
    dq, dk, dv = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C, workspace=ws,
                                reuse_forward_workspace=True)
    dq0, dk0, dv0 = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C)
    torch.cuda.synchronize()
    assert torch.isnan(dq.float()).all()
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)  # dk, dv do not read it
    # the right forward, then two reuse calls: the first overwrites the states
    la.prefill(tq, tk, tv, ts, chunk=C, workspace=ws)
    dq1, _, _ = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C, workspace=ws,
                               reuse_forward_workspace=True)
    dq2, _, _ = la.prefill_bwd(tq, tk, tv, tg, ts, chunk=C, workspace=ws,
                               reuse_forward_workspace=True)
    torch.cuda.synchronize()
    rq, _, _ = oracle_mod.bwd(q, k, v, g, s)
    assert_close(to_host(dq1), rq, "bf16", "dq")
    assert torch.isnan(dq2.float()).all()
    # la_prefill_main after a prepass with another initial state
    S0 = torch.from_numpy(la_inputs.decode_state(21, B, H, d)).to(device())
    la.prefill_prepass(tk, tv, ts, C, ws, state_in=S0)
    o = torch.empty_like(tq)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=device())
    la.prefill_main(tq, tk, tv, ts, C, ws, o, state_out=S, state_in=None)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(S).all()
    la.prefill_main(tq, tk, tv, ts, C, ws, o, state_out=S, state_in=S0)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.fwd(q, k, v, s, to_host(S0))
    assert_close(to_host(o), ro, "bf16", "o")
    assert_close(to_host(S), rS, "bf16", "S", stored_bf16=False)


def test_in_place_continuation_many_segments(oracle_mod):
    """state_out == state_in on a plan with many segments per row (and more
    workgroups than compute units): the first segment reads the pre-pass's
    copy of the initial state, so the last segment's write cannot race it."""
    B, H, N, d, C = 1, 3, 6000, 64, 32
    q, k, v = _inputs(521, B, H, N, d, "bf16")
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(22, B, H, d)
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    tS = torch.from_numpy(S0).to(device())
    o, _ = la.prefill(tq, tk, tv, torch.from_numpy(s).to(device()), chunk=C, state_in=tS,
                      state_out=tS)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(to_host(o), ro, "bf16", "o")
    assert_close(to_host(tS), rS, "bf16", "S", stored_bf16=False)


def test_bitwise_deterministic():
    B, H, N, d, C = 1, 8, 2048, 128, 128
    q, k, v = _inputs(500, B, H, N, d, "bf16")
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    ts = torch.from_numpy(la_inputs.slopes(H)).to(device())
    o1, S1 = la.prefill(tq, tk, tv, ts, chunk=C)
    o2, S2 = la.prefill(tq, tk, tv, ts, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_chunk_length_changes_only_rounding(oracle_mod):
    B, H, N, d = 1, 4, 1000, 128
    q, k, v = _inputs(501, B, H, N, d, "bf16")
    s = la_inputs.slopes(H)
    ro, rS = oracle_mod.fwd(q, k, v, s)
    for C in (16, 32, 64, 128):
        o, S = _run_prefill(q, k, v, s, C, "bf16")
        assert_close(o, ro, "bf16", "o C=%d" % C)
        assert_close(S, rS, "bf16", "S C=%d" % C, stored_bf16=False)


DECODE_TOKENS_CASES = [
    # dtype, B, H, K, d
    ("bf16", 3, 4, 1, 128),
    ("bf16", 2, 3, 3, 128),
    ("bf16", 2, 3, 4, 128),
    ("bf16", 2, 3, 8, 64),
    ("bf16", 2, 3, 16, 128),  # largest K of the streaming kernel
    ("bf16", 2, 3, 13, 128),  # o reduced in rounds of 4 tokens, the last one short
    ("f32", 2, 2, 9, 32),
    ("bf16", 2, 2, 17, 64),  # smallest K of the chunk path
    ("bf16", 2, 2, 33, 64),
    ("f32", 3, 2, 7, 16),
    ("bf16", 1, 2, 128, 128),
    ("f32", 2, 3, 5, 64),
    ("f32", 1, 2, 70, 32),
]


@pytest.mark.parametrize("dtype,B,H,K,d", DECODE_TOKENS_CASES)
def test_decode_tokens(oracle_mod, dtype, B, H, K, d):
    """K tokens on a carried state in one call: the oracle's prefill from that
    state (which equals K decode steps, a pinned identity)."""
    q, k, v = _inputs(900 + K, B, H, K, d, dtype)
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(11, B, H, d)
    tq, tk, tv = (to_dev(x, dtype) for x in (q, k, v))
    tS = torch.from_numpy(S0).to(device())
    o = la.decode_tokens(tq, tk, tv, torch.from_numpy(s).to(device()), tS)
    torch.cuda.synchronize()
    ro, rS = oracle_mod.fwd(q, k, v, s, S0)
    assert_close(to_host(o), ro, dtype, "o")
    assert_close(to_host(tS), rS, dtype, "S", stored_bf16=False)


@pytest.mark.parametrize("load_policy,store_policy", [
    (0, 0), (la.CPOL_NT, la.CPOL_NT), (la.CPOL_NT, la.CPOL_SC1)])
def test_stream_probe_scales_in_place(load_policy, store_policy):
    # the measurement helper the decode step is compared with: x <- a x over
    # three full 1024-float4 workgroups and a ragged fourth, every element once
    n = 4 * (3 * 1024 + 100)
    g = torch.Generator(device="cpu").manual_seed(11)
    x0 = torch.randn(n + 64, generator=g, dtype=torch.float32)
    x = x0.to(device())
    la.probe_stream_rmw(x[:n], a=2.0, load_policy=load_policy, store_policy=store_policy)
    torch.cuda.synchronize()
    got = x.cpu()
    assert torch.equal(got[:n], 2.0 * x0[:n])
    assert torch.equal(got[n:], x0[n:])  # nothing past n is touched


def test_decode_tokens_equals_single_steps():
    """Against K calls of la_decode_step on the same inputs (bf16)."""
    B, H, K, d = 4, 8, 6, 128
    q, k, v = _inputs(950, B, H, K, d, "bf16")
    s = torch.from_numpy(la_inputs.slopes(H)).to(device())
    S0 = torch.from_numpy(la_inputs.decode_state(12, B, H, d)).to(device())
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    Sa = S0.clone()
    oa = la.decode_tokens(tq, tk, tv, s, Sa)
    Sb = S0.clone()
    ob = torch.stack([la.decode_step(tq[:, :, j].contiguous(), tk[:, :, j].contiguous(),
                                     tv[:, :, j].contiguous(), s, Sb) for j in range(K)], dim=2)
    torch.cuda.synchronize()
    ref = to_host(ob)
    assert_close(to_host(oa), ref, "bf16", "o vs decode steps")
    assert_close(to_host(Sa), to_host(Sb), "bf16", "S vs decode steps", stored_bf16=False)


GATED_CASES = [
    # dtype, B, H, N, d, C, with_state
    ("bf16", 1, 2, 1, 128, 64, False),
    ("bf16", 1, 3, 300, 128, 128, True),
    ("bf16", 2, 2, 200, 128, 32, False),
    ("bf16", 1, 4, 777, 64, 64, True),
    ("bf16", 16, 16, 70, 128, 64, False),  # 256 heads: single segment
    ("f32", 1, 2, 100, 128, 64, True),
    ("f32", 2, 2, 70, 32, 32, False),
]


@pytest.mark.parametrize("dtype,B,H,N,d,C,with_state", GATED_CASES)
def test_prefill_gated(oracle_mod, dtype, B, H, N, d, C, with_state):
    """The fused output epilogue (per-head RMSNorm, weight, sigmoid gate)."""
    q, k, v = _inputs(1000 + N, B, H, N, d, dtype)
    g = la_inputs.gate(1000 + N, B, H, N, d, dtype=dtype)
    w = la_inputs.norm_weight(1000 + N, H, d)
    s = la_inputs.slopes(H)
    S0 = la_inputs.decode_state(13, B, H, d) if with_state else None
    eps = 1e-6
    tq, tk, tv, tg = (to_dev(x, dtype) for x in (q, k, v, g))
    tS0 = None if S0 is None else torch.from_numpy(S0).to(device())
    y, S = la.prefill_gated(tq, tk, tv, torch.from_numpy(s).to(device()), tg,
                            torch.from_numpy(w).to(device()), eps=eps, chunk=C, state_in=tS0)
    torch.cuda.synchronize()
    ry, rS = oracle_mod.fwd_gated(q, k, v, s, g, w, eps, S0)
    assert_close(to_host(y), ry, dtype, "y")
    assert_close(to_host(S), rS, dtype, "S", stored_bf16=False)
