#!/usr/bin/env python3
"""Benchmark of the Lightning Attention layer on one MI355X.

One JSON line on stdout.  The headline ("value") is bf16 prefill throughput in
tokens/s on the 128K-token workload (B=1, H=32, N=131072, d=128, chunk 128):
one step is one whole la_prefill call (segment pre-pass + main pass) over the
sequence, inputs resident in HBM.  The same line carries:
  * "roofline": the main prefill kernel's algorithmic HBM bytes per launch over
    its HIP-event-timed average duration, against 8 TB/s;
  * "decode": the batched decode step (B=64, H=32, d=128), 1000 consecutive
    steps with fresh q/k/v each, microseconds per step and HBM fraction;
  * "prefill_gated": the same prefill with the fused output epilogue
    (per-head RMSNorm, weight, sigmoid gate);
  * "decode_tokens": 4 new tokens per (b, h) per call on the same state
    (multi-token generation / draft verification), microseconds per call;
  * "train": forward + backward at B=4, H=16, N=32768, d=128, chunk 64;
  * "varlen": a packed batch of 64 ragged sequences (131072 tokens, H=32,
    d=128, chunk 128) continuing from per-sequence states, forward and
    backward;
  * "cpu_baseline": the fp64 CPU oracle on a bounded sample of the headline
    workload (the first tokens of all 32 heads), on the host's cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix, TFLOP/s
METRIC = "Lightning-attn prefill tokens/s at 128K; decode-step μs; % of MFMA/HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_code_digest():
    """sha256 of the main prefill kernel's code: its two source files with
    // comments, indentation and blank lines removed, so that edits to
    comments alone do not invalidate counters taken on the same code."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in ("la_fwd_bf16.hip", "la_common.h"):
        with open(os.path.join(ROOT, "hybrid_linear_attention_lightning_amd", "csrc", f)) as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the main prefill kernel from the committed
    FETCH_SIZE / WRITE_SIZE summary, or None when the kernel code has
    changed since those counters were taken (its digest no longer matches)."""
    import re

    path = os.path.join(ROOT, "profiles", "prefill_128k_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    m_h = re.search(r"^kernel_code_sha256: ([0-9a-f]{64})$", text, re.M)
    if not (m_t and m_h):
        return None
    return int(m_t.group(1)) if kernel_code_digest() == m_h.group(1) else None


def prefill_counts(B, H, N, d, C):
    """Algorithmic bytes and flops of one forward pass (q, k, v read, o
    written, final state written; causal intra-chunk products counted once)."""
    bytes_ = 4 * B * H * N * d * 2 + B * H * d * d * 4
    flops = B * H * N * (2 * (C + 1) * d + 4 * d * d)
    return bytes_, flops


def prefill_mfma_executed(B, H, N, d, C):
    """Matrix-core flops the bf16 kernel issues: causal 16x16 score tiles, and
    hi+lo passes for P.V, S.Q and K^T.(bV)."""
    nqb, ksd, ksc, nt = C // 16, d // 32, C // 32, d // 16
    tiles = nqb * (nqb + 1) // 2 * ksd
    pv = nt * sum(qb // 2 + 1 for qb in range(nqb)) * 2
    inter = nt * nqb * ksd * 2
    state = nt * nt * ksc * 2
    chunks = B * H * ((N + C - 1) // C)
    return chunks * (tiles + pv + inter + state) * 16 * 16 * 32 * 2


def bench_prefill(args, torch, la, la_inputs):
    B, H, N, d, C = 1, 32, 131072, 128, 128
    dev = torch.device("cuda:0")
    q, k, v = la_inputs.qkv_device(2, B, H, N, d, dev, torch.bfloat16)
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    o = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(e0=None, e1=None, e2=None):
        if e0 is not None:
            e0.record(stream)
        la.prefill_prepass(k, v, slope, C, ws, stream=stream)
        if e1 is not None:
            e1.record(stream)
        la.prefill_main(q, k, v, slope, C, ws, o, state_out=S, stream=stream)
        if e2 is not None:
            e2.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(*ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev[0][0].elapsed_time(ev[-1][2])
    main_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    ms_per_step = total_ms / args.steps
    bytes_, flops = prefill_counts(B, H, N, d, C)
    achieved = bytes_ / (main_ms * 1e-3) / 1e9
    res = {
        "B": B, "H": H, "N": N, "d": d, "C": C,
        "ms_per_step": ms_per_step,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "tokens_per_s": B * N / (ms_per_step * 1e-3),
        "main_kernel_ms": main_ms,
        "prepass_ms": pre_ms,
        "roofline": {
            "kernel": "fwd_bf16_kernel<128,128> (la_prefill_main)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "bytes_per_launch": bytes_,
        },
        "mfma": {
            "algorithmic_tflops": flops / (main_ms * 1e-3) / 1e12,
            "algorithmic_frac": flops / (main_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS,
            "executed_tflops": prefill_mfma_executed(B, H, N, d, C) / (main_ms * 1e-3) / 1e12,
            "executed_frac": prefill_mfma_executed(B, H, N, d, C) / (main_ms * 1e-3) / 1e12
            / BF16_MFMA_PEAK_TFS,
            "peak_tflops": BF16_MFMA_PEAK_TFS,
        },
        "workspace_bytes": nws,
    }
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return res


def bench_prefill_gated(args, torch, la, la_inputs):
    """The 128K prefill with the fused output epilogue (per-head RMSNorm,
    weight, sigmoid gate): whole la_prefill_gated calls."""
    c = la_inputs.CONFIGS["prefill_128k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = torch.device("cuda:0")
    q, k, v = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    gate = la_inputs.gate_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    w = torch.from_numpy(la_inputs.norm_weight(c["seed"], H, d)).to(dev)
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    y = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    nws = la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        la.prefill_gated(q, k, v, slope, gate, w, eps=1e-6, chunk=C, out=y, state_out=S,
                         workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    bytes_ = prefill_counts(B, H, N, d, C)[0] + B * H * N * d * 2  # + the gate read
    res = {
        "B": B, "H": H, "N": N, "d": d, "C": C,
        "ms_per_step": ms,
        "tokens_per_s": B * N / (ms * 1e-3),
        "hbm_frac_whole_call": bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "note": "bytes: q, k, v, gate read, y written, final state written",
    }
    del q, k, v, gate, y, ws
    torch.cuda.empty_cache()
    return res


def bench_decode_graph(torch, la, qs, ks, vs, slope, S0, o, stream):
    """The first 100 decode steps captured once in a HIP graph and replayed.
    The state after one replay is checked bit for bit against the same 100
    steps run eagerly; the timing is reported only if they agree."""
    n = min(100, qs.shape[0])
    S = S0.clone()
    for i in range(n):
        la.decode_step(qs[i], ks[i], vs[i], slope, S, out=o, stream=stream)
    torch.cuda.synchronize()
    S_eager = S.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.copy_(S0)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                la.decode_step(qs[i], ks[i], vs[i], slope, S, out=o, stream=side)
    torch.cuda.synchronize()
    S.copy_(S0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(S, S_eager):
        return {"us_per_step": None, "note": "graph replay differed from eager execution"}
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return {"us_per_step": e0.elapsed_time(e1) * 1e3 / (reps * n), "steps_per_graph": n,
            "replays": reps}


def bench_decode(args, torch, la, la_inputs):
    B, H, d, steps = 64, 32, 128, args.decode_steps
    dev = torch.device("cuda:0")
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    S0 = torch.from_numpy(la_inputs.decode_state(3, B, H, d)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    scale = 1.0 / d ** 0.5
    qs, ks, vs = (
        (torch.randn((steps, B, H, d), generator=g, device=dev) * scale).to(torch.bfloat16)
        for _ in range(3)
    )
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    S = S0.clone()
    stream = torch.cuda.current_stream()
    for i in range(min(10, steps)):
        la.decode_step(qs[i], ks[i], vs[i], slope, S, out=o, stream=stream)
    S.copy_(S0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        la.decode_step(qs[i], ks[i], vs[i], slope, S, out=o, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    bytes_ = 2 * B * H * d * d * 4 + 4 * B * H * d * 2
    achieved = bytes_ / (us * 1e-6) / 1e9
    graph = bench_decode_graph(torch, la, qs, ks, vs, slope, S0, o, stream)
    # context: what a plain device-to-device copy (torch, the same read +
    # write pattern without arithmetic) reaches on this GPU
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        b.copy_(a)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * a.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b
    # cold steps: the same steps rotate over four copies of the state (537 MB,
    # twice the 256 MB Infinity Cache), so each step's state was last touched
    # three steps (805 MB of traffic) earlier and comes from HBM
    n_rot, cold_steps = 4, min(200, steps)
    Ss = [S0.clone() for _ in range(n_rot)]
    for i in range(2 * n_rot):
        la.decode_step(qs[i], ks[i], vs[i], slope, Ss[i % n_rot], out=o, stream=stream)
    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(cold_steps):
        la.decode_step(qs[i], ks[i], vs[i], slope, Ss[i % n_rot], out=o, stream=stream)
    k1.record(stream)
    torch.cuda.synchronize()
    cold_us = k0.elapsed_time(k1) * 1e3 / cold_steps
    del Ss
    res = {
        "B": B, "H": H, "d": d, "steps": steps,
        "us_per_step": us,
        "graph": graph,
        "tokens_per_s": B / (us * 1e-6),
        "roofline": {"kernel": "decode_kernel<128>", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "bytes_per_launch": bytes_},
        "copy_GBs": copy_gbs,
        "cold": {"us_per_step": cold_us, "steps": cold_steps,
                 "hbm_frac": bytes_ / (cold_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                 "note": "consecutive steps rotating over 4 state copies (537 MB), so no "
                         "step finds its state in the Infinity Cache"},
        "note": "the 134 MB state fits the 256 MB Infinity Cache, so repeated steps can "
                "exceed the HBM rate; copy_GBs is a plain 1 GiB device copy (bytes read + "
                "written per second) for comparison",
    }
    del qs, ks, vs, S, S0
    torch.cuda.empty_cache()
    return res


def bench_decode_tokens(args, torch, la, la_inputs):
    """Multi-token decode: K = 4 new tokens per (b, h) per call on the B=64,
    H=32, d=128 decode state, 250 consecutive calls with fresh q, k, v."""
    B, H, d, K, calls = 64, 32, 128, 4, 250
    dev = torch.device("cuda:0")
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    S0 = torch.from_numpy(la_inputs.decode_state(3, B, H, d)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(33)
    scale = 1.0 / d ** 0.5
    qs, ks, vs = (
        (torch.randn((calls, B, H, K, d), generator=g, device=dev) * scale).to(torch.bfloat16)
        for _ in range(3)
    )
    o = torch.empty((B, H, K, d), dtype=torch.bfloat16, device=dev)
    S = S0.clone()
    stream = torch.cuda.current_stream()
    for i in range(10):
        la.decode_tokens(qs[i], ks[i], vs[i], slope, S, out=o, stream=stream)
    S.copy_(S0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(calls):
        la.decode_tokens(qs[i], ks[i], vs[i], slope, S, out=o, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    bytes_ = 2 * B * H * d * d * 4 + 4 * B * H * K * d * 2
    achieved = bytes_ / (us * 1e-6) / 1e9
    res = {
        "B": B, "H": H, "d": d, "K": K, "calls": calls,
        "us_per_call": us,
        "tokens_per_s": B * K / (us * 1e-6),
        "roofline": {"kernel": "decode_kernel<128, bf16, 4> (la_decode_tokens)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "bytes_per_launch": bytes_},
    }
    del qs, ks, vs, S, S0
    torch.cuda.empty_cache()
    return res


def bench_train(args, torch, la, la_inputs):
    B, H, N, d, C = 4, 16, 32768, 128, 64
    dev = torch.device("cuda:0")
    q, k, v = la_inputs.qkv_device(4, B, H, N, d, dev, torch.bfloat16)
    dout = la_inputs.upstream_grad_device(4, B, H, N, d, dev, torch.bfloat16)
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    nws = max(la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C),
              la.workspace_bytes(1, la.LA_BF16, B, H, N, d, C))
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    steps = max(2, args.train_steps)

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        la.prefill(q, k, v, slope, chunk=C, out=o, return_state=False, workspace=ws, stream=stream)
        if e is not None:
            e[1].record(stream)
        # the backward keeps the forward's workspace and reuses its segment
        # start states for the dq pass
        la.prefill_bwd(q, k, v, dout, slope, chunk=C, dq=dq, dk=dk, dv=dv, workspace=ws,
                       stream=stream, reuse_forward_workspace=True)
        if e is not None:
            e[2].record(stream)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fb, _ = prefill_counts(B, H, N, d, C)
    bb = 7 * B * H * N * d * 2
    res = {
        "B": B, "H": H, "N": N, "d": d, "C": C,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "tokens_per_s": B * N / ((fwd_ms + bwd_ms) * 1e-3),
        "fwd_hbm_frac": fb / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "bwd_hbm_frac": bb / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "bwd_bytes_note": "7 tensors of B*H*N*d bf16 (q, k, v, dout read; dq, dk, dv written)",
    }
    del q, k, v, dout, o, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def bench_varlen(args, torch, la, la_inputs):
    """Packed batch: 64 sequences of ragged lengths, 131072 tokens in all,
    H=32, d=128, C=128, every sequence continuing from its own cached state
    (state_in) and returning its final state; then the backward of the same
    batch (zero initial states)."""
    c = la_inputs.CONFIGS["varlen_128k"]
    H, d, C, nseq, T, seed = c["H"], c["d"], c["C"], c["nseq"], c["T"], c["seed"]
    dev = torch.device("cuda:0")
    cu = la_inputs.packed_cu_seqlens(seed, nseq, T)
    q, k, v = (x[0] for x in la_inputs.qkv_device(seed, 1, H, T, d, dev, torch.bfloat16))
    dout = la_inputs.upstream_grad_device(seed, 1, H, T, d, dev, torch.bfloat16)[0]
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    S0 = torch.from_numpy(la_inputs.decode_state(seed, nseq, H, d)).to(dev)
    S = torch.empty_like(S0)
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    nws = max(la.workspace_bytes_varlen(0, la.LA_BF16, H, d, C, cu),
              la.workspace_bytes_varlen(1, la.LA_BF16, H, d, C, cu))
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    steps = max(2, args.train_steps)

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        la.prefill_varlen(q, k, v, slope, cu, chunk=C, state_in=S0, out=o, state_out=S,
                          workspace=ws, stream=stream)
        if e is not None:
            e[1].record(stream)
        la.prefill_bwd_varlen(q, k, v, dout, slope, cu, chunk=C, dq=dq, dk=dk, dv=dv,
                              workspace=ws, stream=stream)
        if e is not None:
            e[2].record(stream)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fb = 4 * H * T * d * 2 + 2 * nseq * H * d * d * 4  # q, k, v, o; state in and out
    bb = 7 * H * T * d * 2
    lens = [b - a for a, b in zip(cu, cu[1:])]
    res = {
        "H": H, "d": d, "C": C, "nseq": nseq, "T": T,
        "lengths": {"min": min(lens), "max": max(lens), "mean": T / nseq},
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
        "fwd_tokens_per_s": T / (fwd_ms * 1e-3),
        "fwd_hbm_frac": fb / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "bwd_hbm_frac": bb / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "note": "fwd bytes: q, k, v read, o written, per-sequence states read and written",
    }
    del q, k, v, dout, o, dq, dk, dv, ws, S0, S
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, la_inputs):
    """The fp64 oracle on the first tokens of the 128K workload (all 32 heads),
    in pieces of 4096 tokens carried through the state, until about
    args.cpu_seconds of oracle time have passed."""
    import oracle

    oracle.build()
    B, H, d, piece = 1, 32, 128, 4096
    s = la_inputs.slopes(H)
    S = None
    done, spent = 0, 0.0
    while spent < args.cpu_seconds and done < 131072:
        q, k, v = la_inputs.qkv(2, B, H, piece, d, dtype="bf16", step=done // piece)
        t0 = time.perf_counter()
        _, S = oracle.fwd(q, k, v, s, S)
        spent += time.perf_counter() - t0
        done += piece
    return {
        "value": done / spent,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "fp64 recurrent oracle, first %d tokens of the B=1 H=32 d=128 prefill "
                  "(all 32 heads, bf16-valued inputs), %.1f s" % (done, spent),
    }


def copy_calibration(torch):
    """A plain 1 GiB device-to-device copy, for scaling HBM counters."""
    dev = torch.device("cuda:0")
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: 1 GiB copied (read 1 GiB, write 1 GiB)")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--train-steps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "train", "varlen"], default=None,
                    help="run one workload only (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB copy (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU; --gpus %d (WORLD_SIZE %d) is not "
              "supported: there is no multi-GPU path" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch

    import hybrid_linear_attention_lightning_amd as la
    import la_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    la.lib()
    if args.copy_calibration:
        copy_calibration(torch)
    out = {}
    if args.only in (None, "prefill"):
        log("prefill 128K ...")
        out["prefill"] = bench_prefill(args, torch, la, la_inputs)
        log("  %.3f ms/step" % out["prefill"]["ms_per_step"])
        log("prefill 128K with the fused output epilogue ...")
        out["prefill_gated"] = bench_prefill_gated(args, torch, la, la_inputs)
        log("  %.3f ms/step" % out["prefill_gated"]["ms_per_step"])
    if args.only in (None, "decode"):
        log("decode B=64 ...")
        out["decode"] = bench_decode(args, torch, la, la_inputs)
        log("  %.2f us/step (graph replay: %s us/step; cold, state evicted: %.2f us/step)" % (
            out["decode"]["us_per_step"], out["decode"]["graph"]["us_per_step"],
            out["decode"]["cold"]["us_per_step"]))
        log("decode 4 tokens per call, B=64 ...")
        out["decode_tokens"] = bench_decode_tokens(args, torch, la, la_inputs)
        log("  %.2f us/call" % out["decode_tokens"]["us_per_call"])
    if args.only in (None, "train"):
        log("train fwd+bwd B=4 H=16 N=32K ...")
        out["train"] = bench_train(args, torch, la, la_inputs)
        log("  fwd %.3f ms, bwd %.3f ms" % (out["train"]["fwd_ms"], out["train"]["bwd_ms"]))
    if args.only in (None, "varlen"):
        log("varlen fwd+bwd, 64 packed sequences, T=128K ...")
        out["varlen"] = bench_varlen(args, torch, la, la_inputs)
        log("  fwd %.3f ms, bwd %.3f ms" % (out["varlen"]["fwd_ms"], out["varlen"]["bwd_ms"]))
    cpu = None
    if not args.no_cpu_baseline and args.only in (None, "prefill"):
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(args, la_inputs)
        log("  %.1f tokens/s on %d threads" % (cpu["value"], cpu["cores"]))

    p = out.get("prefill")
    line = {
        "metric": METRIC,
        "value": p["tokens_per_s"] if p else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": p["ms_per_step"] if p else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: q,k,v ~ N(0,1)/sqrt(d) bf16, slopes 2^(-8(h+1)/H), torch seeded generator",
        "config": {"workload": "lightning-attention prefill, bf16, B=1 H=32 N=131072 d=128 chunk=128",
                   "B": 1, "H": 32, "N": 131072, "d": 128, "C": 128},
        "roofline": p["roofline"] if p else None,
        "cpu_baseline": cpu,
        "prefill": p,
        "prefill_gated": out.get("prefill_gated"),
        "decode": out.get("decode"),
        "decode_tokens": out.get("decode_tokens"),
        "train": out.get("train"),
        "varlen": out.get("varlen"),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
