#!/usr/bin/env python3
"""Benchmark of the Lightning Attention layer on one MI355X.

One JSON line on stdout.  The headline ("value") is bf16 prefill throughput in
tokens/s on the 128K-token workload (B=1, H=32, N=131072, d=128, chunk 128):
one step is one whole la_prefill call (segment pre-pass + main pass) over the
sequence, inputs resident in HBM.  The same line carries:
  * "roofline": the main prefill kernel's algorithmic HBM bytes per launch over
    its HIP-event-timed average duration, against 8 TB/s ("frac"), and the same
    bytes over the whole call ("frac_whole_call");
  * "prefill_8k": the 8K-token prefill (B=1, H=32, N=8192, d=128, chunk 64),
    timed and reported like the headline;
  * "tiny_f32": the tiny fp32 prefill (B=1, H=2, N=256, d=64, chunk 64),
    microseconds per call, back to back and replayed from a HIP graph;
  * "decode": the batched decode step (B=64, H=32, d=128), 1000 consecutive
    steps with fresh q/k/v each, microseconds per step and HBM fraction;
  * "prefill_gated": the same prefill with the fused output epilogue
    (per-head RMSNorm, weight, sigmoid gate);
  * "decode_tokens": 4 new tokens per (b, h) per call on the same state
    (multi-token generation / draft verification), microseconds per call,
    and in "k16" the same with 16 tokens per call;
  * "train": forward + backward at B=4, H=16, N=32768, d=128, chunk 64;
  * "varlen": a packed batch of 64 ragged sequences (131072 tokens, H=32,
    d=128, chunk 128) continuing from per-sequence states, forward and
    backward;
  * "cpu_baseline": the fp64 CPU oracle on a bounded sample of the headline
    workload (the first tokens of all 32 heads), on the host's cores, with the
    CPU model, the 8K prefill on all cores and on one core, and samples of the
    decode and training workloads;
  * "power" (unless --no-power or --only): the board power and shader clock the GPU reports
    (hwmon power1_input, power1_cap and pp_dpm_sclk under /sys/class/drm)
    while the 128K main prefill kernel, the gated prefill, the decode step
    (state from HBM), the training backward and the streaming probe each run
    back to back for --power-seconds.

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


def bench_prefill(args, torch, la, la_inputs, name="prefill_128k"):
    """Whole la_prefill calls on one of the prefill workloads, then the same
    steps as la_prefill_prepass + la_prefill_main with HIP events between
    them on the launch stream (the main kernel's own duration)."""
    c = la_inputs.CONFIGS[name]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = torch.device("cuda:0")
    q, k, v = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
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
    la.prefill(q, k, v, slope, chunk=C, out=o, state_out=S, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    # whole calls: events only around the K steps, so that no event sits
    # between the kernels of a step
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        la.prefill(q, k, v, slope, chunk=C, out=o, state_out=S, workspace=ws, stream=stream)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e_start.elapsed_time(e_end) / args.steps
    # the same K steps again with events between the pre-pass and the main
    # pass: the main kernel's own duration (the roofline's time base)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(*ev[i])
    torch.cuda.synchronize()
    main_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    evented_ms = ev[0][0].elapsed_time(ev[-1][2]) / args.steps
    bytes_, flops = prefill_counts(B, H, N, d, C)
    executed = prefill_mfma_executed(B, H, N, d, C)
    achieved = bytes_ / (main_ms * 1e-3) / 1e9
    whole = bytes_ / (ms_per_step * 1e-3) / 1e9

    def tfs(fl, ms):
        return fl / (ms * 1e-3) / 1e12

    res = {
        "B": B, "H": H, "N": N, "d": d, "C": C,
        "ms_per_step": ms_per_step,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "tokens_per_s": B * N / (ms_per_step * 1e-3),
        "main_kernel_ms": main_ms,
        "prepass_ms": pre_ms,
        "ms_per_step_with_split_events": evented_ms,
        "roofline": {
            "kernel": "fwd_bf16_kernel<%d,%d> (la_prefill_main)" % (C, d),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "frac_whole_call": whole / HBM_PEAK_GBS,
            "achieved_whole_call": whole,
            "traffic": measured_traffic() if name == "prefill_128k" else None,
            "bytes_per_launch": bytes_,
            "note": "frac: the main kernel alone (its HIP-event time); frac_whole_call: the "
                    "same algorithmic bytes over ms_per_step (pre-pass + main pass)",
        },
        "mfma": {
            "algorithmic_flops": flops,
            "executed_flops": executed,
            "algorithmic_frac_main": tfs(flops, main_ms) / BF16_MFMA_PEAK_TFS,
            "executed_frac_main": tfs(executed, main_ms) / BF16_MFMA_PEAK_TFS,
            "algorithmic_frac_whole_call": tfs(flops, ms_per_step) / BF16_MFMA_PEAK_TFS,
            "executed_frac_whole_call": tfs(executed, ms_per_step) / BF16_MFMA_PEAK_TFS,
            "peak_tflops": BF16_MFMA_PEAK_TFS,
            "note": "executed counts the hi+lo products and dense 16x16 causal tiles the "
                    "kernel issues (%.2fx the algorithmic flops)" % (executed / flops),
        },
        "workspace_bytes": nws,
    }
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return res


def bench_tiny_f32(args, torch, la, la_inputs):
    """The tiny fp32 workload (B=1, H=2, N=256, d=64, chunk 64): microseconds
    per la_prefill call, back to back from Python and replayed from a HIP
    graph (the replayed outputs are checked bit for bit against eager ones)."""
    c = la_inputs.CONFIGS["tiny_f32"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in la_inputs.qkv(c["seed"], B, H, N, d, "f32"))
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    o = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    calls = 500
    for _ in range(20):
        la.prefill(q, k, v, slope, chunk=C, out=o, state_out=S, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(calls):
        la.prefill(q, k, v, slope, chunk=C, out=o, state_out=S, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    o_eager, S_eager = o.clone(), S.clone()
    # the same call captured n times in one graph, replayed
    n, reps = 50, 20
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        o.zero_()
        S.zero_()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                la.prefill(q, k, v, slope, chunk=C, out=o, state_out=S, stream=side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    us_graph = None
    if torch.equal(o, o_eager) and torch.equal(S, S_eager):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) * 1e3 / (reps * n)
    return {"B": B, "H": H, "N": N, "d": d, "C": C, "dtype": "f32", "calls": calls,
            "us_per_call": us, "tokens_per_s": B * N / (us * 1e-6),
            "us_per_call_graph": us_graph, "calls_per_graph": n, "replays": reps,
            "note": "fwd_f32_quad_kernel: rows of at most 256 tokens in the parallel form, one "
                    "workgroup (two 256-thread halves taking alternate key steps) per 16 query "
                    "rows and per 16 state rows (40 here); us_per_call: "
                    "calls back to back from Python, us_per_call_graph: the same call replayed "
                    "from a HIP graph (null if a replay differed from the eager result)"}


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
    for i in range(200):  # untimed: the clock settles
        la.decode_step(qs[i % steps], ks[i % steps], vs[i % steps], slope, S, out=o, stream=stream)
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
    # the access pattern's ceiling: a streaming read-modify-write of state-sized
    # buffers (la_probe_stream_rmw: each float read once and written once, no
    # arithmetic of the layer), on one buffer and rotating over four, with the
    # decode kernel's cache policy (nt loads, sc1 stores) and two others
    probe = {}
    nf = B * H * d * d
    policies = (("nt_loads_sc1_stores", la.CPOL_NT, la.CPOL_SC1), ("plain", 0, 0),
                ("nt_loads_nt_stores", la.CPOL_NT, la.CPOL_NT))
    for pname, lp, sp in policies:
        for name, nbuf in (("warm", 1), ("cold", n_rot)):
            bufs = [torch.ones(nf, dtype=torch.float32, device=dev) for _ in range(nbuf)]
            for i in range(2 * nbuf):
                la.probe_stream_rmw(bufs[i % nbuf], 1.0, lp, sp, stream=stream)
            torch.cuda.synchronize()
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 200
            p0.record(stream)
            for i in range(reps):
                la.probe_stream_rmw(bufs[i % nbuf], 1.0, lp, sp, stream=stream)
            p1.record(stream)
            torch.cuda.synchronize()
            pus = p0.elapsed_time(p1) * 1e3 / reps
            probe["%s_%s" % (pname, name)] = {"us": pus, "GBs": 2 * nf * 4 / (pus * 1e-6) / 1e9}
            del bufs
    ceiling = probe["nt_loads_sc1_stores_cold"]["GBs"]
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
                 "frac_of_stream_ceiling": bytes_ / (cold_us * 1e-6) / 1e9 / ceiling,
                 "note": "consecutive steps rotating over 4 state copies (537 MB), so no "
                         "step finds its state in the Infinity Cache"},
        "stream_rmw_probe": probe,
        "frac_of_stream_ceiling_warm": achieved / probe["nt_loads_sc1_stores_warm"]["GBs"],
        "note": "the state is read with nt loads and written with sc1 stores; copy_GBs is a "
                "plain 1 GiB device copy (bytes read + written per second); stream_rmw_probe "
                "is la_probe_stream_rmw on state-sized buffers, the ceiling of the same access "
                "pattern (cold: rotating over 4 buffers)",
    }
    del qs, ks, vs, S, S0
    torch.cuda.empty_cache()
    return res


def _time_decode_tokens(torch, la, la_inputs, K, calls):
    """Microseconds per la_decode_tokens call with K new tokens per (b, h) on
    the B=64, H=32, d=128 decode state, over `calls` consecutive calls with
    fresh q, k, v, and the algorithmic bytes of one call."""
    B, H, d = 64, 32, 128
    dev = torch.device("cuda:0")
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    S0 = torch.from_numpy(la_inputs.decode_state(3, B, H, d)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(33 + K)
    scale = 1.0 / d ** 0.5
    qs, ks, vs = (
        (torch.randn((calls, B, H, K, d), generator=g, device=dev) * scale).to(torch.bfloat16)
        for _ in range(3)
    )
    o = torch.empty((B, H, K, d), dtype=torch.bfloat16, device=dev)
    S = S0.clone()
    stream = torch.cuda.current_stream()
    for i in range(200):  # untimed: the clock settles
        la.decode_tokens(qs[i % calls], ks[i % calls], vs[i % calls], slope, S, out=o, stream=stream)
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
    del qs, ks, vs, S, S0
    torch.cuda.empty_cache()
    return us, bytes_


def bench_decode_tokens(args, torch, la, la_inputs):
    """Multi-token decode: K = 4 new tokens per (b, h) per call on the B=64,
    H=32, d=128 decode state, 250 consecutive calls with fresh q, k, v; and
    the same with K = 16 (the largest count the streaming kernel takes), 100
    calls."""
    B, H, d, K, calls = 64, 32, 128, 4, 250
    us, bytes_ = _time_decode_tokens(torch, la, la_inputs, K, calls)
    achieved = bytes_ / (us * 1e-6) / 1e9
    us16, bytes16 = _time_decode_tokens(torch, la, la_inputs, 16, 100)
    achieved16 = bytes16 / (us16 * 1e-6) / 1e9
    return {
        "B": B, "H": H, "d": d, "K": K, "calls": calls,
        "us_per_call": us,
        "tokens_per_s": B * K / (us * 1e-6),
        "roofline": {"kernel": "decode_kernel<128, bf16, 4> (la_decode_tokens)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "bytes_per_launch": bytes_},
        "k16": {"K": 16, "calls": 100, "us_per_call": us16,
                "tokens_per_s": B * 16 / (us16 * 1e-6),
                "hbm_frac": achieved16 / HBM_PEAK_GBS, "bytes_per_launch": bytes16},
    }


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

    for _ in range(20):  # untimed: the clock settles
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

    for _ in range(20):  # untimed: the clock settles
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


_ONE_CORE = r"""
import json, sys, time
sys.path.insert(0, %r)
import la_inputs, oracle
c = la_inputs.CONFIGS["prefill_8k"]
heads = %d
q, k, v = la_inputs.qkv(c["seed"], c["B"], heads, c["N"], c["d"], dtype="bf16")
s = la_inputs.slopes(c["H"])[:heads]
t0 = time.perf_counter()
oracle.fwd(q, k, v, s)
print(json.dumps({"seconds": time.perf_counter() - t0, "threads": oracle.num_threads()}))
"""


def cpu_baseline(args, la_inputs):
    """The fp64 oracle (test infrastructure, timed as it stands) on bounded
    samples of the workloads, on the host's cores:
      * headline: the first tokens of the 128K prefill (all 32 heads), in
        pieces of 4096 tokens carried through the state, for about
        args.cpu_seconds;
      * the 8K prefill: all 32 heads on all cores, and 8 of its 32 heads in
        a child process with one OpenMP thread (scaled to 32 heads);
      * decode: a few B=64 H=32 steps; train: forward + backward of the first
        4096 tokens of every (b, h) row of the training workload."""
    import subprocess

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
    res = {
        "value": done / spent,
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "fp64 recurrent oracle, first %d tokens of the B=1 H=32 d=128 prefill "
                  "(all 32 heads, bf16-valued inputs), %.1f s" % (done, spent),
        "cpu_model": cpu_model(),
        "host_logical_cpus": os.cpu_count(),
    }
    # 8K prefill, all cores
    c = la_inputs.CONFIGS["prefill_8k"]
    q, k, v = la_inputs.qkv(c["seed"], c["B"], c["H"], c["N"], c["d"], dtype="bf16")
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, la_inputs.slopes(c["H"]))
    t8 = time.perf_counter() - t0
    res["prefill_8k"] = {"tokens_per_s": c["B"] * c["N"] / t8, "seconds": t8,
                         "threads": oracle.num_threads()}
    # 8K prefill, one core, 8 of the 32 heads (heads are independent)
    heads = 8
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _ONE_CORE % (ROOT, heads)], env=env,
                       capture_output=True, text=True, timeout=300)
    if r.returncode == 0:
        one = json.loads(r.stdout.strip().splitlines()[-1])
        t_full = one["seconds"] * c["H"] / heads
        res["prefill_8k_1core"] = {"tokens_per_s": c["B"] * c["N"] / t_full,
                                   "threads": one["threads"],
                                   "sample": "%d of %d heads in %.2f s, scaled to all heads"
                                             % (heads, c["H"], one["seconds"])}
    else:
        res["prefill_8k_1core"] = {"error": r.stderr[-500:]}
    del q, k, v
    # decode: a few steps of the B=64, H=32 state (the oracle copies the state
    # on each call; the copy is included)
    c = la_inputs.CONFIGS["decode_b64"]
    Bd, Hd, dd = c["B"], c["H"], c["d"]
    sd = la_inputs.slopes(Hd)
    st = la_inputs.decode_state(c["seed"], Bd, Hd, dd)
    nsteps = 5
    t0 = time.perf_counter()
    for i in range(nsteps):
        q1, k1, v1 = (x[:, :, 0] for x in la_inputs.qkv(c["seed"], Bd, Hd, 1, dd, "bf16", step=i))
        _, st = oracle.decode(q1, k1, v1, sd, st)
    td = (time.perf_counter() - t0) / nsteps
    res["decode_b64"] = {"us_per_step": td * 1e6, "tokens_per_s": Bd / td, "steps": nsteps}
    del st
    # train: forward + backward over the first 4096 tokens of every row
    c = la_inputs.CONFIGS["train_32k"]
    n = 4096
    q, k, v = la_inputs.qkv(c["seed"], c["B"], c["H"], n, c["d"], dtype="bf16")
    g = la_inputs.upstream_grad(c["seed"], c["B"], c["H"], n, c["d"], dtype="bf16")
    st_ = la_inputs.slopes(c["H"])
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, st_)
    t_f = time.perf_counter() - t0
    oracle.bwd(q, k, v, g, st_)
    t_b = time.perf_counter() - t0 - t_f
    res["train_32k"] = {"fwd_tokens_per_s": c["B"] * n / t_f, "bwd_tokens_per_s": c["B"] * n / t_b,
                        "sample": "first %d of %d tokens of all B=%d x H=%d rows"
                                  % (n, c["N"], c["B"], c["H"])}
    return res


def _sysfs_power_files():
    """hwmon power files and the sclk table of the first card that has them."""
    import glob

    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        inp = sorted(glob.glob(card + "/hwmon/hwmon*/power1_input")) or sorted(
            glob.glob(card + "/hwmon/hwmon*/power1_average"))
        if inp:
            cap = sorted(glob.glob(card + "/hwmon/hwmon*/power1_cap"))
            return inp[0], cap[0] if cap else None, card + "/pp_dpm_sclk"
    return None, None, None


def bench_power(args, torch, la, la_inputs):
    """Board power and shader clock while one kernel runs back to back: the
    GPU's own hwmon readings (microwatts) and its current sclk level, sampled
    every 50 ms from another thread, averaged over the steady part of each
    phase.  None if the files cannot be read."""
    import threading

    f_in, f_cap, f_sclk = _sysfs_power_files()
    if f_in is None:
        return None

    def read(f):
        try:
            with open(f) as fh:
                return fh.read()
        except OSError:
            return None

    if read(f_in) is None:
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            p_ = read(f_in)
            sc = read(f_sclk) or ""
            cur = [ln for ln in sc.splitlines() if ln.strip().endswith("*")]
            mhz = None
            if cur:
                try:
                    mhz = float(cur[0].split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
                except (IndexError, ValueError):
                    mhz = None
            samples.append((time.time(), float(p_) / 1e6 if p_ else None, mhz))
            time.sleep(0.05)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    phases = {}

    def phase(name, fn):
        torch.cuda.synchronize()
        t0 = time.time()
        calls = 0
        while time.time() - t0 < args.power_seconds:
            for _ in range(10):
                fn()
            calls += 10
            torch.cuda.synchronize()
        t1 = time.time()
        rows = [r for r in samples if t0 + 0.5 <= r[0] <= t1]
        pw = [r[1] for r in rows if r[1] is not None]
        mz = [r[2] for r in rows if r[2] is not None]
        phases[name] = {"board_W": sum(pw) / len(pw) if pw else None,
                        "board_W_max": max(pw) if pw else None,
                        "sclk_MHz": sum(mz) / len(mz) if mz else None,
                        "samples": len(rows), "calls": calls,
                        "ms_per_call": (t1 - t0) * 1e3 / calls}

    time.sleep(1.0)
    idle = [r[1] for r in samples if r[1] is not None]
    c = la_inputs.CONFIGS["prefill_128k"]
    B, H, N, d, C = c["B"], c["H"], c["N"], c["d"], c["C"]
    q, k, v = la_inputs.qkv_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    slope = torch.from_numpy(la_inputs.slopes(H)).to(dev)
    o = torch.empty_like(q)
    S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(la.workspace_bytes(0, la.LA_BF16, B, H, N, d, C), dtype=torch.uint8,
                     device=dev)
    la.prefill_prepass(k, v, slope, C, ws, stream=stream)
    phase("prefill_main_128k",
          lambda: la.prefill_main(q, k, v, slope, C, ws, o, state_out=S, stream=stream))
    g = la_inputs.gate_device(c["seed"], B, H, N, d, dev, torch.bfloat16)
    w = torch.from_numpy(la_inputs.norm_weight(c["seed"], H, d)).to(dev)
    phase("prefill_gated_128k",
          lambda: la.prefill_gated(q, k, v, slope, g, w, chunk=C, out=o, state_out=S,
                                   workspace=ws, stream=stream))
    del g, o, ws
    Bd, Hd = 64, 32
    S0 = torch.from_numpy(la_inputs.decode_state(3, Bd, Hd, d)).to(dev)
    Ss = [S0.clone() for _ in range(4)]
    qd = (torch.randn((Bd, Hd, d), device=dev) / d ** 0.5).to(torch.bfloat16)
    sd = torch.from_numpy(la_inputs.slopes(Hd)).to(dev)
    od = torch.empty_like(qd)
    step = [0]

    def dstep():
        step[0] += 1
        la.decode_step(qd, qd, qd, sd, Ss[step[0] % 4], out=od, stream=stream)

    phase("decode_state_from_hbm", dstep)
    del Ss, S0
    # training backward (B=4, H=16, N=32768, chunk 64) on the forward's workspace
    Bt, Ht, Nt, Ct = 4, 16, 32768, 64
    qt, kt, vt = la_inputs.qkv_device(4, Bt, Ht, Nt, d, dev, torch.bfloat16)
    gt = la_inputs.upstream_grad_device(4, Bt, Ht, Nt, d, dev, torch.bfloat16)
    st = torch.from_numpy(la_inputs.slopes(Ht)).to(dev)
    ot = torch.empty_like(qt)
    dq, dk, dv = torch.empty_like(qt), torch.empty_like(qt), torch.empty_like(qt)
    wst = torch.empty(max(la.workspace_bytes(0, la.LA_BF16, Bt, Ht, Nt, d, Ct),
                          la.workspace_bytes(1, la.LA_BF16, Bt, Ht, Nt, d, Ct)),
                      dtype=torch.uint8, device=dev)
    la.prefill(qt, kt, vt, st, chunk=Ct, out=ot, return_state=False, workspace=wst, stream=stream)
    phase("train_backward",
          lambda: la.prefill_bwd(qt, kt, vt, gt, st, chunk=Ct, dq=dq, dk=dk, dv=dv, workspace=wst,
                                 stream=stream, reuse_forward_workspace=True))
    del qt, kt, vt, gt, ot, dq, dk, dv, wst
    x = torch.ones(B * H * N * d // 2, dtype=torch.float32, device=dev)  # q, k, v's size
    phase("stream_rmw_probe", lambda: la.probe_stream_rmw(x, 1.0, stream=stream))
    stop.set()
    th.join()
    del q, k, v, x
    torch.cuda.empty_cache()
    cap = read(f_cap) if f_cap else None
    return {"cap_W": float(cap) / 1e6 if cap else None,
            "idle_W": sum(idle) / len(idle) if idle else None,
            "seconds_per_phase": args.power_seconds,
            "phases": phases,
            "source": f_in}


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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the clock settles at the power limit within tens of ms")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--train-steps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "small", "decode", "train", "varlen"],
                    default=None,
                    help="run one workload only (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB copy (HBM counter calibration)")
    ap.add_argument("--no-power", dest="power", action="store_false",
                    help="skip sampling board power and shader clock per kernel")
    ap.add_argument("--power-seconds", type=float, default=2.0)
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
    if args.only in (None, "small"):
        log("prefill 8K ...")
        out["prefill_8k"] = bench_prefill(args, torch, la, la_inputs, "prefill_8k")
        log("  %.1f us/step" % (out["prefill_8k"]["ms_per_step"] * 1e3))
        log("tiny fp32 prefill ...")
        out["tiny_f32"] = bench_tiny_f32(args, torch, la, la_inputs)
        log("  %.1f us/call (graph replay: %s us/call)" % (out["tiny_f32"]["us_per_call"],
                                                           out["tiny_f32"]["us_per_call_graph"]))
    if args.only in (None, "decode"):
        log("decode B=64 ...")
        out["decode"] = bench_decode(args, torch, la, la_inputs)
        log("  %.2f us/step (graph replay: %s us/step; cold, state evicted: %.2f us/step; "
            "streaming ceiling %.0f GB/s)" % (
                out["decode"]["us_per_step"], out["decode"]["graph"]["us_per_step"],
                out["decode"]["cold"]["us_per_step"],
                out["decode"]["stream_rmw_probe"]["nt_loads_sc1_stores_cold"]["GBs"]))
        log("decode 4 (and 16) tokens per call, B=64 ...")
        out["decode_tokens"] = bench_decode_tokens(args, torch, la, la_inputs)
        log("  %.2f us/call (16 tokens: %.2f us/call)" % (out["decode_tokens"]["us_per_call"],
                                                         out["decode_tokens"]["k16"]["us_per_call"]))
    if args.only in (None, "train"):
        log("train fwd+bwd B=4 H=16 N=32K ...")
        out["train"] = bench_train(args, torch, la, la_inputs)
        log("  fwd %.3f ms, bwd %.3f ms" % (out["train"]["fwd_ms"], out["train"]["bwd_ms"]))
    if args.only in (None, "varlen"):
        log("varlen fwd+bwd, 64 packed sequences, T=128K ...")
        out["varlen"] = bench_varlen(args, torch, la, la_inputs)
        log("  fwd %.3f ms, bwd %.3f ms" % (out["varlen"]["fwd_ms"], out["varlen"]["bwd_ms"]))
    if args.power and args.only is None:
        log("board power per kernel ...")
        out["power"] = bench_power(args, torch, la, la_inputs)
        if out["power"]:
            log("  " + ", ".join("%s %.0f W at %s MHz" % (k_, v_["board_W"] or 0, v_["sclk_MHz"])
                                 for k_, v_ in out["power"]["phases"].items()))
        else:
            log("  no readable power sensor")
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
        "prefill_8k": out.get("prefill_8k"),
        "tiny_f32": out.get("tiny_f32"),
        "prefill_gated": out.get("prefill_gated"),
        "decode": out.get("decode"),
        "decode_tokens": out.get("decode_tokens"),
        "train": out.get("train"),
        "varlen": out.get("varlen"),
    }
    if "power" in out:
        line["power"] = out["power"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
