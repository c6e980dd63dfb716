"""Calls on different streams run concurrently without interfering: the
library keeps no per-call state outside its arguments (the allocation-free
entry point's scratch buffer aside, whose overlapping calls are documented to
race and are not used here).  Two independent problems -- a segmented bf16
prefill with its own workspace each, and a decode step on its own state --
run on two streams (default priority), launched from one host thread and
then from two, and every result equals the sequential one bit for bit.
"""
import threading

import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import device

pytestmark = pytest.mark.gpu


class Problem:
    def __init__(self, dev, seed, H, N):
        B, d, self.C = 1, 128, 64
        self.q, self.k, self.v = la_inputs.qkv_device(seed, B, H, N, d, dev, torch.bfloat16)
        self.sl = torch.from_numpy(la_inputs.slopes(H)).to(dev)
        self.ws = torch.empty(la.workspace_bytes(0, la.LA_BF16, B, H, N, d, self.C),
                              dtype=torch.uint8, device=dev)
        self.o = torch.empty_like(self.q)
        self.S = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
        Bd, Hd = 16, H
        self.S0 = torch.from_numpy(la_inputs.decode_state(seed, Bd, Hd, d)).to(dev)
        self.state = self.S0.clone()
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        self.qd, self.kd, self.vd = ((torch.randn((Bd, Hd, d), generator=gen, device=dev)
                                      / d ** 0.5).to(torch.bfloat16) for _ in range(3))
        self.od = torch.empty((Bd, Hd, d), dtype=torch.bfloat16, device=dev)

    def run(self, stream, steps=3):
        with torch.cuda.stream(stream):  # the state reset is ordered on the same stream
            self.state.copy_(self.S0)
        for _ in range(steps):
            la.prefill(self.q, self.k, self.v, self.sl, chunk=self.C, out=self.o,
                       state_out=self.S, workspace=self.ws, stream=stream)
            la.decode_step(self.qd, self.kd, self.vd, self.sl, self.state, out=self.od,
                           stream=stream)

    def results(self):
        return [t.clone() for t in (self.o, self.S, self.od, self.state)]

    def clear(self):
        for t in (self.o, self.S, self.od):
            t.fill_(float("nan"))


def _check(problems, refs):
    for p, r in zip(problems, refs):
        for a, b in zip(p.results(), r):
            assert torch.equal(a, b)


def test_two_streams_one_thread():
    dev = device()
    ps = [Problem(dev, 21, 8, 4096), Problem(dev, 22, 4, 6144)]
    main = torch.cuda.current_stream()
    refs = []
    for p in ps:  # sequential reference
        p.run(main)
        torch.cuda.synchronize()
        refs.append(p.results())
    for p in ps:
        p.clear()
    streams = [torch.cuda.Stream() for _ in ps]
    for s in streams:
        s.wait_stream(main)
    for _ in range(2):
        for p, s in zip(ps, streams):
            p.run(s)
    torch.cuda.synchronize()
    _check(ps, refs)


def test_two_streams_two_threads():
    dev = device()
    ps = [Problem(dev, 23, 8, 4096), Problem(dev, 24, 16, 2048)]
    main = torch.cuda.current_stream()
    refs = []
    for p in ps:
        p.run(main)
        torch.cuda.synchronize()
        refs.append(p.results())
    for p in ps:
        p.clear()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in ps]
    errors = []

    def worker(p, s):
        try:
            with torch.cuda.device(dev):
                p.run(s)
                s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(p, s)) for p, s in zip(ps, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    _check(ps, refs)
