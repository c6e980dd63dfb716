"""GPU parity on seeded random shapes: prefill (with and without an initial
state, including slope-0 and very large slopes), backward and multi-token
decode, for both dtypes, every head dim and chunk length, and lengths drawn
around multiples of the chunk, of the segment and piece lengths and of the
256-token switch of the fp32 path.  Each case is checked against the fp64
oracle with the same bars as the hand-picked cases."""
import random

import numpy as np
import pytest
import torch

import la_inputs
import hybrid_linear_attention_lightning_amd as la
from tests._gpu import assert_close, device, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(rng):
    dt = rng.choice(["bf16", "bf16", "f32"])
    d = rng.choice([64, 128]) if dt == "bf16" else rng.choice([16, 32, 64, 128])
    C = rng.choice([16, 32, 64, 128])
    B, H = rng.choice([1, 1, 2, 3]), rng.choice([1, 2, 3, 5, 8])
    base = rng.choice([C, 64, 128, 256, 512, 1024])
    N = min(4000, max(1, base * rng.randint(1, 6) + rng.choice([-1, 0, 0, 1, 17, -C // 2])))
    kind = rng.choice(["fwd", "fwd", "bwd", "tokens"])
    odd_slope = rng.choice([None, None, 0.0, 1e4, 2.0 ** -12])
    with_state = rng.random() < 0.5
    K = rng.randint(1, 20)
    return dt, d, C, B, H, N, kind, odd_slope, with_state, K


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_random_shapes(oracle_mod, seed):
    rng = random.Random(seed)
    dev = device()
    for case in range(40):
        dt, d, C, B, H, N, kind, odd_slope, with_state, K = _case(rng)
        s = la_inputs.slopes(H).copy()
        if odd_slope is not None:
            s[0] = odd_slope
        ts = torch.from_numpy(s).to(dev)
        tag = "seed %d case %d: %s d=%d C=%d B=%d H=%d N=%d %s" % (seed, case, dt, d, C, B, H, N, kind)
        data_seed = 1000 * seed + case
        if kind == "tokens":
            S0 = la_inputs.decode_state(data_seed, B, H, d)
            q, k, v = la_inputs.qkv(data_seed, B, H, K, d, dtype=dt)
            tS = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(dev)
            o = la.decode_tokens(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), ts, tS)
            torch.cuda.synchronize()
            ro, rS = oracle_mod.fwd(q, k, v, s, S0)
            assert_close(to_host(o), ro, dt, tag + " K=%d o" % K)
            assert_close(to_host(tS), rS, dt, tag + " K=%d S" % K, stored_bf16=False)
            continue
        q, k, v = la_inputs.qkv(data_seed, B, H, N, d, dtype=dt)
        tq, tk, tv = (to_dev(x, dt) for x in (q, k, v))
        if kind == "fwd":
            S0 = la_inputs.decode_state(data_seed, B, H, d) if with_state else None
            tS0 = (None if S0 is None else
                   torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(dev))
            o, S = la.prefill(tq, tk, tv, ts, chunk=C, state_in=tS0)
            torch.cuda.synchronize()
            ro, rS = oracle_mod.fwd(q, k, v, s, S0)
            assert_close(to_host(o), ro, dt, tag + " o")
            assert_close(to_host(S), rS, dt, tag + " S", stored_bf16=False)
        else:
            g = la_inputs.upstream_grad(data_seed, B, H, N, d, dtype=dt)
            dq, dk, dv = la.prefill_bwd(tq, tk, tv, to_dev(g, dt), ts, chunk=C)
            torch.cuda.synchronize()
            rq, rk, rv = oracle_mod.bwd(q, k, v, g, s)
            assert_close(to_host(dq), rq, dt, tag + " dq")
            assert_close(to_host(dk), rk, dt, tag + " dk")
            assert_close(to_host(dv), rv, dt, tag + " dv")


@pytest.mark.parametrize("seed", [1, 2])
def test_random_packed_and_gated(oracle_mod, seed):
    """Packed batches (random cuts, empty and one-token sequences, initial
    states) forward and backward, and the gated prefill, on random shapes."""
    rng = random.Random(100 + seed)
    dev = device()
    for case in range(20):
        dt = rng.choice(["bf16", "bf16", "f32"])
        d = rng.choice([64, 128]) if dt == "bf16" else rng.choice([16, 32, 64, 128])
        C = rng.choice([16, 32, 64, 128])
        H = rng.choice([1, 2, 3, 8, 32])
        s = la_inputs.slopes(H).copy()
        if rng.random() < 0.3:
            s[0] = rng.choice([0.0, 1e4])
        ts = torch.from_numpy(s).to(dev)
        kind = rng.choice(["packed", "packed_bwd", "gated"])
        data_seed = 5000 + 100 * seed + case
        if kind != "gated":
            nseq = rng.randint(1, 12)
            lens = [rng.choice([0, 1, rng.randint(1, 300), rng.randint(1, 3000), C, 2 * C + 1])
                    for _ in range(nseq)]
            if sum(lens) == 0:
                lens[-1] = 5
            cu = [0] + np.cumsum(lens).tolist()
            T = cu[-1]
            q, k, v = (x[0] for x in la_inputs.qkv(data_seed, 1, H, T, d, dtype=dt))
            tq, tk, tv = (to_dev(x, dt) for x in (q, k, v))
            tag = "seed %d case %d: %s %s d=%d C=%d H=%d cu=%s" % (seed, case, kind, dt, d, C, H, cu)
            if kind == "packed":
                S0 = la_inputs.decode_state(data_seed, nseq, H, d) if rng.random() < 0.6 else None
                tS0 = (None if S0 is None else
                       torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(dev))
                o, S = la.prefill_varlen(tq, tk, tv, ts, cu, chunk=C, state_in=tS0)
                torch.cuda.synchronize()
                ro, rS = oracle_mod.fwd_varlen(q, k, v, s, cu, S0)
                assert_close(to_host(o), ro, dt, tag + " o")
                assert_close(to_host(S), rS, dt, tag + " S", stored_bf16=False)
            else:
                g = la_inputs.upstream_grad(data_seed, 1, H, T, d, dtype=dt)[0]
                dq, dk, dv = la.prefill_bwd_varlen(tq, tk, tv, to_dev(g, dt), ts, cu, chunk=C)
                torch.cuda.synchronize()
                rq, rk, rv = oracle_mod.bwd_varlen(q, k, v, g, s, cu)
                assert_close(to_host(dq), rq, dt, tag + " dq")
                assert_close(to_host(dk), rk, dt, tag + " dk")
                assert_close(to_host(dv), rv, dt, tag + " dv")
        else:
            B = rng.choice([1, 2])
            N = max(1, rng.choice([C, 64, 256, 1024]) * rng.randint(1, 4) + rng.choice([-1, 0, 5]))
            q, k, v = la_inputs.qkv(data_seed, B, H, N, d, dtype=dt)
            gt = la_inputs.gate(data_seed, B, H, N, d, dtype=dt)
            wn = la_inputs.norm_weight(data_seed, H, d)
            S0 = la_inputs.decode_state(data_seed, B, H, d) if rng.random() < 0.5 else None
            tS0 = (None if S0 is None else
                   torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(dev))
            y, S = la.prefill_gated(*(to_dev(x, dt) for x in (q, k, v)), ts, to_dev(gt, dt),
                                    torch.from_numpy(wn).to(dev), eps=1e-6, chunk=C, state_in=tS0)
            torch.cuda.synchronize()
            ry, rS = oracle_mod.fwd_gated(q, k, v, s, gt, wn, 1e-6, S0)
            tag = "seed %d case %d: gated %s d=%d C=%d B=%d H=%d N=%d" % (seed, case, dt, d, C, B, H, N)
            assert_close(to_host(y), ry, dt, tag + " y")
            assert_close(to_host(S), rS, dt, tag + " S", stored_bf16=False)
