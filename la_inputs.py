"""Seeded synthetic inputs for the Lightning Attention layer.

This module is shared by the tests, the benchmark and the smoke check. It holds
none of the method's arithmetic: it only draws random tensors, rounds them to
the storage precision and lists the per-head slopes that parameterise the decay.

Workload recipe (Ling & Ring 2.6 Technical Report pages, "Hybrid Linear
Attention" section, give no numbers for the operator; the shapes below are
synthetic stand-ins):
  * q, k, v ~ N(0, 1) / sqrt(d), drawn in fp32, then rounded to bf16
    (round-to-nearest-even) for the bf16 workloads;
  * upstream gradient dO ~ N(0, 1);
  * decode state S0 ~ N(0, 0.1^2) in fp32 (variance 0.01);
  * per-head slope s_h = 2^(-8 (h+1) / H), h = 0..H-1, so the decay is
    lambda_h = exp(-s_h);
  * packed (varlen) batches: sequence boundaries at nseq - 1 distinct cut
    points drawn uniformly over the packed tokens;
  * output epilogue: gate pre-activations ~ N(0, 1), RMSNorm weights
    1 + N(0, 0.1^2) per (head, channel), eps = 1e-6.

Each tensor draws from numpy.random.default_rng([seed, tensor_id, step]), so a
tensor never depends on the sizes of the tensors drawn before it.
"""
from __future__ import annotations

import numpy as np

# tensor ids for the seed sequence
Q_ID, K_ID, V_ID, DO_ID, S0_ID = 1, 2, 3, 4, 5
GATE_ID, NORMW_ID = 7, 8


def slopes(H: int) -> np.ndarray:
    """Per-head slope s_h = 2^(-8(h+1)/H) as fp32, h = 0..H-1 (0-based)."""
    h = np.arange(H, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / H).astype(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of fp32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(seed: int, tid: int, step: int, shape, scale: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, step])
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def qkv(seed: int, B: int, H: int, N: int, d: int, dtype: str = "bf16", step: int = 0):
    """q, k, v of shape [B,H,N,d] ~ N(0,1)/sqrt(d), as fp32 arrays holding `dtype` values."""
    out = []
    for tid in (Q_ID, K_ID, V_ID):
        x = _normal(seed, tid, step, (B, H, N, d), 1.0 / np.sqrt(d))
        out.append(bf16_round(x) if dtype == "bf16" else x)
    return tuple(out)


def upstream_grad(seed: int, B: int, H: int, N: int, d: int, dtype: str = "bf16"):
    """dO of shape [B,H,N,d] ~ N(0,1)."""
    x = _normal(seed, DO_ID, 0, (B, H, N, d), 1.0)
    return bf16_round(x) if dtype == "bf16" else x


def gate(seed: int, B: int, H: int, N: int, d: int, dtype: str = "bf16"):
    """Output-gate pre-activations of shape [B,H,N,d] ~ N(0,1)."""
    x = _normal(seed, GATE_ID, 0, (B, H, N, d), 1.0)
    return bf16_round(x) if dtype == "bf16" else x


def norm_weight(seed: int, H: int, d: int) -> np.ndarray:
    """Per-(head, channel) RMSNorm weights [H,d] fp32, 1 + N(0, 0.1^2)."""
    return (1.0 + _normal(seed, NORMW_ID, 0, (H, d), 0.1)).astype(np.float32)


def gate_device(seed: int, B: int, H: int, N: int, d: int, device, torch_dtype):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + GATE_ID)
    return torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32).to(torch_dtype)


def decode_state(seed: int, B: int, H: int, d: int) -> np.ndarray:
    """Decode state S0 of shape [B,H,d,d] in fp32, ~ N(0, 0.1^2)."""
    return _normal(seed, S0_ID, 0, (B, H, d, d), 0.1)


def qkv_device(seed: int, B: int, H: int, N: int, d: int, device, torch_dtype):
    """Large-workload variant drawn with torch's seeded generator on `device`.

    Same distributions as `qkv`; the values differ from the numpy stream, so a
    check against the oracle copies these exact tensors back to the host.
    """
    import torch

    g = torch.Generator(device=device)
    out = []
    for tid in (Q_ID, K_ID, V_ID):
        g.manual_seed(seed * 1000003 + tid)
        x = torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32)
        x.mul_(1.0 / float(np.sqrt(d)))
        out.append(x.to(torch_dtype))
    return tuple(out)


def upstream_grad_device(seed: int, B: int, H: int, N: int, d: int, device, torch_dtype):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + DO_ID)
    return torch.randn((B, H, N, d), generator=g, device=device, dtype=torch.float32).to(torch_dtype)


def packed_cu_seqlens(seed: int, nseq: int, T: int) -> list:
    """cu_seqlens of a packed batch: nseq - 1 distinct cut points drawn
    uniformly from 1 .. T-1, so lengths run from a few tokens to several
    times the mean T / nseq (a ragged mix of short and long sequences)."""
    rng = np.random.default_rng([seed, 6, 0])
    cuts = np.sort(rng.choice(np.arange(1, T), size=nseq - 1, replace=False))
    return [0] + [int(x) for x in cuts] + [int(T)]


# The five workloads (seed = config index, 0-based), and a packed-batch
# workload for the varlen path.
CONFIGS = {
    "tiny_f32": dict(seed=0, dtype="f32", B=1, H=2, N=256, d=64, C=64),
    "prefill_8k": dict(seed=1, dtype="bf16", B=1, H=32, N=8192, d=128, C=64),
    "prefill_128k": dict(seed=2, dtype="bf16", B=1, H=32, N=131072, d=128, C=128),
    "decode_b64": dict(seed=3, dtype="bf16", B=64, H=32, d=128, steps=1000),
    "train_32k": dict(seed=4, dtype="bf16", B=4, H=16, N=32768, d=128, C=64),
    "varlen_128k": dict(seed=5, dtype="bf16", nseq=64, H=32, T=131072, d=128, C=128),
}
