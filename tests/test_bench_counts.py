"""The benchmark's algorithmic and issued work counts (CPU).

* The algorithmic bytes and flops of a forward pass follow the per-token
  costs 4 d 2 bytes (q, k, v read, o written, bf16) and 2(C+1)d + 4d^2 flops,
  plus the final fp32 state.
* The issued matrix-core work of the bf16 kernel (causal 16x16 score tiles,
  hi + lo passes for P.V, S.Q and K^T.(bV)) agrees with the SQ_INSTS_MFMA
  counter per wave and chunk in the committed SQ-counter profiles, for the
  128K workload (128-token chunks) and the training forward (64-token chunks).
"""
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MFMA_FLOPS = 16 * 16 * 32 * 2  # one v_mfma_f32_16x16x32_bf16


def test_prefill_128k_algorithmic_counts():
    B, H, N, d, C = 1, 32, 131072, 128, 128
    nbytes, flops = bench.prefill_counts(B, H, N, d, C)
    assert nbytes == 4 * B * H * N * d * 2 + B * H * d * d * 4 == 4_297_064_448
    assert flops == B * H * N * (2 * (C + 1) * d + 4 * d * d)
    assert flops == pytest.approx(4.13e11, rel=2e-3)
    # arithmetic intensity of the pass: about 96 flop per byte
    assert flops / nbytes == pytest.approx(96.2, abs=0.05)


def test_prefill_8k_algorithmic_counts():
    nbytes, flops = bench.prefill_counts(1, 32, 8192, 128, 64)
    assert nbytes == 270_532_608
    assert flops == pytest.approx(2.15e10, rel=3e-3)


def _sq_mfma_per_wave_chunk(profile, section):
    text = open(os.path.join(ROOT, "profiles", profile)).read()
    part = text.split("## " + section, 1)[1]
    m = re.search(r"^\| SQ_INSTS_MFMA \| [^|]+ \| ([0-9.]+) \|", part, re.M)
    return float(m.group(1))


@pytest.mark.parametrize("profile,section,shape", [
    ("prefill_128k_sq_counters.md", "main kernel", (1, 32, 131072, 128, 128)),
    ("train_32k_sq_counters.md", "forward / dq pass", (4, 16, 32768, 128, 64)),
])
def test_issued_mfma_matches_the_counter(profile, section, shape):
    B, H, N, d, C = shape
    waves = d // 32  # per workgroup, one per 32 value columns
    chunks = B * H * (N // C)
    per_wave_chunk = bench.prefill_mfma_executed(B, H, N, d, C) / (chunks * waves * MFMA_FLOPS)
    assert per_wave_chunk == _sq_mfma_per_wave_chunk(profile, section)


def test_issued_over_algorithmic_at_128k():
    B, H, N, d, C = 1, 32, 131072, 128, 128
    _, flops = bench.prefill_counts(B, H, N, d, C)
    assert bench.prefill_mfma_executed(B, H, N, d, C) / flops == pytest.approx(1.93, abs=0.01)
