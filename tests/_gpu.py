"""Shared helpers of the GPU parity tests: device transfer and the tolerances.

Tolerances, per tensor:
  * fp32 inputs: max|got - ref| / max|ref| <= 1e-4 (normwise relative error);
  * bf16 inputs: max|got - ref| <= 2e-2 * rms(ref), rms over the whole tensor.
    For tensors the library stores in bf16 (o, dq, dk, dv) the final
    round-to-nearest of each element to bf16 is not counted as error: the
    element test is |got - ref| - u |ref| <= 2e-2 * rms(ref) with u = 2^-8, the
    bf16 unit roundoff.  Without that allowance the exact result itself, once
    stored in bf16, fails the bar whenever max|ref| > 5.12 rms(ref), which the
    mix of fast and slow heads produces (max/rms is about 11 at H = 32).
    fp32 tensors (the state S) get no allowance.
"""
import os
import re

import numpy as np
import torch

F32_TOL = 1e-4
BF16_TOL = 2e-2
BF16_U = 2.0**-8


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device())


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_ratio(got, ref, dtype: str, stored_bf16: bool = None) -> float:
    """Worst element error over the tensor's bar; <= 1 passes.

    stored_bf16 defaults to (dtype == "bf16") and should be False for fp32
    outputs of the bf16 path (the state)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite values"
    if got.size == 0:
        return 0.0
    if stored_bf16 is None:
        stored_bf16 = dtype == "bf16"
    if dtype == "bf16":
        rms = max(np.sqrt(np.mean(ref * ref)), 1e-30)
        err = np.abs(got - ref)
        if stored_bf16:
            err = err - BF16_U * np.abs(ref)
        return float(np.max(err)) / (BF16_TOL * rms)
    return float(np.max(np.abs(got - ref))) / (F32_TOL * max(np.max(np.abs(ref)), 1e-30))


# Worst ratio seen per (test, tensor): with the bar as tested, and for bf16
# tensors stored in bf16 also without the rounding allowance.  conftest.py
# writes them out at the end of the session when LA_MARGINS_OUT names a file.
MARGINS = {}


def _record(what, got, ref, dtype, stored_bf16, r):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    # one entry per check kind: the head or row a check covers is dropped
    key = "%s :: %s" % (test, re.sub(r" (head \d+|\(b=\d+,h=\d+\))$", "", what))
    m = MARGINS.setdefault(key, {"ratio": 0.0, "ratio_no_allowance": 0.0, "checks": 0})
    m["ratio"] = max(m["ratio"], r)
    m["checks"] += 1
    if dtype == "bf16" and (stored_bf16 is None or stored_bf16):
        raw = err_ratio(got, ref, dtype, stored_bf16=False)
    else:
        raw = r
    m["ratio_no_allowance"] = max(m["ratio_no_allowance"], raw)


def assert_close(got, ref, dtype: str, what: str = "", stored_bf16: bool = None):
    r = err_ratio(got, ref, dtype, stored_bf16)
    _record(what, got, ref, dtype, stored_bf16, r)
    assert r <= 1.0, "%s: error is %.3g of the %s bar" % (what, r, dtype)
    return r
