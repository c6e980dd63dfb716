"""Shared helpers of the GPU parity tests: device transfer and the tolerances.

Tolerances (the per-tensor bars; see the design doc for their derivation):
  * fp32 inputs: max|got - ref| / max|ref| <= 1e-4 (normwise relative error);
  * bf16 inputs: max|got - ref| <= 2e-2 * rms(ref), rms over the whole tensor.
"""
import numpy as np
import torch

F32_TOL = 1e-4
BF16_TOL = 2e-2


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device())


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_ratio(got, ref, dtype: str) -> float:
    """Error over the tensor's bar; <= 1 passes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite values"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    if dtype == "bf16":
        rms = np.sqrt(np.mean(ref * ref)) if ref.size else 1.0
        return err / (BF16_TOL * max(rms, 1e-30))
    return err / (F32_TOL * max(np.max(np.abs(ref)), 1e-30))


def assert_close(got, ref, dtype: str, what: str = ""):
    r = err_ratio(got, ref, dtype)
    assert r <= 1.0, "%s: error is %.3g of the %s bar" % (what, r, dtype)
    return r
