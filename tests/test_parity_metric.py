"""The parity metric of the GPU tests (tests/_gpu.py), on the CPU: it passes
what the stated bars pass and rejects what they reject.

Bars: fp32 max|got - ref| <= 1e-4 max|ref|; bf16 max|got - ref| <= 2e-2 rms(ref),
with the final rounding of a bf16-stored element (u |ref|, u = 2^-8) not
counted as error.
"""
import numpy as np
import pytest

from tests._gpu import BF16_TOL, BF16_U, F32_TOL, assert_close, err_ratio


def _bf16(x):
    """Round to bf16, nearest even, as the library stores its outputs."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _ref(seed, n=4096, outlier=11.0):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(n)
    r[7] = outlier * np.sqrt(np.mean(r * r))  # a large element, as fast and slow heads give
    return r


def test_exact_result_scores_zero():
    r = _ref(0)
    # with the allowance the element score is -u |ref|: at most 0
    assert err_ratio(r, r, "bf16") <= 0.0
    assert err_ratio(r, r, "bf16", stored_bf16=False) == 0.0
    assert err_ratio(r, r, "f32") == 0.0


def test_bf16_storage_rounding_passes_only_with_the_allowance():
    r = _ref(1, outlier=40.0)
    got = _bf16(r)
    assert err_ratio(got, r, "bf16") <= 0.0  # rounding is absorbed element by element
    # without the allowance the rounding of the large element alone is above the bar
    assert err_ratio(got, r, "bf16", stored_bf16=False) > 1.0


@pytest.mark.parametrize("stored", [True, False])
def test_bf16_bar_is_two_percent_of_the_rms(stored):
    r = _ref(2)
    rms = np.sqrt(np.mean(r * r))
    i = 100  # an ordinary element
    allowance = BF16_U * abs(r[i]) if stored else 0.0
    for f, ok in ((0.9, True), (1.1, False)):
        got = r.copy()
        got[i] += f * BF16_TOL * rms + allowance
        ratio = err_ratio(got, r, "bf16", stored_bf16=stored)
        assert (ratio <= 1.0) == ok, (f, ratio)
        if not ok:
            with pytest.raises(AssertionError):
                assert_close(got, r, "bf16", "perturbed", stored_bf16=stored)


def test_f32_bar_is_relative_to_the_largest_element():
    r = _ref(3)
    m = np.max(np.abs(r))
    for f, ok in ((0.9, True), (1.1, False)):
        got = r.copy()
        got[5] -= f * F32_TOL * m
        assert (err_ratio(got, r, "f32") <= 1.0) == ok


def test_rejects_non_finite_and_mismatched_shapes():
    r = _ref(4)
    bad = r.copy()
    bad[3] = np.nan
    with pytest.raises(AssertionError):
        err_ratio(bad, r, "bf16")
    bad[3] = np.inf
    with pytest.raises(AssertionError):
        err_ratio(bad, r, "f32")
    with pytest.raises(AssertionError):
        err_ratio(r[:-1], r, "bf16")


def test_empty_tensors_pass():
    e = np.zeros((0, 4))
    assert err_ratio(e, e, "bf16") == 0.0 and err_ratio(e, e, "f32") == 0.0
