"""The parity rules themselves, on the CPU: the bf16 ulp is the spacing of bf16 values in the
binade of the reference (8 significant bits), floored at the subnormal step, so "within one ulp"
admits exactly the neighbouring bf16 values and nothing further."""
import numpy as np
import pytest

import acceptance as acc


def test_bf16_ulp_values():
    r = np.array([1.0, 1.5, 1.9921875, 0.99609375, 2.0, 3.0, -1.0, 2.0 ** -126, 2.0 ** -130, 0.0, 3.0e38])
    want = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -8, 2.0 ** -6, 2.0 ** -6, 2.0 ** -7, 2.0 ** -133,
                     2.0 ** -133, 2.0 ** -133, 2.0 ** 120])
    np.testing.assert_array_equal(acc.bf16_ulp(r), want)


def test_bf16_ulp_is_the_spacing_of_bf16_values():
    """For random bf16 values, the next bf16 value up (bit pattern + 1) lies exactly one ulp away."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0x0080, 0x7F00, size=2000, dtype=np.uint32)  # positive normal bf16 patterns
    v = (bits << 16).view(np.float32).astype(np.float64)
    nxt = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(nxt - v, acc.bf16_ulp(v))


def test_bf16_output_check_admits_one_ulp_only():
    y_ref = np.array([[1.0, 1.5, -3.0, 0.0]])
    one_up = y_ref + acc.bf16_ulp(acc.bf16_round(y_ref))
    acc.check_outputs(one_up, y_ref, True, "one ulp")
    two_up = y_ref + 2 * acc.bf16_ulp(acc.bf16_round(y_ref))
    with pytest.raises(AssertionError):
        acc.check_outputs(two_up, y_ref, True, "two ulps")
    # Just above a power of two the binade's ulp is the larger one; 1.5 ulps in the upper binade fail.
    with pytest.raises(AssertionError):
        acc.check_outputs(np.array([[1.0 + 1.5 * 2.0 ** -7]]), np.array([[1.0]]), True, "1.5 ulp")
