"""The acceptance gate's bf16 half-ulp, checked against the bf16 number line
itself (every normal bf16 value), and the gate's 2e-2 floor."""
import numpy as np

import oracle
from gpu_util import ABS_TOL, gate, half_ulp_bf16


def _all_positive_normal_bf16():
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint16)  # smallest normal .. largest finite
    return bits, oracle.bits_to_f64(bits)


def test_half_ulp_is_half_the_spacing_above_every_bf16_value():
    bits, x = _all_positive_normal_bf16()
    nxt = oracle.bits_to_f64((bits[:-1] + 1).astype(np.uint16))
    spacing = nxt - x[:-1]
    np.testing.assert_array_equal(half_ulp_bf16(x[:-1]), spacing / 2)
    np.testing.assert_array_equal(half_ulp_bf16(-x[:-1]), spacing / 2)


def test_one_rounding_step_stays_within_half_ulp():
    # fp32 values (as the kernels hold before their one bf16 rounding): a
    # single round-to-nearest step, error at most the half-ulp
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))
    x = x.astype(np.float32).astype(np.float64)
    r = oracle.bits_to_f64(oracle.f64_to_bf16_bits(x))
    assert np.all(np.abs(r - x) <= half_ulp_bf16(x))


def test_gate_is_the_absolute_bound_below_8():
    x = np.array([0.0, 1e-30, 0.5, 1.0, 5.12, 5.9, 7.99, -7.99])
    np.testing.assert_array_equal(gate(x), ABS_TOL)
    assert gate(np.array([8.0]))[0] == 1.01 * 2.0 ** -5
    assert gate(np.array([-12.0]))[0] == 1.01 * 2.0 ** -5
    assert gate(np.array([16.0]))[0] == 1.01 * 2.0 ** -4
