"""CPU checks of the comparison rule itself (on synthetic data, no GPU)."""
import numpy as np
import pytest

import oracle
import parity


def test_ulp16_values():
    assert parity.ulp16(1.0) == 2.0 ** -10
    assert parity.ulp16(1.5) == 2.0 ** -10
    assert parity.ulp16(2.0) == 2.0 ** -9
    assert parity.ulp16(-1000.0) == 0.5
    assert parity.ulp16(2.0 ** -14) == 2.0 ** -24
    assert parity.ulp16(1e-6) == 2.0 ** -24
    assert parity.ulp16(0.0) == 2.0 ** -24


def test_rule_accepts_rounded_reference_and_rejects_large_errors():
    rng = np.random.default_rng(0)
    cref = rng.standard_normal((8, 8))
    K = 100
    parity.check(oracle.output_typed(cref, "f16"), cref, K, "f16", False)
    parity.check(oracle.output_typed(cref, "f32"), cref, K, "f32", False)
    bad = oracle.output_typed(cref, "f32").copy()
    bad[3, 4] += np.float32(0.02)            # > 1e-3 * sqrt(100) = 0.01
    with pytest.raises(AssertionError):
        parity.check(bad, cref, K, "f32", False)


def test_integer_rule_is_bit_exact_and_ignores_zero_sign():
    cref = np.array([[3.0, 0.0, -5.0, 2049.0]])
    got = oracle.output_typed(cref, "f16").copy()
    got[0, 1] = 0x8000                        # -0
    parity.check(got, cref, 1, "f16", True)
    got[0, 3] = np.float16(2050.0).view(np.uint16)   # off by one fp16 ulp
    with pytest.raises(AssertionError):
        parity.check(got, cref, 1, "f16", True)
