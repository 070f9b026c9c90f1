"""The parity bars themselves (CPU only): a NaN code is never accepted for a
finite one, the one-step FP8 window is what the stated tolerance says, and the
combine check demands identical bits on top of the 8e-3 bar."""
import numpy as np
import pytest

from parity import assert_combine, assert_fp8_codes, combine_rel_err, fp8_ulp_ok


@pytest.mark.parametrize("got,ref", [(0x7F, 0x7E), (0x7E, 0x7F), (0xFF, 0xFE), (0xFE, 0xFF),
                                     (0x7F, 0xFF), (0xFF, 0x7F), (0x7F, 0x00), (0x80, 0xFF)])
def test_nan_code_never_matches_another_code(got, ref):
    assert not fp8_ulp_ok(np.uint8([got]), np.uint8([ref]))


@pytest.mark.parametrize("got,ref,ok", [
    (0x7F, 0x7F, True), (0xFF, 0xFF, True),        # NaN matches only itself
    (0x7E, 0x7D, True), (0x10, 0x11, True), (0x91, 0x90, True),
    (0x10, 0x12, False), (0x10, 0x90, False),      # two steps; opposite signs
    (0x00, 0x80, True), (0x01, 0x80, True),        # a zero of either sign
    (0x81, 0x00, True), (0x02, 0x80, False),
])
def test_one_step_window(got, ref, ok):
    assert fp8_ulp_ok(np.uint8([got]), np.uint8([ref])) is ok


def test_assert_fp8_codes_demands_identical_codes():
    a = np.uint8([0x10, 0x7E, 0x00])
    assert_fp8_codes(a, a.copy())
    with pytest.raises(AssertionError, match="within one code step: True"):
        assert_fp8_codes(np.uint8([0x10, 0x7D, 0x00]), a)
    with pytest.raises(AssertionError, match="within one code step: False"):
        assert_fp8_codes(np.uint8([0x10, 0x7F, 0x00]), a)


def test_combine_bar():
    one = np.uint16([0x3F80])                       # 1.0
    next_up = np.uint16([0x3F81])                   # 1 + 2^-7
    assert combine_rel_err(next_up, one) == pytest.approx(2.0 ** -7)
    assert_combine(one, one.copy())
    # 2^-7 = 7.8e-3 is inside the 8e-3 bar, but the bits differ: rejected
    with pytest.raises(AssertionError, match="differ in their bits"):
        assert_combine(next_up, one)
    # 1 + 2^-6 is outside the bar itself
    with pytest.raises(AssertionError, match="> 0.008"):
        assert_combine(np.uint16([0x3F82]), one)
