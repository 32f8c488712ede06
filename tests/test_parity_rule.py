"""The comparison rule of tests/_parity.py, checked on the CPU with hand-made values:
the bf16 output-floor exception applies only where half a bf16 ulp exceeds the bar,
and only to the two bf16 values that bracket the exact result."""

import numpy as np
import pytest

from _parity import bf16_bracket, bf16_rne, check_bf16, check_f32

L1 = np.zeros(1)


def test_bracket_values():
    lo, hi, sp = bf16_bracket(np.array([4.0131, -4.0131, 4.0, 0.3, -2.5, 7.99999]))
    assert lo.tolist() == [4.0, -4.03125, 4.0, 0.298828125, -2.5, 7.96875]
    assert hi.tolist() == [4.03125, -4.0, 4.03125, 0.30078125, -2.484375, 8.0]
    assert sp.tolist() == [2**-5, 2**-5, 2**-5, 2**-9, 2**-6, 2**-5]


def test_correct_rounding_and_other_neighbour_pass_where_the_format_is_coarser_than_the_bar():
    ref = np.array([[4.0131, 4.0157, 1.0]])
    out = bf16_rne(ref)                      # 4.0, 4.03125, 1.0: errors 0.0131 and 0.0156
    check_bf16(out, L1, ref, L1, "correctly rounded")
    other = out.copy()
    other[0, 1] = 4.0                        # the lower bracketing bf16 of 4.0157: error 0.0157
    check_bf16(other, L1, ref, L1, "other neighbour")


@pytest.mark.parametrize("bad", [
    (0, 0, 4.0625),      # two ulps away at |O| ~ 4
    (0, 2, 1.0117),      # above the bar where half an ulp (2^-9) is far below it
    (0, 3, -2.515625),   # a bracketing value at |O| in [2, 4), but above the bar: half an ulp is 0.0078
])
def test_other_errors_above_the_bar_fail(bad):
    ref = np.array([[4.0131, 4.0157, 1.0, -2.5039]])
    out = bf16_rne(ref)
    r, c, v = bad
    out[r, c] = v
    with pytest.raises(AssertionError):
        check_bf16(out, L1, ref, L1, "planted error")


def test_l_bar_and_empty_rows():
    O = np.zeros((2, 3))
    check_bf16(O, np.array([0.5, -np.inf]), O, np.array([0.5005, -np.inf]), "L within 1e-3")
    with pytest.raises(AssertionError):
        check_bf16(O, np.array([0.5, -np.inf]), O, np.array([0.502, -np.inf]), "L off by 2e-3")
    with pytest.raises(AssertionError):
        check_bf16(O, np.array([0.5, 0.0]), O, np.array([0.5, -np.inf]), "empty row must have L = -inf")


def test_fp32_bar_has_no_floor_rule():
    ref = np.array([[4.0131]])
    with pytest.raises(AssertionError):
        check_f32(ref + 2e-4, L1, ref, L1, "fp32")
    check_f32(ref + 5e-5, L1, ref, L1, "fp32")
