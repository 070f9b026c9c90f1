"""The expert -> rank division of the kernels (rank_of in csrc/ep_ids.h): a
multiply-high by magic = ceil(2^32 / epr), with magic 0 meaning epr == 1.  Its
exactness is integer arithmetic, so it is checked here exhaustively over every
experts-per-rank count and expert id the ABI admits (E <= EP_MAX_EXPERTS =
2048); the GPU parity tests cover the kernels that use it."""
import numpy as np

MAX_EXPERTS = 2048


def rank_magic(epr: int) -> int:
    return 0 if epr <= 1 else ((1 << 32) + epr - 1) // epr


def test_magic_fits_32_bits():
    assert rank_magic(1) == 0
    assert rank_magic(2) == 1 << 31
    assert all(0 < rank_magic(d) < (1 << 32) for d in range(2, MAX_EXPERTS + 1))


def test_multiply_high_equals_division_for_every_id_and_divisor():
    e = np.arange(MAX_EXPERTS, dtype=np.uint64)
    for epr in range(1, MAX_EXPERTS + 1):
        m = rank_magic(epr)
        got = e if m == 0 else (e * np.uint64(m)) >> np.uint64(32)
        np.testing.assert_array_equal(got, e // np.uint64(epr), err_msg=f"epr={epr}")


def test_a_truncated_magic_would_be_caught():
    # floor(2^32 / epr) instead of the ceiling is off by one somewhere for
    # every epr that does not divide 2^32 (epr = 3: e = 3 gives 0, not 1)
    e = np.arange(MAX_EXPERTS, dtype=np.uint64)
    m = (1 << 32) // 3
    assert np.any(((e * np.uint64(m)) >> np.uint64(32)) != e // np.uint64(3))
