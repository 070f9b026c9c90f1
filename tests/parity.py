"""Acceptance bars of the GPU parity tests (plain numpy: importable without a GPU).

The bars (page "[Not ready] MSCCLPP EP implementation #852" defines the
operations; the bars are the stated contract of this library):
  * layout, offsets, maps and dispatched bytes: bit-exact;
  * FP8 scales: bit-exact; FP8 codes: at most one code step apart (same sign,
    or either code a zero, and magnitude ordinals within 1).  A NaN code (0x7F
    or 0xFF) is never "one step" from a finite code: it matches only itself.
    Both sides divide x by the scale in IEEE fp32 and round to nearest even,
    so the codes are in fact identical, and every FP8 check here asserts that
    stronger property (assert_fp8_codes), reporting whether the one-step bar
    still holds when it fails;
  * combine: max relative error 8e-3 against the oracle (bf16 outputs), and,
    because both sides run the same fp32 fused multiply-add chain in slot
    order, bit-exact (assert_combine checks both).
"""
import numpy as np

COMBINE_RTOL = 8e-3
FP8_NAN_MAG = 0x7F


def f32(bits):
    """bf16 bit patterns (uint16) -> fp32 values."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def combine_rel_err(got_bits, ref_bits):
    """max |g - o| / max(|o|, 1e-6) over all outputs (bf16 bits in)."""
    g, r = f32(got_bits).astype(np.float64), f32(ref_bits).astype(np.float64)
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), 1e-6))) if r.size else 0.0


def fp8_ulp_ok(got, ref):
    """True iff every E4M3FN code pair is within one code step (see above)."""
    got = np.asarray(got).astype(np.int32)
    ref = np.asarray(ref).astype(np.int32)
    nan_g = (got & 0x7F) == FP8_NAN_MAG
    nan_r = (ref & 0x7F) == FP8_NAN_MAG
    any_nan = nan_g | nan_r
    same_sign = ((got ^ ref) & 0x80) == 0
    either_zero = ((got & 0x7F) == 0) | ((ref & 0x7F) == 0)
    close = np.abs((got & 0x7F) - (ref & 0x7F)) <= 1
    finite_ok = close & (same_sign | either_zero)
    return bool(np.all(np.where(any_nan, got == ref, finite_ok)))


def assert_fp8_codes(got, ref, what="fp8 codes"):
    """Codes identical (which implies the one-step bar)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = int(np.count_nonzero(got != ref))
        raise AssertionError(f"{what}: {bad} codes differ from the oracle "
                             f"(within one code step: {fp8_ulp_ok(got, ref)})")


def assert_combine(got_bits, ref_bits, what="combine"):
    """Within the 8e-3 bar, and bit-exact."""
    got_bits = np.asarray(got_bits)
    ref_bits = np.asarray(ref_bits)
    assert got_bits.shape == ref_bits.shape, (what, got_bits.shape, ref_bits.shape)
    err = combine_rel_err(got_bits, ref_bits)
    assert err <= COMBINE_RTOL, f"{what}: max relative error {err} > {COMBINE_RTOL}"
    if not np.array_equal(got_bits, ref_bits):
        bad = int(np.count_nonzero(got_bits != ref_bits))
        raise AssertionError(f"{what}: {bad} outputs differ in their bits "
                             f"(max relative error {err}, within the bar)")
