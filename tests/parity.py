"""Tolerance rules shared by the GPU parity tests.

fp32 outputs: max |g - r| <= 1e-5.

bf16 outputs: max relative error <= 1.6e-2 (two bf16 steps), where the error
of an element is measured against the magnitude it belongs to:
  - un-rotated elements (plain norm outputs, dims past rotary_dim): |r|;
  - rotated elements: the norm of the reference pair (r_i, r_j), which the
    rotation preserves.  o_i = n_i c - n_j s can cancel to ~0, and a one-step
    difference in the bf16-rounded normalised value n (any last-bit
    difference in rrms can cause one) then makes |g - r| / |r| unbounded even
    for a correct kernel.
FP8 E4M3 codes: both sides decide the code in fp32 from y / scale; the
kernel's y differs from the oracle's in the last fp32 bits (fp32 rsqrt and
rounding order against a double reference), so a code may differ by one step
where the quotient sits at a rounding boundary, and nowhere else: every code
equal or adjacent in sign-magnitude order (+0 and -0 equal), and at least
99.9% of them equal.
Exact: integer maps, copied rows, the residual stream and the bitwise
invariants.
"""
import numpy as np

F32_ATOL = 1e-5
BF16_RTOL = 1.6e-2


def pair_index(d, rotary_dim, pairing):
    """Partner index of every element of a head_dim row (itself if unrotated)."""
    idx = np.arange(d)
    half = rotary_dim // 2
    if pairing == "neox":
        p = np.arange(half)
        idx[p], idx[p + half] = p + half, p
    else:
        p = np.arange(half)
        idx[2 * p], idx[2 * p + 1] = 2 * p + 1, 2 * p
    return idx


def bf16_errors(got, ref, rotary_dim=0, pairing="neox"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = ref.shape[-1]
    partner = pair_index(d, rotary_dim, pairing)
    rotated = np.zeros(d, bool)
    rotated[:rotary_dim] = True
    mag = np.where(rotated, np.hypot(ref, ref[..., partner]), np.abs(ref))
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(mag > 0, diff / mag, np.where(diff == 0, 0.0, np.inf))
    return err


def assert_bf16_close(got, ref, rotary_dim=0, pairing="neox", what=""):
    err = bf16_errors(got, ref, rotary_dim, pairing)
    worst = float(err.max()) if err.size else 0.0
    equal = float(np.mean(np.asarray(got) == np.asarray(ref))) if err.size else 1.0
    assert worst <= BF16_RTOL, f"{what}: max pair-relative error {worst:.3g} > {BF16_RTOL} (bit-equal {equal:.4f})"
    return worst, equal


def assert_f32_close(got, ref, what=""):
    diff = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    worst = float(diff.max()) if diff.size else 0.0
    assert worst <= F32_ATOL, f"{what}: max abs error {worst:.3g} > {F32_ATOL}"
    return worst


FP8_EQUAL_FRACTION = 0.999


def _fp8_ordinal(codes):
    c = np.asarray(codes, np.int32)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)      # +0 and -0 both map to 0


def assert_fp8_close(got, ref, what=""):
    got, ref = np.asarray(got, np.uint8), np.asarray(ref, np.uint8)
    step = np.abs(_fp8_ordinal(got) - _fp8_ordinal(ref))
    equal = float(np.mean(step == 0)) if step.size else 1.0
    assert (step <= 1).all(), f"{what}: FP8 codes {int(step.max())} steps apart"
    assert equal >= FP8_EQUAL_FRACTION, f"{what}: only {equal:.5f} of FP8 codes equal"
    return equal
