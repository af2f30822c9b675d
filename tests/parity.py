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
bf16 outputs must also agree bit for bit almost everywhere: the pages fix
the rounding points (the bf16-rounded normalised value with the weight
included, an fp32 rotation, one final rounding), so a correct kernel differs
from the oracle only where its fp32 arithmetic (reciprocal square root, sum
order, sincos) lands on the other side of a bf16 rounding boundary, about 4
in 100 000 elements for an fp32 emulation of the contract.  At most 0.1% of
the elements (plus 4, for small arrays) may differ in their bits.  A kernel
that skips the contract rounding agrees on about 69% of the elements, one
that rounds x * rrms before the weight on about 73%: both fail.
Exact: integer maps, copied rows, the residual stream and the bitwise
invariants.

With QKR_PARITY_REPORT set to a file name, every bf16 comparison appends
one JSON line with its statistics (maximum pair-relative and raw relative
error, bit-equal fraction, ulp histogram, NMSE) to that file.
"""
import json
import os

import numpy as np

F32_ATOL = 1e-5
BF16_RTOL = 1.6e-2
BF16_EQUAL_FLOOR = 0.999
BF16_EQUAL_SLACK = 4

# Name of the running test, set by tests/conftest.py (report lines carry it).
CURRENT_TEST = ""


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


def _bf16_bits(a):
    """bf16 bit patterns (as int32) of float32 values that lie on the bf16 grid."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    if (u & 0xFFFF).any():
        raise ValueError("values are not bf16")
    return (u >> 16).astype(np.int32)


def _bf16_ordinal(bits):
    """Position of each bf16 value on the number line (+0 and -0 both 0)."""
    mag = bits & 0x7FFF
    return np.where(bits & 0x8000, -mag, mag)


def bf16_stats(got, ref, rotary_dim=0, pairing="neox"):
    """Agreement of two bf16 arrays (as float32 values on the bf16 grid)."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    n = int(ref.size)
    if n == 0:
        return {"n": 0, "max_pair_rel": 0.0, "max_raw_rel": 0.0, "bit_equal": 1.0, "unequal": 0,
                "ulp_hist": {"0": 0, "1": 0, "2": 0, ">2": 0}, "nmse": 0.0}
    err = bf16_errors(got, ref, rotary_dim, pairing)
    gb, rb = _bf16_bits(got), _bf16_bits(ref)
    ulp = np.abs(_bf16_ordinal(gb) - _bf16_ordinal(rb))
    g64, r64 = got.astype(np.float64), ref.astype(np.float64)
    nz = r64 != 0
    raw = np.abs(g64[nz] - r64[nz]) / np.abs(r64[nz])
    den = float(np.sum(r64 * r64))
    unequal = int(np.count_nonzero(gb != rb))
    return {
        "n": n,
        "max_pair_rel": float(err.max()),
        "max_raw_rel": float(raw.max()) if raw.size else 0.0,
        "bit_equal": 1.0 - unequal / n,
        "unequal": unequal,
        "ulp_hist": {"0": int(np.count_nonzero(ulp == 0)), "1": int(np.count_nonzero(ulp == 1)),
                     "2": int(np.count_nonzero(ulp == 2)), ">2": int(np.count_nonzero(ulp > 2))},
        "nmse": float(np.sum((g64 - r64) ** 2) / den) if den > 0 else 0.0,
    }


def _report(what, stats):
    path = os.environ.get("QKR_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"test": CURRENT_TEST, "what": what, **stats}) + "\n")


def assert_bf16_close(got, ref, rotary_dim=0, pairing="neox", what="", floor=BF16_EQUAL_FLOOR):
    st = bf16_stats(got, ref, rotary_dim, pairing)
    _report(what, st)
    worst, equal = st["max_pair_rel"], st["bit_equal"]
    assert worst <= BF16_RTOL, f"{what}: max pair-relative error {worst:.3g} > {BF16_RTOL} (bit-equal {equal:.5f})"
    allowed = int((1.0 - floor) * st["n"]) + BF16_EQUAL_SLACK
    assert st["unequal"] <= allowed, (f"{what}: {st['unequal']} of {st['n']} bf16 elements differ in their bits "
                                      f"(bit-equal {equal:.5f}, at most {allowed} may differ)")
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
