"""The bf16 tolerance rule of tests/parity.py, checked on the CPU.

The rule must accept a kernel that keeps the pages' rounding contract
([Ovis] kernel review: the normalised value, weight included, rounded to
bf16, an fp32 rotation, one final rounding) and reject two plausible
slips: a kernel that skips the contract rounding, and one that rounds
x * rrms to bf16 before multiplying by the weight (the order the [VecRMS]
review thread quotes from vLLM's RMSNorm kernel).  The candidates are built
here from oracle outputs and numpy float32 arithmetic.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import assert_bf16_close, bf16_stats


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _case(mode):
    case = W.imrope(tokens=192, seed_stream=17)
    x, w = W.as_f32(case.q), W.as_f32(case.q_weight)
    if mode == "imrope":
        rope = oracle.Rope("imrope", 128, "neox", inv_freq=case.inv_freq, sections=case.sections,
                           positions=case.positions)
        pos = case.positions[oracle.axis_map(rope, 64), :x.shape[0]].T          # [tokens, pairs]
    else:
        rope = oracle.Rope("1d", 128, "neox", inv_freq=case.inv_freq, positions=case.positions[:1])
        pos = np.repeat(case.positions[0, :x.shape[0], None], 64, axis=1)
    theta = (pos.astype(np.float32) * case.inv_freq[None, :]).astype(np.float32)
    return case, x, w, rope, theta


def _rotate(n, theta, dtype):
    """NeoX rotation of rows n [tokens, heads, 128] by theta [tokens, 64] in
    numpy float32 (separate products, no fused multiply-add) or float64."""
    c = np.cos(theta.astype(np.float64))[:, None, :].astype(dtype)
    s = np.sin(theta.astype(np.float64))[:, None, :].astype(dtype)
    a, b = n[..., :64].astype(dtype), n[..., 64:].astype(dtype)
    return _bf16(np.concatenate([a * c - b * s, b * c + a * s], -1))


@pytest.mark.parametrize("mode", ["1d", "imrope"])
def test_contract_kernel_passes_and_slips_fail(mode):
    case, x, w, rope, theta = _case(mode)
    ref = oracle.qk_norm_rope(x, w, case.eps, rope, "bf16")
    n_contract = oracle.qk_norm_rope(x, w, case.eps, None, "bf16")           # bf16(x * rrms * w)
    u = oracle.qk_norm_rope(x, w, case.eps, None, "f32")                     # fl32(x * rrms * w)
    xr = oracle.qk_norm_rope(x, np.ones_like(w), case.eps, None, "f32")      # fl32(x * rrms)

    good = _rotate(n_contract, theta, np.float32)
    assert_bf16_close(good, ref, 128, "neox", "fp32 rotation of the contract-rounded value")

    # An fp32 kernel end to end: fp32 sum of squares and reciprocal square
    # root, the contract rounding, fp32 trig and rotation.
    ss = (x * x).sum(-1, dtype=np.float32)
    rr = (1.0 / np.sqrt((ss / np.float32(128) + np.float32(case.eps)).astype(np.float64))).astype(np.float32)
    emu = _rotate(_bf16((x * rr[..., None]).astype(np.float32) * w), theta, np.float32)
    st = bf16_stats(emu, ref, 128, "neox")
    assert st["bit_equal"] > 0.9999, st
    assert_bf16_close(emu, ref, 128, "neox", "fp32 emulation")

    no_contract = _rotate(u, theta, np.float64)
    double_round = _rotate(_bf16(_bf16(xr) * w), theta, np.float64)
    for name, cand in (("no contract rounding", no_contract), ("x*rrms rounded before the weight", double_round)):
        st = bf16_stats(cand, ref, 128, "neox")
        assert st["max_pair_rel"] <= 1.6e-2, (name, st)      # the magnitude bound alone cannot see it
        assert st["bit_equal"] < 0.8, (name, st)
        with pytest.raises(AssertionError, match="differ in their bits"):
            assert_bf16_close(cand, ref, 128, "neox", name)


def test_stats_fields():
    rng = np.random.default_rng(5)
    ref = _bf16(rng.normal(0, 1, 4096))
    got = ref.copy()
    st = bf16_stats(got, ref)
    assert st["bit_equal"] == 1.0 and st["unequal"] == 0 and st["nmse"] == 0.0
    assert st["ulp_hist"] == {"0": 4096, "1": 0, "2": 0, ">2": 0}
    # one, two and three bf16 steps away
    bits = got.view(np.uint32)
    bits[10] += 1 << 16
    bits[20] += 2 << 16
    bits[25] += 3 << 16
    st = bf16_stats(got, ref)
    assert st["unequal"] == 3 and st["ulp_hist"] == {"0": 4093, "1": 1, "2": 1, ">2": 1}
    assert 0 < st["nmse"] < 1e-4 and st["max_raw_rel"] > 0
    bits[25] -= 3 << 16
    # the slack admits a handful of differences in a small array, no more
    assert_bf16_close(got, ref)
    for i in range(30, 60):
        bits[i] += 1 << 16
    with pytest.raises(AssertionError, match="differ in their bits"):
        assert_bf16_close(got, ref)
    # values off the bf16 grid are not bf16 outputs
    with pytest.raises(ValueError):
        bf16_stats(np.float32([1.0 + 2 ** -20]), np.float32([1.0]))
