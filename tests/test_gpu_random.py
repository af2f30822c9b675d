"""Seeded random sweep of the QK RMSNorm + RoPE path against the oracle.

Each case draws a dtype, head_dim, rotary_dim, pairing and position mode
(1-D, t/h/w axes, IMROPE sections or precomputed cos/sin planes), a batch, a
token count, Q and K head counts (one of them possibly absent), a token offset
into longer position planes, strided head views carved from a wider buffer and
sometimes in-place outputs, then compares every output element with the
oracle under the same tolerances as the other parity tests.  Each case prints
its parameters before it runs.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_qk_rmsnorm_amd as qkr
import workloads as W
from parity import assert_bf16_close, assert_f32_close

pytestmark = pytest.mark.gpu

N_CASES = 480
DEV = "cuda"
HEAD_DIMS = (8, 16, 24, 32, 40, 48, 64, 72, 80, 96, 120, 128, 136, 160, 192, 200, 256)


def split(rng, total, parts):
    """`parts` non-negative ints summing to `total`."""
    cuts = np.sort(rng.integers(0, total + 1, parts - 1))
    return [int(x) for x in np.diff(np.concatenate([[0], cuts, [total]]))]


def draw(i):
    rng = np.random.default_rng([W.SEED, 4711, i])
    c = {"dtype": str(rng.choice(["bf16", "f32"]))}
    ve = 8 if c["dtype"] == "bf16" else 4
    c["d"] = int(rng.choice([h for h in HEAD_DIMS if h % ve == 0]))
    c["pairing"] = str(rng.choice(["neox", "adjacent"]))
    step = 2 * ve if c["pairing"] == "neox" else 2          # NeoX halves are whole 16-byte vectors
    r_choices = [r for r in range(0, c["d"] + 1, step)]
    full = c["d"] if c["d"] % step == 0 else r_choices[-1]
    c["rot"] = full if rng.random() < 0.5 else int(rng.choice(r_choices))
    c["mode"] = str(rng.choice(["1d", "axes", "imrope", "planes"])) if c["rot"] else "1d"
    half = c["rot"] // 2
    if c["mode"] in ("axes", "planes"):
        c["sections"] = tuple(split(rng, half, 3)) + (0,)
    elif c["mode"] == "imrope":
        total = int(rng.integers(half, 2 * half + 1))
        c["sections"] = tuple(split(rng, total, 4))
    else:
        c["sections"] = (0, 0, 0, 0)
    c["batch"] = int(rng.integers(1, 4))
    c["tokens"] = int(rng.integers(1, 160))
    c["hq"] = int(rng.integers(0, 14))
    c["hk"] = int(rng.integers(0 if c["hq"] else 1, 14))
    c["token_base"] = int(rng.integers(0, 40))
    c["pad_heads"] = int(rng.integers(0, 3))
    c["in_place"] = bool(rng.random() < 0.25)
    c["theta"] = float(rng.choice([1e4, 1e6]))
    c["scale"] = float(rng.choice([1e-3, 1.0, 37.0]))
    return c


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = draw(i)
    print(f"case {i}: {c}", flush=True)
    rng = np.random.default_rng([W.SEED, 4712, i])
    d, rot, half, dtype = c["d"], c["rot"], c["rot"] // 2, c["dtype"]
    b, t, hq, hk = c["batch"], c["tokens"], c["hq"], c["hk"]
    length = c["token_base"] + t + int(rng.integers(0, 9))

    # Q and K as head slices of one wider buffer (strided views).
    width = hq + hk + c["pad_heads"]
    big = W.to_dtype(rng.normal(0, c["scale"], (b, t, width, d)).astype(np.float32), dtype)
    wq = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
    wk = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
    q_sl = slice(0, hq)
    k_sl = slice(hq + c["pad_heads"], hq + c["pad_heads"] + hk)

    orope, rope = None, None
    if rot:
        if c["mode"] == "planes":
            ang = rng.uniform(-40.0, 40.0, (3, length, half))
            cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
            orope = oracle.Rope("planes", rot, c["pairing"], sections=c["sections"], cos_planes=cos,
                                sin_planes=sin, token_base=c["token_base"])
            rope = qkr.Rope("planes", rot, c["pairing"], sections=c["sections"], token_base=c["token_base"],
                            cos_planes=torch.from_numpy(cos).to(DEV), sin_planes=torch.from_numpy(sin).to(DEV))
        else:
            planes = {"1d": 1, "axes": 3, "imrope": 4}[c["mode"]]
            pos = rng.integers(0, 8192, (planes, length)).astype(np.int32)
            inv = W.inv_freq_ladder(c["theta"], rot)
            orope = oracle.Rope(c["mode"], rot, c["pairing"], inv_freq=inv, sections=c["sections"], positions=pos,
                                token_base=c["token_base"])
            rope = qkr.Rope(c["mode"], rot, c["pairing"], inv_freq=torch.from_numpy(inv).to(DEV),
                            positions=torch.from_numpy(pos).to(DEV), sections=c["sections"],
                            token_base=c["token_base"])

    # Rows whose vector pairs take 3, 5, 6 or 7 lanes, with the token's Q and
    # K rows within 320 vectors, run on token tiles by default unless cos/sin
    # come from planes; such cases also run on the other kernel, forced.
    nv = d // (8 if dtype == "bf16" else 4)
    lanes = (nv + 1) // 2
    shape_ok = lanes in (3, 5, 6, 7) and (hq + hk) * nv <= 320
    token = shape_ok and c["mode"] != "planes"
    for variant in [None] + (["rope:tile"] if token else ["rope:token"] if shape_ok else []):
        gbig = big.to(DEV)
        q = gbig[:, :, q_sl] if hq else None
        k = gbig[:, :, k_sl] if hk else None
        kw = {}
        if c["in_place"]:
            kw = {"q_out": q, "k_out": k}
        qkr.set_variant_override(variant)
        try:
            qo, ko = qkr.qk_norm_rope(q, k, wq.to(DEV) if hq else None, wk.to(DEV) if hk else None, W.EPS, rope,
                                      **kw)
            chosen = qkr.last_variant()
        finally:
            qkr.set_variant_override(None)
        torch.cuda.synchronize()
        on_token = variant == "rope:token" or (variant is None and token)
        assert chosen.startswith("rope:token:" if on_token else "rope:np"), chosen

        for name, out, sl, w, heads in (("q", qo, q_sl, wq, hq), ("k", ko, k_sl, wk, hk)):
            if not heads:
                assert out is None
                continue
            got = out.detach().float().cpu().numpy()
            for bi in range(b):
                ref = oracle.qk_norm_rope(W.as_f32(big[bi, :, sl]), W.as_f32(w), W.EPS, orope, dtype)
                what = f"case {i} {name} batch {bi} {chosen}"
                if dtype == "f32":
                    assert_f32_close(got[bi], ref, what)
                else:
                    assert_bf16_close(got[bi], ref, rot, c["pairing"], what)
        # In place, the heads between the two slices stay as they were.
        if c["pad_heads"] and c["in_place"]:
            assert torch.equal(gbig[:, :, hq:hq + c["pad_heads"]].cpu(), big[:, :, hq:hq + c["pad_heads"]])
