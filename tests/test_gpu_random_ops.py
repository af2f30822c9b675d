"""Seeded random sweeps of the row RMSNorm (plain, residual add, FP8 output),
the joint text/image op, the KV-cache write and the ViT entry points (fused
norm + rotation from patch grids, and the cos/sin setup) against the oracle.

Every case prints its parameters before it runs.  Residual streams, copied V
rows and untouched cache rows are compared bit for bit; normalised outputs
under the tolerances of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_qk_rmsnorm_amd as qkr
import workloads as W
from parity import assert_bf16_close, assert_f32_close, assert_fp8_close

pytestmark = pytest.mark.gpu

DEV = "cuda"
HEAD_DIMS = (16, 32, 48, 64, 80, 96, 128, 160, 256)


def check(got, ref, dtype, rotary_dim=0, pairing="neox", what=""):
    if dtype == "f32":
        return assert_f32_close(got, ref, what)
    return assert_bf16_close(got, ref, rotary_dim, pairing, what)


def host(t):
    return t.detach().float().cpu().numpy()


def split(rng, total, parts):
    cuts = np.sort(rng.integers(0, total + 1, parts - 1))
    return [int(x) for x in np.diff(np.concatenate([[0], cuts, [total]]))]


# ---------------------------------------------------------------- rows -----

def draw_rows(i):
    rng = np.random.default_rng([W.SEED, 5101, i])
    c = {"dtype": str(rng.choice(["bf16", "f32"]))}
    ve = 8 if c["dtype"] == "bf16" else 4
    max_vec = 4096
    nvec = int(np.clip(np.exp(rng.uniform(0, np.log(max_vec))), 1, max_vec))
    c["width"] = nvec * ve
    c["rows"] = int(rng.choice([1, 2, 3, 7, 31, 64, 300, 777, 2100]))
    c["add"] = bool(rng.random() < 0.6)
    c["fp8"] = bool(rng.random() < 0.4)
    c["variant"] = rng.choice([None, "rms:rows", "rms:wide", "rms:split"])
    c["res_out"] = str(rng.choice(["residual", "x", "separate"])) if c["add"] else "none"
    c["pad"] = int(rng.choice([0, 0, ve, 4 * ve]))          # extra elements per input row
    c["scale"] = float(rng.choice([0.005, 0.02, 0.3, 1.7]))
    c["mag"] = float(rng.choice([1e-2, 1.0, 50.0]))
    return c


@pytest.mark.parametrize("i", range(160))
def test_random_rows(i):
    c = draw_rows(i)
    print(f"rows case {i}: {c}", flush=True)
    rng = np.random.default_rng([W.SEED, 5102, i])
    dtype, rows, width, pad = c["dtype"], c["rows"], c["width"], c["pad"]
    xb = W.to_dtype(rng.normal(0, c["mag"], (rows, width + pad)).astype(np.float32), dtype)
    rb = W.to_dtype(rng.normal(0, c["mag"], (rows, width + pad)).astype(np.float32), dtype)
    w = W.to_dtype(rng.normal(1, 0.1, width).astype(np.float32), dtype)
    gx, gr = xb.to(DEV), rb.to(DEV)
    x, r = gx[:, :width], gr[:, :width]
    scale = torch.tensor([c["scale"]], dtype=torch.float32, device=DEV)
    x_in, r_in = W.as_f32(xb[:, :width]), W.as_f32(rb[:, :width])

    nvec = width // (8 if dtype == "bf16" else 4)
    variant = c["variant"]
    # A forced variant that cannot run the call is refused, never swapped:
    # one wavefront holds at most 1024 vectors, and the split rows cannot
    # take the residual add.
    runs = variant in (None, "rms:wide") or (nvec <= 1024 and not (variant == "rms:split" and c["add"]))

    def call():
        if not c["add"] and not c["fp8"]:
            return qkr.rms_norm(x, w.to(DEV), W.EPS), None
        res_out = None
        if c["res_out"] == "x":
            res_out = x
        elif c["res_out"] == "separate":
            res_out = torch.empty((rows, width), dtype=x.dtype, device=DEV)
        return qkr.add_rms_norm(x, w.to(DEV), W.EPS, residual=r if c["add"] else None, residual_out=res_out,
                                out_dtype="fp8_e4m3" if c["fp8"] else None, scale=scale)

    qkr.set_variant_override(variant)
    try:
        if not runs:
            with pytest.raises(qkr.QkrError, match="forced variant"):
                call()
            qkr.set_variant_override(None)
        y, s = call()
        if runs and variant is not None:
            assert qkr.last_variant().startswith(variant + ":"), qkr.last_variant()
        torch.cuda.synchronize()
    finally:
        qkr.set_variant_override(None)

    rs, ry = oracle.add_rms_norm(x_in, W.as_f32(w), W.EPS, r_in if c["add"] else None, dtype,
                                 "fp8_e4m3" if c["fp8"] else dtype, c["scale"])
    what = f"rows case {i}"
    if c["add"]:
        assert np.array_equal(host(s), rs), f"{what}: the residual stream must be bit-exact"
        if c["res_out"] != "residual":
            assert torch.equal(gr[:, :width].cpu(), rb[:, :width]), f"{what}: residual input changed"
    if c["fp8"]:
        assert_fp8_close(y.view(torch.uint8).cpu().numpy(), ry, what=what)
    else:
        check(host(y), ry, dtype, what=what)
    if pad:   # the elements past each row are never written
        assert torch.equal(gx[:, width:].cpu(), xb[:, width:]) and torch.equal(gr[:, width:].cpu(), rb[:, width:])


# ---------------------------------------------------------------- joint ----

def draw_joint(i):
    rng = np.random.default_rng([W.SEED, 5201, i])
    c = {"dtype": str(rng.choice(["bf16", "f32"]))}
    ve = 8 if c["dtype"] == "bf16" else 4
    c["d"] = int(rng.choice(HEAD_DIMS))
    c["pairing"] = str(rng.choice(["neox", "adjacent"]))
    step = 2 * ve if c["pairing"] == "neox" else 2
    choices = list(range(step, c["d"] + 1, step))
    c["rot"] = c["d"] if rng.random() < 0.6 and c["d"] % step == 0 else int(rng.choice(choices))
    c["sections"] = tuple(split(rng, c["rot"] // 2, 3)) + (0,)
    c["batch"] = int(rng.integers(1, 3))
    c["txt"] = int(rng.choice([0, 1, 5, 17, 64]))
    c["img"] = int(rng.integers(1, 150))
    c["heads"] = int(rng.integers(1, 13))
    return c


@pytest.mark.parametrize("i", range(96))
def test_random_joint(i):
    c = draw_joint(i)
    print(f"joint case {i}: {c}", flush=True)
    rng = np.random.default_rng([W.SEED, 5202, i])
    dtype, d, h, b = c["dtype"], c["d"], c["heads"], c["batch"]
    total = c["txt"] + c["img"]
    pos = rng.integers(0, 4096, (3, total)).astype(np.int32)
    inv = W.inv_freq_ladder(1e4, c["rot"])
    streams_cpu, streams_gpu, streams_ref = {}, {}, {}
    for nm, n in (("text", c["txt"]), ("image", c["img"])):
        qkv = W.to_dtype(rng.normal(0, 1, (b, n, 3, h, d)).astype(np.float32), dtype)   # packed projection
        wq = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
        wk = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
        g = qkv.to(DEV)
        streams_gpu[nm] = {"q": g[:, :, 0], "k": g[:, :, 1], "v": g[:, :, 2], "q_weight": wq.to(DEV),
                           "k_weight": wk.to(DEV)}
        streams_ref[nm] = {"q": W.as_f32(qkv[:, :, 0]), "k": W.as_f32(qkv[:, :, 1]), "v": W.as_f32(qkv[:, :, 2]),
                           "q_weight": W.as_f32(wq), "k_weight": W.as_f32(wk)}
        streams_cpu[nm] = qkv
    rope = qkr.Rope("axes", c["rot"], c["pairing"], inv_freq=torch.from_numpy(inv).to(DEV),
                    positions=torch.from_numpy(pos).to(DEV), sections=c["sections"])
    q, k, v = qkr.joint_qk_norm_rope(streams_gpu["text"], streams_gpu["image"], W.EPS, rope)
    orope = oracle.Rope("axes", c["rot"], c["pairing"], inv_freq=inv, sections=c["sections"], positions=pos)
    rq, rk, rv = oracle.joint_qk_norm_rope(streams_ref["text"], streams_ref["image"], W.EPS, orope, dtype)
    for bi in range(b):
        check(host(q[bi]), rq[bi], dtype, c["rot"], c["pairing"], f"joint case {i} q batch {bi}")
        check(host(k[bi]), rk[bi], dtype, c["rot"], c["pairing"], f"joint case {i} k batch {bi}")
    assert np.array_equal(host(v), rv), f"joint case {i}: V must be copied bit for bit"


# ---------------------------------------------------------------- cache ----

def draw_cache(i):
    rng = np.random.default_rng([W.SEED, 5301, i])
    c = {"dtype": str(rng.choice(["bf16", "f32"]))}
    ve = 8 if c["dtype"] == "bf16" else 4
    c["d"] = int(rng.choice(HEAD_DIMS))
    c["mode"] = str(rng.choice(["1d", "imrope", "axes"]))
    c["pairing"] = "neox" if (c["d"] // 2) % ve == 0 and rng.random() < 0.7 else "adjacent"
    c["tokens"] = int(rng.integers(1, 200))
    c["qh"] = int(rng.integers(1, 13))
    c["kvh"] = int(rng.integers(1, 9))
    c["with_v"] = bool(rng.random() < 0.7)
    c["paged"] = bool(rng.random() < 0.5)
    c["block"] = int(rng.choice([1, 16, 32]))
    return c


@pytest.mark.parametrize("i", range(96))
def test_random_cache(i):
    c = draw_cache(i)
    print(f"cache case {i}: {c}", flush=True)
    rng = np.random.default_rng([W.SEED, 5302, i])
    dtype, d, t, qh, kvh = c["dtype"], c["d"], c["tokens"], c["qh"], c["kvh"]
    rot, half = d, d // 2
    q = W.to_dtype(rng.normal(0, 1, (t, qh, d)).astype(np.float32), dtype)
    k = W.to_dtype(rng.normal(0, 1, (t, kvh, d)).astype(np.float32), dtype)
    v = W.to_dtype(rng.normal(0, 1, (t, kvh, d)).astype(np.float32), dtype)
    wq = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
    wk = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
    planes = {"1d": 1, "axes": 3, "imrope": 4}[c["mode"]]
    pos = rng.integers(0, 8192, (planes, t)).astype(np.int32)
    inv = W.inv_freq_ladder(1e6, rot)
    sections = ((0, 0, 0, 0) if c["mode"] == "1d" else
                tuple(split(rng, half, 3)) + (0,) if c["mode"] == "axes" else
                tuple(split(rng, int(rng.integers(half, 2 * half + 1)), 4)))
    blocks = int(np.ceil((t + 8) / c["block"])) + 2
    num_slots = blocks * c["block"]
    slots = rng.permutation(num_slots)[:t].astype(np.int64)
    if t > 4:
        slots[rng.choice(t, t // 5, replace=False)] = -1           # padding tokens
        slots[rng.choice(t, 2, replace=False)] = [num_slots, 1 << 35]   # outside the cache
    fill = 0.75
    shape = (blocks, c["block"], kvh, d) if c["paged"] else (num_slots, kvh, d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.full(shape, fill, dtype=tdt, device=DEV)
    vc = torch.full(shape, fill, dtype=tdt, device=DEV) if c["with_v"] else None
    rope = qkr.Rope(c["mode"], rot, c["pairing"], inv_freq=torch.from_numpy(inv).to(DEV),
                    positions=torch.from_numpy(pos).to(DEV), sections=sections)
    qo = qkr.qk_norm_rope_cache(q.to(DEV), k.to(DEV), v.to(DEV) if c["with_v"] else None, wq.to(DEV), wk.to(DEV),
                                kc, vc, torch.from_numpy(slots).to(DEV), W.EPS, rope)
    orope = oracle.Rope(c["mode"], rot, c["pairing"], inv_freq=inv, sections=sections, positions=pos)
    kc0 = np.full((num_slots, kvh, d), fill, np.float32)
    rq, rk, rv = oracle.qk_norm_rope_cache(W.as_f32(q), W.as_f32(k), W.as_f32(v) if c["with_v"] else None,
                                           W.as_f32(wq), W.as_f32(wk), W.EPS, orope, slots, kc0,
                                           kc0.copy() if c["with_v"] else None, dtype)
    what = f"cache case {i}"
    check(host(qo), rq, dtype, rot, c["pairing"], f"{what} q")
    gk = host(kc).reshape(num_slots, kvh, d)
    mapped = np.zeros(num_slots, bool)
    mapped[slots[(slots >= 0) & (slots < num_slots)]] = True
    assert np.array_equal(gk[~mapped], rk[~mapped]), f"{what}: unmapped cache rows changed"
    if mapped.any():
        check(gk[mapped], rk[mapped], dtype, rot, c["pairing"], f"{what} k cache")
    if c["with_v"]:
        assert np.array_equal(host(vc).reshape(num_slots, kvh, d), rv), f"{what}: V must be copied bit for bit"


# ---------------------------------------------------------------- ViT ------

def split_positive(rng, total, parts):
    """`parts` ints >= 1 summing to `total` (total >= parts)."""
    return [x + 1 for x in split(rng, total - parts, parts)]


def draw_vit(i):
    rng = np.random.default_rng([W.SEED, 5401, i])
    c = {"dtype": str(rng.choice(["bf16", "f32"])), "pairing": str(rng.choice(["neox", "adjacent"]))}
    ve = 8 if c["dtype"] == "bf16" else 4
    c["merge"] = int(rng.choice([1, 2, 3]))
    n_grids = int(rng.choice([1, 2, 3, 6, 33, 40]))
    m = c["merge"]
    c["grids"] = [[int(rng.integers(1, 4)), m * int(rng.integers(1, 6)), m * int(rng.integers(1, 6))]
                  for _ in range(n_grids)]
    c["d"] = int(rng.choice([d for d in HEAD_DIMS if d % ve == 0 and d >= 16]))
    unit = ve if c["pairing"] == "neox" else 1            # NeoX halves are whole 16-byte vectors
    max_half = c["d"] // 2
    half = unit * int(rng.integers(max(1, -(-3 // unit)), max_half // unit + 1))
    c["halves"] = tuple(split_positive(rng, half, 3))
    c["hq"] = int(rng.integers(1, 5))
    c["hk"] = int(rng.integers(1, 5))
    return c


@pytest.mark.parametrize("i", range(64))
def test_random_vit(i):
    c = draw_vit(i)
    print(f"vit case {i}: {c}", flush=True)
    rng = np.random.default_rng([W.SEED, 5402, i])
    dtype, d, grids, merge = c["dtype"], c["d"], c["grids"], c["merge"]
    n = sum(t * h * w for t, h, w in grids)
    ht, hh, hw = c["halves"]
    half = ht + hh + hw
    inv = [W.inv_freq_ladder(1e4, 2 * x) for x in (ht, hh, hw)]
    ginv = [torch.from_numpy(a).to(DEV) for a in inv]
    q = W.to_dtype(rng.normal(0, 1, (n, c["hq"], d)).astype(np.float32), dtype)
    k = W.to_dtype(rng.normal(0, 1, (n, c["hk"], d)).astype(np.float32), dtype)
    wq = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
    wk = W.to_dtype(rng.normal(1, 0.1, d).astype(np.float32), dtype)
    qo, ko = qkr.vit_qk_norm_rope(q.to(DEV), k.to(DEV), wq.to(DEV), wk.to(DEV), W.EPS, *ginv, grids, merge,
                                  c["pairing"])
    for name, x, w, out in (("q", q, wq, qo), ("k", k, wk, ko)):
        ref = oracle.vit_qk_norm_rope(W.as_f32(x), W.as_f32(w), W.EPS, *inv, grids, merge, c["pairing"], dtype)
        check(host(out), ref, dtype, 2 * half, c["pairing"], f"vit case {i} {name}")
    # The setup planes of the same grids: each plane's own columns, nothing else.
    cos = torch.full((3, n, half), float("nan"), device=DEV)
    sin = torch.full((3, n, half), float("nan"), device=DEV)
    qkr.mrope_cos_sin_setup(*ginv, grids, merge, out=(cos, sin))
    rc, rs = oracle.vit_cos_sin(*inv, grids, merge)
    gc, gs = cos.cpu().numpy(), sin.cpu().numpy()
    written = ~np.isnan(rc)
    assert np.array_equal(np.isnan(gc), ~written) and np.array_equal(np.isnan(gs), ~written)
    assert_f32_close(gc[written], rc[written], f"vit case {i} cos")
    assert_f32_close(gs[written], rs[written], f"vit case {i} sin")
