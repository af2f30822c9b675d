"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input is seeded and synthetic (workloads.py); the oracle receives the
exact values the GPU reads.  Tolerances are in tests/parity.py.
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


def gpu(t):
    return t.to(DEV)


def host(t):
    return t.detach().float().cpu().numpy()


def dt_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def check(got, ref, dtype, rotary_dim=0, pairing="neox", what=""):
    if dtype == "f32":
        return assert_f32_close(got, ref, what)
    return assert_bf16_close(got, ref, rotary_dim, pairing, what)


# ---------------------------------------------------------------------------
# index maps (exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode,sections,pairs", [
    ("imrope", (24, 20, 20, 0), 64), ("imrope", (20, 24, 16, 4), 64), ("imrope", (0, 0, 0, 64), 64),
    ("imrope", (40, 40, 40, 8), 64), ("axes", (8, 28, 28, 0), 64), ("planes", (8, 16, 16, 0), 40),
    ("1d", (0, 0, 0, 0), 128),
])
def test_device_axis_map_matches_oracle(mode, sections, pairs):
    got = qkr.debug_axis_map(mode, sections, pairs).cpu().numpy()
    expect = oracle.axis_map(oracle.Rope(mode, 2 * pairs, sections=sections), pairs)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("grids,merge", [
    ([[1, 64, 64], [2, 32, 48], [1, 28, 28]], 2),
    ([[1, 4, 6], [2, 2, 4]], 2),
    ([[2, 6, 9]], 3),
    ([[1, 8, 8]] * 70, 2),
])
def test_device_vit_positions_match_oracle(grids, merge):
    got = qkr.debug_vit_positions(grids, merge).cpu().numpy()
    assert np.array_equal(got, oracle.vit_positions(grids, merge))


# ---------------------------------------------------------------------------
# tiny: fp32 [4, 2, 64], NeoX 1-D RoPE (and bf16 / other head dims)
# ---------------------------------------------------------------------------

def run_1d(case, pairing="neox", rotary_dim=None, positions=None):
    rd = case.rotary_dim if rotary_dim is None else rotary_dim
    pos = case.positions if positions is None else positions
    inv = W.inv_freq_ladder(1e4, rd) if rd else case.inv_freq
    rope = qkr.Rope("1d", rd, pairing, inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    qo, ko = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    orope = oracle.Rope("1d", rd, pairing, inv_freq=inv, positions=pos)
    rq = oracle.qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), case.eps, orope, case.dtype)
    rk = oracle.qk_norm_rope(W.as_f32(case.k), W.as_f32(case.k_weight), case.eps, orope, case.dtype)
    return host(qo), host(ko), rq, rk


def test_tiny_fp32_neox():
    case = W.tiny()
    qo, ko, rq, rk = run_1d(case)
    assert_f32_close(qo, rq, "q")
    assert_f32_close(ko, rk, "k")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("head_dim", [16, 32, 64, 80, 128, 256])
@pytest.mark.parametrize("pairing", ["neox", "adjacent"])
def test_head_dims_and_pairings(dtype, head_dim, pairing):
    case = W.tiny(tokens=37, heads=5, head_dim=head_dim, dtype=dtype, seed_stream=head_dim)
    pos = np.random.default_rng(head_dim).integers(0, 9000, (1, 37)).astype(np.int32)
    qo, ko, rq, rk = run_1d(case, pairing, positions=pos)
    check(qo, rq, dtype, head_dim, pairing, "q")
    check(ko, rk, dtype, head_dim, pairing, "k")


@pytest.mark.parametrize("dtype,head_dim,rotary_dim,pairing", [
    ("bf16", 128, 64, "neox"), ("bf16", 128, 32, "neox"), ("bf16", 256, 128, "neox"),
    ("f32", 64, 24, "neox"), ("bf16", 128, 96, "adjacent"), ("bf16", 80, 34, "adjacent"),
    ("f32", 128, 2, "adjacent"), ("bf16", 128, 0, "neox"),
])
def test_partial_rotary(dtype, head_dim, rotary_dim, pairing):
    case = W.tiny(tokens=19, heads=3, head_dim=head_dim, dtype=dtype, seed_stream=rotary_dim + 1000)
    pos = np.random.default_rng(rotary_dim).integers(0, 5000, (1, 19)).astype(np.int32)
    qo, ko, rq, rk = run_1d(case, pairing, rotary_dim=rotary_dim, positions=pos)
    check(qo, rq, dtype, rotary_dim, pairing, "q")
    check(ko, rk, dtype, rotary_dim, pairing, "k")


def test_position_zero_equals_norm_only_bitwise():
    case = W.tiny(tokens=64, heads=7, head_dim=128, dtype="bf16", seed_stream=5)
    zeros = np.zeros((1, 64), np.int32)
    for pairing in ("neox", "adjacent"):
        rope = qkr.Rope("1d", 128, pairing, inv_freq=gpu(torch.from_numpy(W.inv_freq_ladder(1e4, 128))),
                        positions=gpu(torch.from_numpy(zeros)))
        a, b = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), 1e-6, rope)
        c, d = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), 1e-6, None)
        assert torch.equal(a, c) and torch.equal(b, d)


@pytest.mark.parametrize("d", [128, 80])
def test_batch_and_strided_views(d):
    """[batch, tokens, heads, D] views carved out of a wider buffer, positions
    shared across the batch."""
    rng = np.random.default_rng(11 + d)
    b, t, hq, hk = 3, 50, 6, 2
    big = torch.from_numpy(rng.normal(0, 1, (b, t, hq + hk + 3, d)).astype(np.float32)).to(torch.bfloat16)
    q, k = big[:, :, :hq], big[:, :, hq + 1:hq + 1 + hk]
    wq = torch.from_numpy(rng.normal(1, 0.1, d).astype(np.float32)).to(torch.bfloat16)
    wk = torch.from_numpy(rng.normal(1, 0.1, d).astype(np.float32)).to(torch.bfloat16)
    pos = rng.integers(0, 4096, (1, t)).astype(np.int32)
    inv = W.inv_freq_ladder(1e4, d)
    gbig = gpu(big)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    qo, ko = qkr.qk_norm_rope(gbig[:, :, :hq], gbig[:, :, hq + 1:hq + 1 + hk], gpu(wq), gpu(wk), 1e-6, rope)
    orope = oracle.Rope("1d", d, "neox", inv_freq=inv, positions=pos)
    for bi in range(b):
        assert_bf16_close(host(qo[bi]), oracle.qk_norm_rope(W.as_f32(q[bi]), W.as_f32(wq), 1e-6, orope), d)
        assert_bf16_close(host(ko[bi]), oracle.qk_norm_rope(W.as_f32(k[bi]), W.as_f32(wk), 1e-6, orope), d)


def test_in_place():
    case = W.tiny(tokens=40, heads=4, head_dim=128, dtype="bf16", seed_stream=9)
    pos = np.arange(40, dtype=np.int32)[None] * 7
    inv = W.inv_freq_ladder(1e4, 128)
    rope = qkr.Rope("1d", 128, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    q, k = gpu(case.q), gpu(case.k)
    ref_q, ref_k = qkr.qk_norm_rope(q, k, gpu(case.q_weight), gpu(case.k_weight), 1e-6, rope)
    qkr.qk_norm_rope(q, k, gpu(case.q_weight), gpu(case.k_weight), 1e-6, rope, q_out=q, k_out=k)
    assert torch.equal(q, ref_q) and torch.equal(k, ref_k)


def test_q_only_and_k_only():
    case = W.tiny(tokens=21, heads=3, head_dim=64, dtype="bf16", seed_stream=3)
    pos = np.arange(21, dtype=np.int32)[None]
    inv = W.inv_freq_ladder(1e4, 64)
    rope = qkr.Rope("1d", 64, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    orope = oracle.Rope("1d", 64, "neox", inv_freq=inv, positions=pos)
    qo, ko = qkr.qk_norm_rope(gpu(case.q), None, gpu(case.q_weight), None, 1e-6, rope)
    assert ko is None
    assert_bf16_close(host(qo), oracle.qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), 1e-6, orope), 64)
    qo, ko = qkr.qk_norm_rope(None, gpu(case.k), None, gpu(case.k_weight), 1e-6, rope)
    assert qo is None
    assert_bf16_close(host(ko), oracle.qk_norm_rope(W.as_f32(case.k), W.as_f32(case.k_weight), 1e-6, orope), 64)


@pytest.mark.parametrize("eps", [0.0, 1e-40])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_eps_below_the_normal_range(eps, dtype):
    """An eps of zero or a subnormal eps takes the kernels' library reciprocal
    square root (the bare instruction is used only for a normal eps)."""
    case = W.tiny(tokens=23, heads=4, head_dim=128, dtype=dtype, seed_stream=4242)
    case.eps = eps
    pos = np.random.default_rng(11).integers(0, 3000, (1, 23)).astype(np.int32)
    qo, ko, rq, rk = run_1d(case, "neox", positions=pos)
    check(qo, rq, dtype, 128, "neox", "q")
    check(ko, rk, dtype, 128, "neox", "k")
    rows = W.rows(9, width=1000, dtype=dtype, seed_stream=4243)
    for variant in (None, "rms:rows", "rms:wide"):
        qkr.set_variant_override(variant)
        try:
            y = qkr.rms_norm(gpu(rows.x), gpu(rows.weight), eps)
        finally:
            qkr.set_variant_override(None)
        ref = oracle.rms_norm(W.as_f32(rows.x), W.as_f32(rows.weight), eps, dtype)
        check(host(y), ref, dtype, what=f"rms eps={eps} {variant}")


# ---------------------------------------------------------------------------
# rows: plain RMSNorm, bf16 [t, 5120], t in {1, 32, 4096}; every variant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("t", [1, 32, 4096])
@pytest.mark.parametrize("variant", [None, "rms:rows", "rms:split", "rms:wide"])
def test_rms_norm_rows(t, variant):
    case = W.rows(t)
    qkr.set_variant_override(variant)
    try:
        y = qkr.rms_norm(gpu(case.x), gpu(case.weight), case.eps)
        name = qkr.last_variant()
    finally:
        qkr.set_variant_override(None)
    if variant is not None:
        assert name.startswith(variant + ":"), name
    else:
        assert name.startswith("rms:rows" if 2048 <= t <= 4096 else "rms:wide"), name
    ref = oracle.rms_norm(W.as_f32(case.x), W.as_f32(case.weight), case.eps, "bf16")
    assert_bf16_close(host(y), ref, what=f"rms t={t} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("width", [8, 64, 1000, 2048, 4104, 8192, 12800, 16384, 32768])
def test_rms_norm_widths(dtype, width):
    if dtype == "f32" and width % 4:
        pytest.skip("fp32 rows must be 16-byte multiples")
    if dtype == "f32" and width > 16384:
        pytest.skip("fp32 rows are limited to 16384 elements (65536 bytes, the bf16 maximum of 32768)")
    case = W.rows(7, width=width, dtype=dtype, seed_stream=width)
    nvec = width // (8 if dtype == "bf16" else 4)
    for variant in (None, "rms:rows", "rms:split", "rms:wide"):
        qkr.set_variant_override(variant)
        try:
            if variant in ("rms:rows", "rms:split") and nvec > 1024:
                # one wavefront holds at most 1024 vectors: refused, not swapped
                with pytest.raises(qkr.QkrError, match="forced variant"):
                    qkr.rms_norm(gpu(case.x), gpu(case.weight), case.eps)
                continue
            y = qkr.rms_norm(gpu(case.x), gpu(case.weight), case.eps)
            if variant is not None:
                assert qkr.last_variant().startswith(variant + ":"), qkr.last_variant()
        finally:
            qkr.set_variant_override(None)
        ref = oracle.rms_norm(W.as_f32(case.x), W.as_f32(case.weight), case.eps, dtype)
        check(host(y), ref, dtype, what=f"width {width} {variant}")


def test_rms_norm_strided_rows():
    case = W.rows(33, width=5120, seed_stream=77)
    buf = torch.zeros(33, 5120 + 64, dtype=torch.bfloat16)
    buf[:, 32:32 + 5120] = case.x
    g = gpu(buf)
    x = g[:, 32:32 + 5120]
    out = torch.zeros(33, 5120 + 128, dtype=torch.bfloat16, device=DEV)
    y = qkr.rms_norm(x, gpu(case.weight), case.eps, out=out[:, 64:64 + 5120])
    ref = oracle.rms_norm(W.as_f32(case.x), W.as_f32(case.weight), case.eps, "bf16")
    assert_bf16_close(host(y), ref)
    assert (out[:, :64] == 0).all() and (out[:, 64 + 5120:] == 0).all()


# ---------------------------------------------------------------------------
# joint text/image op (512 + 4096 tokens, 24 x 128, 3-axis RoPE)
# ---------------------------------------------------------------------------

def joint_gpu(case, pairing, rope_tokens=None):
    hd = case.head_dim
    g = {}
    for nm, s in (("text", case.text), ("image", case.image)):
        qkv = gpu(s.qkv)
        v = qkv.view(qkv.shape[0], qkv.shape[1], 3, case.heads, hd)
        g[nm] = {"q": v[:, :, 0], "k": v[:, :, 1], "v": v[:, :, 2], "q_weight": gpu(s.q_weight),
                 "k_weight": gpu(s.k_weight)}
    rope = qkr.Rope("axes", hd, pairing, inv_freq=gpu(torch.from_numpy(case.inv_freq)),
                    positions=gpu(torch.from_numpy(case.positions)), sections=case.sections)
    return g, rope


def joint_oracle(case, pairing):
    hd = case.head_dim

    def stream(s):
        return {"q": W.as_f32(s.view(0, case.heads, hd)), "k": W.as_f32(s.view(1, case.heads, hd)),
                "v": W.as_f32(s.view(2, case.heads, hd)), "q_weight": W.as_f32(s.q_weight),
                "k_weight": W.as_f32(s.k_weight)}

    rope = oracle.Rope("axes", hd, pairing, inv_freq=case.inv_freq, sections=case.sections,
                       positions=case.positions)
    return oracle.joint_qk_norm_rope(stream(case.text), stream(case.image), case.eps, rope, "bf16")


@pytest.mark.parametrize("pairing", ["adjacent", "neox"])
def test_joint_full_size(pairing):
    case = W.joint()
    g, rope = joint_gpu(case, pairing)
    q, k, v = qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope)
    # 24 heads: three passes of 8 in tiles of two, a quarter of them idle
    assert qkr.last_variant().startswith("rope:np2:"), qkr.last_variant()
    rq, rk, rv = joint_oracle(case, pairing)
    assert_bf16_close(host(q), rq, 128, pairing, "joint q")
    assert_bf16_close(host(k), rk, 128, pairing, "joint k")
    assert np.array_equal(host(v), rv)


def test_joint_equals_per_stream_bitwise():
    """joint == cat(text, image) of per-stream qk_norm_rope calls reading the
    joint positions at token_base 0 and S_txt."""
    case = W.joint(tokens_txt=77, grid=(12, 20), heads=5, batch=2, seed_stream=3)
    g, rope = joint_gpu(case, "adjacent")
    q, k, v = qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope)
    st = 77
    for nm, base, sl in (("text", 0, slice(0, st)), ("image", st, slice(st, None))):
        r = qkr.Rope("axes", 128, "adjacent", inv_freq=rope.inv_freq, positions=rope.positions,
                     sections=case.sections, token_base=base)
        s = g[nm]
        qs, ks = qkr.qk_norm_rope(s["q"], s["k"], s["q_weight"], s["k_weight"], case.eps, r)
        assert torch.equal(q[:, sl], qs) and torch.equal(k[:, sl], ks)
        assert torch.equal(v[:, sl], s["v"])


def test_joint_ragged_and_empty_streams():
    for st, grid in ((0, (8, 8)), (13, (1, 1)), (5, (3, 7))):
        case = W.joint(tokens_txt=st, grid=grid, heads=3, seed_stream=st)
        g, rope = joint_gpu(case, "adjacent")
        q, k, v = qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope)
        rq, rk, rv = joint_oracle(case, "adjacent")
        assert_bf16_close(host(q), rq, 128, "adjacent")
        assert_bf16_close(host(k), rk, 128, "adjacent")
        assert np.array_equal(host(v), rv)


# ---------------------------------------------------------------------------
# IMROPE (8192 tokens, 16 + 8 heads, sections [24, 20, 20, 0], 2048-token chunks)
# ---------------------------------------------------------------------------

def imrope_call(case, q, k, pos, inv, token_base, tokens=None):
    rope = qkr.Rope("imrope", 128, "neox", inv_freq=inv, positions=pos, sections=case.sections,
                    token_base=token_base)
    return qkr.qk_norm_rope(q, k, gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)


def test_imrope_full_size_chunked():
    case = W.imrope()
    pos, inv = gpu(torch.from_numpy(case.positions)), gpu(torch.from_numpy(case.inv_freq))
    q, k = gpu(case.q), gpu(case.k)
    outs = [imrope_call(case, q[b:b + case.chunk], k[b:b + case.chunk], pos, inv, b)
            for b in range(0, 8192, case.chunk)]
    # 16 Q heads fill a tile of two passes, 8 K heads half of one
    assert qkr.last_variant().startswith("rope:np2:"), qkr.last_variant()
    qo = torch.cat([o[0] for o in outs])
    ko = torch.cat([o[1] for o in outs])
    orope = oracle.Rope("imrope", 128, "neox", inv_freq=case.inv_freq, sections=case.sections,
                        positions=case.positions)
    assert_bf16_close(host(qo), oracle.qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), case.eps, orope),
                      128, "neox", "imrope q")
    assert_bf16_close(host(ko), oracle.qk_norm_rope(W.as_f32(case.k), W.as_f32(case.k_weight), case.eps, orope),
                      128, "neox", "imrope k")
    # chunked == one launch, bitwise
    q1, k1 = imrope_call(case, q, k, pos, inv, 0)
    assert torch.equal(q1, qo) and torch.equal(k1, ko)


@pytest.mark.parametrize("tokens", [2, 300, 2457])
def test_imrope_test_sizes(tokens):
    """Token counts the IMROPE page tests (2, 300, 2,457), with ragged chunks."""
    case = W.imrope(tokens=tokens, seed_stream=tokens)
    pos, inv = gpu(torch.from_numpy(case.positions)), gpu(torch.from_numpy(case.inv_freq))
    q, k = gpu(case.q), gpu(case.k)
    full = imrope_call(case, q, k, pos, inv, 0)
    orope = oracle.Rope("imrope", 128, "neox", inv_freq=case.inv_freq, sections=case.sections,
                        positions=case.positions)
    assert_bf16_close(host(full[0]), oracle.qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), case.eps,
                                                         orope), 128)
    assert_bf16_close(host(full[1]), oracle.qk_norm_rope(W.as_f32(case.k), W.as_f32(case.k_weight), case.eps,
                                                         orope), 128)
    step = 1000
    for b in range(0, tokens, step):
        part = imrope_call(case, q[b:b + step], k[b:b + step], pos, inv, b)
        assert torch.equal(part[0], full[0][b:b + step]) and torch.equal(part[1], full[1][b:b + step])


def test_imrope_differs_from_plain_and_collapses():
    case = W.imrope(tokens=64, seed_stream=8)
    pos, inv = gpu(torch.from_numpy(case.positions)), gpu(torch.from_numpy(case.inv_freq))
    q, k = gpu(case.q), gpu(case.k)
    sect = imrope_call(case, q, k, pos, inv, 0)
    plain = qkr.qk_norm_rope(q, k, gpu(case.q_weight), gpu(case.k_weight), case.eps,
                             qkr.Rope("1d", 128, "neox", inv_freq=inv, positions=pos[0:1]))
    assert (sect[0] - plain[0]).abs().max().item() > 0.1
    # all pairs on e == plain over plane e
    all_e = qkr.Rope("imrope", 128, "neox", inv_freq=inv, positions=pos, sections=(0, 0, 0, 64))
    plain_e = qkr.Rope("1d", 128, "neox", inv_freq=inv, positions=pos[3:4].contiguous())
    a = qkr.qk_norm_rope(q, k, gpu(case.q_weight), gpu(case.k_weight), case.eps, all_e)
    b = qkr.qk_norm_rope(q, k, gpu(case.q_weight), gpu(case.k_weight), case.eps, plain_e)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# ViT setup + apply (grids [[1,64,64],[2,32,48],[1,28,28]], merge 2, 16 x 80)
# ---------------------------------------------------------------------------

def test_vit_setup_planes_and_sentinel():
    case = W.vit()
    n, half = case.n_tokens, case.half_rot
    inv = [gpu(torch.from_numpy(a)) for a in (case.inv_t, case.inv_h, case.inv_w)]
    cos = torch.full((3, n, half), float("nan"), device=DEV)
    sin = torch.full((3, n, half), float("nan"), device=DEV)
    qkr.mrope_cos_sin_setup(*inv, case.grid_thw, case.merge, out=(cos, sin))
    rc, rs = oracle.vit_cos_sin(case.inv_t, case.inv_h, case.inv_w, case.grid_thw, case.merge)
    gc, gs = cos.cpu().numpy(), sin.cpu().numpy()
    written = ~np.isnan(rc)
    assert np.array_equal(np.isnan(gc), ~written) and np.array_equal(np.isnan(gs), ~written)
    assert_f32_close(gc[written], rc[written], "cos")
    assert_f32_close(gs[written], rs[written], "sin")


def test_vit_apply_chain():
    """setup -> planes -> apply on the GPU against the oracle's own chain
    (oracle planes, oracle apply); the apply never reads an unwritten column
    (those are NaN)."""
    case = W.vit()
    n, half = case.n_tokens, case.half_rot
    inv = [gpu(torch.from_numpy(a)) for a in (case.inv_t, case.inv_h, case.inv_w)]
    cos = torch.full((3, n, half), float("nan"), device=DEV)
    sin = torch.full((3, n, half), float("nan"), device=DEV)
    qkr.mrope_cos_sin_setup(*inv, case.grid_thw, case.merge, out=(cos, sin))
    secs = (case.inv_t.size, case.inv_h.size, case.inv_w.size, 0)
    rope = qkr.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=cos, sin_planes=sin)
    qo, ko = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    rc, rs = oracle.vit_cos_sin(case.inv_t, case.inv_h, case.inv_w, case.grid_thw, case.merge)
    orope = oracle.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=rc, sin_planes=rs)
    rq = oracle.qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), case.eps, orope)
    rk = oracle.qk_norm_rope(W.as_f32(case.k), W.as_f32(case.k_weight), case.eps, orope)
    assert not torch.isnan(qo.float()).any() and not torch.isnan(ko.float()).any()
    assert_bf16_close(host(qo), rq, 2 * half, "neox", "vit q")
    assert_bf16_close(host(ko), rk, 2 * half, "neox", "vit k")


# ---------------------------------------------------------------------------
# 64-bit addressing: a view more than 2^31 elements into a > 4 GiB buffer
# ---------------------------------------------------------------------------

def test_large_storage_offset():
    case = W.tiny(tokens=16, heads=8, head_dim=128, dtype="bf16", seed_stream=21)
    off = (1 << 31) + 4096                     # elements
    total = off + 16 * 8 * 128 + 4096
    buf = torch.empty(total, dtype=torch.bfloat16, device=DEV)
    x = buf[off:off + 16 * 8 * 128].view(16, 8, 128)
    x.copy_(gpu(case.q))
    pos = np.arange(16, dtype=np.int32)[None] * 31
    inv = W.inv_freq_ladder(1e4, 128)
    rope = qkr.Rope("1d", 128, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    out = buf[off - 16 * 8 * 128 - 2048:off - 2048].view(16, 8, 128)
    qkr.qk_norm_rope(x, None, gpu(case.q_weight), None, 1e-6, rope, q_out=out)
    ref = oracle.qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), 1e-6,
                              oracle.Rope("1d", 128, "neox", inv_freq=inv, positions=pos))
    assert_bf16_close(host(out), ref, 128)
    del buf
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# HIP graph capture: replays match eager calls, every replay
# ---------------------------------------------------------------------------

def test_maximum_row_count():
    """A call at the row limit: 2^31 - 64 rows (2^25 - 1 tokens x 64 heads of
    fp32 x 8, 64 GiB each way), checked against the oracle on sampled tokens,
    the first and last included."""
    tokens, heads, d = (1 << 25) - 1, 64, 8
    rows = tokens * heads
    assert rows == (1 << 31) - 64
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    if free < 2 * rows * d * 4 + (4 << 30):
        pytest.skip(f"needs {2 * rows * d * 4 / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free")
    g = torch.Generator(device=DEV).manual_seed(W.SEED)
    q = torch.randn((tokens, heads, d), device=DEV, generator=g)
    w = torch.rand(d, device=DEV, generator=g) + 0.5
    pos = torch.randint(0, 8192, (1, tokens), dtype=torch.int32, device=DEV, generator=g)
    inv = W.inv_freq_ladder(1e4, d)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=pos)
    try:
        qo, ko = qkr.qk_norm_rope(q, None, w, None, W.EPS, rope)
        assert ko is None
        rng = np.random.default_rng(W.SEED)
        toks = torch.from_numpy(np.unique(np.concatenate([[0, 1, tokens - 2, tokens - 1],
                                                          rng.integers(0, tokens, 1024)]))).to(DEV)
        qs, got, ps = host(q[toks]), host(qo[toks]), pos[:, toks].cpu().numpy()
    finally:
        del q
        qo = None
        torch.cuda.empty_cache()
    orope = oracle.Rope("1d", d, "neox", inv_freq=inv, positions=ps)
    ref = oracle.qk_norm_rope(qs, host(w), W.EPS, orope, "f32")
    assert_f32_close(got, ref, "maximum row count")


def _sampled_rows(n, boundary, rng):
    """Row indices to check: both ends, both sides of a launch boundary and a
    random sample."""
    edge = [0, 1, boundary - 2, boundary - 1, boundary, boundary + 1, n - 2, n - 1]
    return np.unique(np.concatenate([edge, rng.integers(0, n, 2048)]))


@pytest.mark.parametrize("variant", [None, "rms:wide"])
def test_rms_norm_rows_past_one_dispatch(variant):
    """2^26 rows of 8 bf16: one wavefront per row needs 2^32 work-items and
    one workgroup per row 2^34, more than one dispatch counts, so the call
    takes several launches, each told its first row; sampled rows on both
    sides of each launch boundary match the oracle."""
    rows, width = 1 << 26, 8
    g = torch.Generator(device=DEV).manual_seed(W.SEED)
    x = torch.randn((rows, width), device=DEV, generator=g).to(torch.bfloat16)
    w = (torch.rand(width, device=DEV, generator=g) + 0.5).to(torch.bfloat16)
    qkr.set_variant_override(variant)
    try:
        y = qkr.rms_norm(x, w, W.EPS)
        name = qkr.last_variant()
    finally:
        qkr.set_variant_override(None)
    assert name.startswith("rms:rows" if variant is None else variant), name
    per_launch = (1 << 23) * (4 if variant is None else 1)     # rows of one launch
    idx = _sampled_rows(rows, per_launch, np.random.default_rng(1))
    for b in range(per_launch, rows, per_launch):
        idx = np.union1d(idx, [b - 1, b])
    ti = torch.from_numpy(idx).to(DEV)
    got, xs = host(y[ti]), host(x[ti])
    del x, y
    torch.cuda.empty_cache()
    ref = oracle.rms_norm(xs, host(w), W.EPS, "bf16")
    assert_bf16_close(got, ref, what=f"rows past one dispatch {name}")


def test_qk_norm_rope_tiles_past_one_dispatch():
    """2^26 tokens of one fp32 head of 8: 2^26 tiles of one wavefront, 2^32
    work-items, two launches; sampled tokens on both sides of the boundary
    match the oracle."""
    tokens, d = 1 << 26, 8
    g = torch.Generator(device=DEV).manual_seed(W.SEED + 1)
    q = torch.randn((tokens, 1, d), device=DEV, generator=g)
    w = torch.rand(d, device=DEV, generator=g) + 0.5
    pos = torch.randint(0, 8192, (1, tokens), dtype=torch.int32, device=DEV, generator=g)
    inv = W.inv_freq_ladder(1e4, d)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=pos)
    qo, _ = qkr.qk_norm_rope(q, None, w, None, W.EPS, rope)
    assert ":lpr1:" in qkr.last_variant(), qkr.last_variant()
    idx = _sampled_rows(tokens, (1 << 23) * 4, np.random.default_rng(2))
    ti = torch.from_numpy(idx).to(DEV)
    got, qs, ps = host(qo[ti]), host(q[ti]), pos[:, ti].cpu().numpy()
    del q, qo
    torch.cuda.empty_cache()
    ref = oracle.qk_norm_rope(qs, host(w), W.EPS, oracle.Rope("1d", d, "neox", inv_freq=inv, positions=ps), "f32")
    assert_f32_close(got, ref, "tiles past one dispatch")


def test_graph_capture_replays_match_eager():
    case = W.joint(tokens_txt=40, grid=(8, 12), heads=6, seed_stream=31)
    g, rope = joint_gpu(case, "adjacent")
    eager = qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope)
    rows = W.rows(3, seed_stream=31)
    x, wgt = gpu(rows.x), gpu(rows.weight)
    y_eager = qkr.rms_norm(x, wgt, rows.eps)
    outs = [torch.empty_like(t) for t in eager]
    y = torch.empty_like(y_eager)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope, out=outs)
        qkr.rms_norm(x, wgt, rows.eps, out=y)
    for _ in range(3):
        for t in outs + [y]:
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b)
        assert torch.equal(y, y_eager)
        # eager work between replays
        qkr.rms_norm(x, wgt, rows.eps)
        torch.cuda.synchronize()


def test_graph_capture_of_chunked_imrope_vit_and_setup():
    """A chunked IMROPE call (token_base), the fused ViT call over 70 grids
    (three launches) and the ViT setup (two launches) feeding a planes-mode
    apply, captured in one graph: every replay equals the eager results bit
    for bit, with eager work between replays."""
    im = W.imrope(tokens=600, chunk=256, seed_stream=41)
    pos, inv = gpu(torch.from_numpy(im.positions)), gpu(torch.from_numpy(im.inv_freq))
    q, k = gpu(im.q), gpu(im.k)
    wq, wk = gpu(im.q_weight), gpu(im.k_weight)
    rope = qkr.Rope("imrope", 128, "neox", inv_freq=inv, positions=pos, sections=im.sections, token_base=256)
    vt = W.vit(grid_thw=[[1, 4, 4]] * 70, heads=4, seed_stream=41)
    vq, vk, vwq, vwk = gpu(vt.q), gpu(vt.k), gpu(vt.q_weight), gpu(vt.k_weight)
    vinv = [gpu(torch.from_numpy(a_)) for a_ in (vt.inv_t, vt.inv_h, vt.inv_w)]
    half = sum(a_.size for a_ in (vt.inv_t, vt.inv_h, vt.inv_w))
    secs = (vt.inv_t.size, vt.inv_h.size, vt.inv_w.size, 0)
    n = vq.shape[0]

    def run(o):
        qkr.qk_norm_rope(q[256:512], k[256:512], wq, wk, im.eps, rope, q_out=o[0], k_out=o[1])
        qkr.vit_qk_norm_rope(vq, vk, vwq, vwk, 1e-6, *vinv, vt.grid_thw, vt.merge, q_out=o[2], k_out=o[3])
        qkr.mrope_cos_sin_setup(*vinv, vt.grid_thw, vt.merge, out=(o[4], o[5]))
        pr = qkr.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=o[4], sin_planes=o[5])
        qkr.qk_norm_rope(vq, vk, vwq, vwk, 1e-6, pr, q_out=o[6], k_out=o[7])

    def fresh():
        return [torch.empty_like(q[256:512]), torch.empty_like(k[256:512]), torch.empty_like(vq),
                torch.empty_like(vk), torch.zeros((3, n, half), device=DEV), torch.zeros((3, n, half), device=DEV),
                torch.empty_like(vq), torch.empty_like(vk)]

    eager = fresh()
    run(eager)
    outs = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(outs)
    for _ in range(3):
        for i, t in enumerate(outs):
            t.fill_(0.0 if i in (4, 5) else float("nan"))   # setup planes keep unwritten columns
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(outs, eager):
            assert torch.equal(a_, b_)
        whole = qkr.Rope("imrope", 128, "neox", inv_freq=inv, positions=pos, sections=im.sections)
        qkr.qk_norm_rope(q, k, wq, wk, im.eps, whole)         # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# ViT setup folded into the rotation (positions from the grids in the kernel)
# ---------------------------------------------------------------------------

def vit_fused_case(case, pairing="neox"):
    inv = [gpu(torch.from_numpy(a)) for a in (case.inv_t, case.inv_h, case.inv_w)]
    qo, ko = qkr.vit_qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps,
                                  *inv, case.grid_thw, case.merge, pairing)
    rq = oracle.vit_qk_norm_rope(W.as_f32(case.q), W.as_f32(case.q_weight), case.eps, case.inv_t, case.inv_h,
                                 case.inv_w, case.grid_thw, case.merge, pairing)
    rk = oracle.vit_qk_norm_rope(W.as_f32(case.k), W.as_f32(case.k_weight), case.eps, case.inv_t, case.inv_h,
                                 case.inv_w, case.grid_thw, case.merge, pairing)
    return qo, ko, rq, rk


@pytest.mark.parametrize("pairing", ["neox", "adjacent"])
def test_vit_fused_full_size(pairing):
    case = W.vit()
    qo, ko, rq, rk = vit_fused_case(case, pairing)
    assert "vit" in qkr.last_variant()
    assert_bf16_close(host(qo), rq, 2 * case.half_rot, pairing, "vit fused q")
    assert_bf16_close(host(ko), rk, 2 * case.half_rot, pairing, "vit fused k")


def test_vit_fused_many_grids_and_partial_rotary():
    """More grids than one launch carries (several launches over token
    ranges), head_dim 96 with 80 rotary dims, merge 2."""
    rng = np.random.default_rng(41)
    grids = [[int(t), 2 * int(h), 2 * int(w)] for t, h, w in rng.integers(1, 4, (45, 3))]
    case = W.vit(grid_thw=grids, heads=3, head_dim=96, seed_stream=41)
    qo, ko, rq, rk = vit_fused_case(case)
    assert_bf16_close(host(qo), rq, 80, "neox", "q")
    assert_bf16_close(host(ko), rk, 80, "neox", "k")


def test_vit_fused_equals_axes_mode_bitwise():
    """The same rotation through the AXES mode, fed the device-computed ViT
    positions and the concatenated ladders, is the same arithmetic: equal
    bit for bit."""
    case = W.vit(grid_thw=[[1, 16, 16], [2, 8, 12], [1, 6, 6]], seed_stream=42)
    qo, ko, _, _ = vit_fused_case(case)
    pos = qkr.debug_vit_positions(case.grid_thw, case.merge)
    inv = gpu(torch.from_numpy(np.concatenate([case.inv_t, case.inv_h, case.inv_w])))
    secs = (case.inv_t.size, case.inv_h.size, case.inv_w.size, 0)
    rope = qkr.Rope("axes", 2 * case.half_rot, "neox", inv_freq=inv, positions=pos, sections=secs)
    qa, ka = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    assert torch.equal(qo, qa) and torch.equal(ko, ka)


def test_vit_fused_close_to_setup_and_planes():
    case = W.vit(grid_thw=[[1, 16, 16], [2, 8, 12]], seed_stream=43)
    qo, ko, _, _ = vit_fused_case(case)
    n, half = case.n_tokens, case.half_rot
    inv = [gpu(torch.from_numpy(a)) for a in (case.inv_t, case.inv_h, case.inv_w)]
    cos, sin = qkr.mrope_cos_sin_setup(*inv, case.grid_thw, case.merge)
    secs = (case.inv_t.size, case.inv_h.size, case.inv_w.size, 0)
    rope = qkr.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=cos, sin_planes=sin)
    qp, kp = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    assert_bf16_close(host(qo), host(qp), 2 * half)
    assert_bf16_close(host(ko), host(kp), 2 * half)


@pytest.mark.parametrize("dtype,head_dim,rotary_dim,pairing,lpr", [
    ("f32", 40, 40, "neox", 8), ("bf16", 72, 72, "adjacent", 8), ("bf16", 80, 64, "neox", 8),
    ("bf16", 80, 48, "adjacent", 8), ("bf16", 72, 0, "neox", 8), ("f32", 40, 24, "adjacent", 8),
    ("f32", 36, 36, "adjacent", 8), ("bf16", 104, 104, "adjacent", 8), ("bf16", 120, 64, "neox", 8),
    ("f32", 60, 60, "adjacent", 8), ("bf16", 24, 24, "adjacent", 2), ("f32", 20, 20, "adjacent", 4),
])
def test_odd_vector_counts(dtype, head_dim, rotary_dim, pairing, lpr):
    """Rows whose vector count is not a power of two leave lanes without a
    vector of their own, and an odd count leaves one lane a single vector."""
    case = W.tiny(tokens=29, heads=13, head_dim=head_dim, dtype=dtype, seed_stream=head_dim + rotary_dim)
    pos = np.random.default_rng(head_dim).integers(0, 7000, (1, 29)).astype(np.int32)
    # the tile kernel, forced (some of these rows go to token tiles by
    # default), then the default choice
    for variants in (["rope:tile"], []):
        (qo, ko, rq, rk), name = _with_variants(variants, lambda: run_1d(case, pairing, rotary_dim=rotary_dim,
                                                                         positions=pos))
        if variants:
            assert f":lpr{lpr}:" in name, name
        check(qo, rq, dtype, rotary_dim, pairing, f"q {name}")
        check(ko, rk, dtype, rotary_dim, pairing, f"k {name}")


# ---------------------------------------------------------------------------
# staged stores (through LDS, contiguous runs) against direct stores
# ---------------------------------------------------------------------------

def _with_variants(names, fn):
    for nm in names:
        qkr.set_variant_override(nm)
    try:
        out = fn()
        return out, qkr.last_variant()
    finally:
        qkr.set_variant_override(None)


@pytest.mark.parametrize("dtype,head_dim,pairing", [
    ("bf16", 128, "neox"), ("f32", 64, "adjacent"), ("bf16", 80, "neox"), ("f32", 256, "neox"),
])
def test_pass_counts_and_cache_policy_agree_bitwise(dtype, head_dim, pairing):
    """Every passes-per-tile count (1 to 4, so tiles with partial and wholly
    unused passes) with nontemporal accesses on and off gives the same bits;
    the first is also checked against the oracle.  13 heads: ragged passes."""
    case = W.tiny(tokens=37, heads=13, head_dim=head_dim, dtype=dtype, seed_stream=head_dim + 101)
    pos = np.random.default_rng(head_dim + 1).integers(0, 8000, (1, 37)).astype(np.int32)
    ref = None
    for np_ in ("rope:np1", "rope:np2", "rope:np3", "rope:np4"):
        for nt in ("nt:0", "nt:1"):
            (qo, ko, rq, rk), name = _with_variants([np_, nt], lambda: run_1d(case, pairing, positions=pos))
            assert name.startswith(f"rope:np{np_[-1]}:nt{nt[-1]}:"), name
            if ref is None:
                check(qo, rq, dtype, head_dim, pairing, "q")
                check(ko, rk, dtype, head_dim, pairing, "k")
                ref = (qo, ko)
            else:
                assert np.array_equal(qo, ref[0]) and np.array_equal(ko, ref[1]), name


@pytest.mark.parametrize("dtype,head_dim,rotary_dim,pairing,heads", [
    ("bf16", 80, 80, "neox", 16), ("bf16", 80, 34, "adjacent", 5), ("bf16", 96, 64, "neox", 13),
    ("bf16", 48, 48, "adjacent", 26), ("bf16", 112, 112, "neox", 11), ("bf16", 72, 48, "neox", 7),
    ("f32", 40, 40, "adjacent", 16), ("f32", 24, 16, "neox", 26), ("f32", 48, 48, "neox", 13),
    ("bf16", 80, 0, "neox", 9),
])
def test_token_tiles_and_tile_kernel_match_the_oracle(dtype, head_dim, rotary_dim, pairing, heads):
    """Rows whose vector pairs take 3, 5, 6 or 7 lanes run on token tiles
    (one wave per token, Q and K rows together) by default when the token's
    Q and K rows fit 320 vectors.  Token tiles and the tile kernel, each
    forced, with nontemporal accesses on and off, against the oracle; ragged
    passes (13, 11, 7, 9 heads), partial rotary and norm only included."""
    case = W.tiny(tokens=45, heads=heads, head_dim=head_dim, dtype=dtype, seed_stream=head_dim + 211)
    pos = np.random.default_rng(head_dim + 2).integers(0, 8000, (1, 45)).astype(np.int32)
    (_, _, _, _), name = _with_variants([], lambda: run_1d(case, pairing, rotary_dim=rotary_dim, positions=pos))
    nv = head_dim // (8 if dtype == "bf16" else 4)
    fits = (nv + 1) // 2 in (3, 5, 6, 7) and 2 * heads * nv <= 320
    assert name.startswith("rope:token:" if fits else "rope:np"), name
    for variant in ("rope:token", "rope:tile"):
        for nt in ("nt:1", "nt:0"):
            (qo, ko, rq, rk), name = _with_variants(
                [variant, nt], lambda: run_1d(case, pairing, rotary_dim=rotary_dim, positions=pos))
            assert name.startswith("rope:token:" if variant == "rope:token" else "rope:np"), name
            assert f":nt{nt[-1]}:" in name, name
            check(qo, rq, dtype, rotary_dim, pairing, f"q {name}")
            check(ko, rk, dtype, rotary_dim, pairing, f"k {name}")


@pytest.mark.parametrize("dtype,head_dim,rotary_dim,pairing", [
    ("bf16", 80, 80, "neox"), ("bf16", 64, 64, "adjacent"), ("bf16", 96, 64, "neox"),
    ("f32", 40, 40, "adjacent"), ("bf16", 72, 48, "neox"), ("f32", 32, 16, "neox"),
    ("bf16", 128, 128, "neox"), ("bf16", 24, 0, "adjacent"),
])
def test_staged_stores_equal_direct_bitwise(dtype, head_dim, rotary_dim, pairing):
    """Staging changes where results are stored from, never their values."""
    case = W.tiny(tokens=45, heads=11, head_dim=head_dim, dtype=dtype, seed_stream=head_dim + 7)
    pos = np.random.default_rng(head_dim).integers(0, 6000, (1, 45)).astype(np.int32)
    ref = None
    for np_ in ("rope:np1", "rope:np3"):
        for st in ("rope:stage0", "rope:stage1"):
            (qo, ko, rq, rk), name = _with_variants(
                [np_, st], lambda: run_1d(case, pairing, rotary_dim=rotary_dim, positions=pos))
            assert f":stage{st[-1]}" in name, name
            if ref is None:
                ref = (qo, ko)
                check(qo, rq, dtype, rotary_dim, pairing, "q")
                check(ko, rk, dtype, rotary_dim, pairing, "k")
            else:
                assert np.array_equal(qo, ref[0]) and np.array_equal(ko, ref[1]), (np_, st)


def test_joint_head_dim_80_staged():
    """Q, K and copied V rows all leave through the staged path."""
    case = W.joint(tokens_txt=33, grid=(6, 10), heads=5, head_dim=80, axes_pairs=(8, 16, 16), batch=2,
                   seed_stream=8)
    g, rope = joint_gpu(case, "neox")
    outs = {}
    for st in ("rope:stage0", "rope:stage1"):
        (q, k, v), name = _with_variants([st], lambda: qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope))
        assert f":stage{st[-1]}" in name, name
        outs[st] = (q, k, v)
    for a, b in zip(outs["rope:stage0"], outs["rope:stage1"]):
        assert torch.equal(a, b)
    rq, rk, rv = joint_oracle(case, "neox")
    q, k, v = outs["rope:stage1"]
    assert_bf16_close(host(q), rq, 80, "neox", "joint q")
    assert_bf16_close(host(k), rk, 80, "neox", "joint k")
    assert np.array_equal(host(v), rv)


# ---------------------------------------------------------------------------
# residual add + RMSNorm, static FP8 output
# ---------------------------------------------------------------------------

def _fp8_codes(t):
    return t.view(torch.uint8).cpu().numpy()


def test_fp8_encoder_matches_oracle_bitwise():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle.fp8_e4m3_decode(codes).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)   # exact in fp32
    rng = np.random.default_rng(11)
    xs = np.concatenate([vals, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                         rng.uniform(-500, 500, 20000), rng.uniform(-2 ** -5, 2 ** -5, 20000),
                         np.exp2(rng.uniform(-140, 12, 20000)), [0.0, 448.0, 464.0, 1e30, 3.4e38]]).astype(np.float32)
    xs = np.concatenate([xs, -xs])
    got = qkr.debug_fp8_e4m3(gpu(torch.from_numpy(xs))).cpu().numpy()
    assert np.array_equal(got, oracle.fp8_e4m3_encode(xs))


@pytest.mark.parametrize("scale", [0.02, 1.0 / 3.0, 3.7, 0.1, 1e-3, 65.5])
def test_fp8_codes_of_the_kernel_quotient(scale):
    """Codes of the kernel's y / scale (reciprocal, one FMA remainder, one FMA
    correction) equal the codes of the correctly rounded fp32 quotient, on
    values across the range the quotient can take."""
    rng = np.random.default_rng(int(scale * 1e4))
    ys = np.concatenate([rng.normal(0, 3, 200000), np.exp2(rng.uniform(-30, 8, 200000)),
                         rng.uniform(-448 * scale, 448 * scale, 200000)]).astype(np.float32)
    sc = np.float32(scale)
    quo = (ys / sc).astype(np.float32)                       # numpy: correctly rounded fp32 division
    got = qkr.debug_fp8_e4m3(gpu(torch.from_numpy(ys)), gpu(torch.tensor([scale], dtype=torch.float32)))
    ref = oracle.fp8_e4m3_encode(quo)
    assert np.array_equal(got.cpu().numpy(), ref)


def _addrms_case(rows, width, act, seed):
    x = W.to_dtype(W.normal((rows, width), 0.0, 1.0, 41, seed, 0), act)
    r = W.to_dtype(W.normal((rows, width), 0.0, 1.0, 41, seed, 1), act)
    w = W.to_dtype(W.normal((width,), 1.0, 0.1, 41, seed, 2), act)
    return x, r, w


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_row_kernels_cache_policy_agrees_bitwise(act):
    """Every row variant with nontemporal accesses on and off: the plain norm,
    the residual add (both outputs) and the FP8 output give the same bits."""
    # 10 KB rows: one wave per row holds them whole in either type
    x, r, w = _addrms_case(37, 5120 if act == "bf16" else 2560, act, 7)
    scale = gpu(torch.tensor([0.03], dtype=torch.float32))
    for kind in ("rms:rows", "rms:wide", "rms:split"):
        outs = {}
        for nt in ("nt:0", "nt:1"):
            (y, name) = _with_variants([kind, nt], lambda: qkr.rms_norm(gpu(x), gpu(w), 1e-6))
            assert name.startswith(f"{kind}:nt{nt[-1]}:"), name
            (y8n, name), _ = _with_variants([kind, nt], lambda: (qkr.add_rms_norm(
                gpu(x), gpu(w), 1e-6, out_dtype="fp8_e4m3", scale=scale)[0], qkr.last_variant()))
            assert name.startswith(f"{kind}:nt{nt[-1]}:") and name.endswith(":fp8"), name
            outs[nt] = [host(y), _fp8_codes(y8n)]
            if kind == "rms:split":      # the split rows cannot take the residual add
                continue
            gr = gpu(r)
            (ya, s, name), _ = _with_variants([kind, nt], lambda: qkr.add_rms_norm(
                gpu(x), gpu(w), 1e-6, residual=gr) + (qkr.last_variant(),))
            assert name.startswith(f"{kind}:nt{nt[-1]}:") and name.endswith(":add"), name
            gr8 = gpu(r)
            (y8, s8, name), _ = _with_variants([kind, nt], lambda: qkr.add_rms_norm(
                gpu(x), gpu(w), 1e-6, residual=gr8, out_dtype="fp8_e4m3", scale=scale) + (qkr.last_variant(),))
            assert name.startswith(f"{kind}:nt{nt[-1]}:") and name.endswith(":add:fp8"), name
            outs[nt] += [host(ya), host(s), _fp8_codes(y8), host(s8)]
        for a_, b_ in zip(outs["nt:0"], outs["nt:1"]):
            assert np.array_equal(a_, b_), kind


@pytest.mark.parametrize("rows", [1, 7, 300, 4096])
@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("out", ["act", "fp8_e4m3"])
def test_add_rms_norm(rows, act, out):
    width = 5120
    x, r, w = _addrms_case(rows, width, act, rows)
    scale = torch.tensor([0.02], dtype=torch.float32)
    gr = gpu(r)
    y, s = qkr.add_rms_norm(gpu(x), gpu(w), 1e-6, residual=gr, out_dtype=None if out == "act" else out,
                            scale=gpu(scale))
    assert s.data_ptr() == gr.data_ptr()                     # updated in place
    name = qkr.last_variant()
    assert ":add" in name and (":fp8" in name) == (out != "act"), name
    rs, ry = oracle.add_rms_norm(W.as_f32(x), W.as_f32(w), 1e-6, W.as_f32(r), act,
                                 act if out == "act" else out, float(scale[0]))
    assert np.array_equal(host(s), rs), "the residual stream must be bit-exact"
    if out == "act":
        check(host(y), ry, act, what=f"add_rms_norm y {name}")
    else:
        assert_fp8_close(_fp8_codes(y), ry, what=f"add_rms_norm fp8 {name}")


@pytest.mark.parametrize("variant", ["rms:rows", "rms:wide", "rms:split"])
def test_add_rms_norm_variants_and_in_place_on_x(variant):
    """Every row variant that takes the residual add, with the residual
    output written over x; the split rows refuse the add (never swapped for
    another variant) and leave x untouched."""
    x, r, w = _addrms_case(9, 2048, "bf16", 5)
    gx = gpu(x)
    qkr.set_variant_override(variant)
    try:
        if variant == "rms:split":
            with pytest.raises(qkr.QkrError, match="forced variant"):
                qkr.add_rms_norm(gx, gpu(w), 1e-6, residual=gpu(r), residual_out=gx)
            torch.cuda.synchronize()
            assert torch.equal(gx.cpu(), x)
            return
        y, s = qkr.add_rms_norm(gx, gpu(w), 1e-6, residual=gpu(r), residual_out=gx)
        name = qkr.last_variant()
    finally:
        qkr.set_variant_override(None)
    assert name.startswith(variant), name
    rs, ry = oracle.add_rms_norm(W.as_f32(x), W.as_f32(w), 1e-6, W.as_f32(r), "bf16", "bf16")
    assert np.array_equal(host(s), rs) and s.data_ptr() == gx.data_ptr()
    assert_bf16_close(host(y), ry, what=name)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_rms_norm_fp8_without_residual(act):
    x, _, w = _addrms_case(33, 4096, act, 9)
    scale = gpu(torch.tensor([0.05], dtype=torch.float32))
    y, s = qkr.add_rms_norm(gpu(x), gpu(w), 1e-6, out_dtype="fp8_e4m3", scale=scale)
    assert s is None
    _, ry = oracle.add_rms_norm(W.as_f32(x), W.as_f32(w), 1e-6, None, act, "fp8_e4m3", 0.05)
    assert_fp8_close(_fp8_codes(y), ry, what="rms fp8")
    # plain output without residual equals rms_norm bitwise
    y2, _ = qkr.add_rms_norm(gpu(x), gpu(w), 1e-6)
    assert torch.equal(y2, qkr.rms_norm(gpu(x), gpu(w), 1e-6))


def test_add_rms_norm_strided_rows_and_separate_output():
    big = W.to_dtype(W.normal((6, 3 * 1024), 0.0, 1.0, 43), "bf16")
    x, r = big[:, :1024], big[:, 1024:2048]
    w = W.to_dtype(W.normal((1024,), 1.0, 0.1, 44), "bf16")
    gbig = gpu(big)
    sout = torch.empty((6, 1024), dtype=torch.bfloat16, device=DEV)
    y, s = qkr.add_rms_norm(gbig[:, :1024], gpu(w), 1e-6, residual=gbig[:, 1024:2048], residual_out=sout)
    rs, ry = oracle.add_rms_norm(W.as_f32(x), W.as_f32(w), 1e-6, W.as_f32(r), "bf16", "bf16")
    assert np.array_equal(host(s), rs)
    assert_bf16_close(host(y), ry)
    assert torch.equal(gbig[:, 1024:2048].cpu(), r)            # the residual input is untouched


# ---------------------------------------------------------------------------
# K and V written into cache rows picked per token
# ---------------------------------------------------------------------------

def _cache_case(tokens, qh, kvh, d, dtype, seed):
    case = W.tiny(tokens=tokens, heads=qh, head_dim=d, dtype=dtype, seed_stream=seed)
    k = W.to_dtype(W.normal((tokens, kvh, d), 0.0, 1.0, 51, seed, 0), dtype)
    v = W.to_dtype(W.normal((tokens, kvh, d), 0.0, 1.0, 51, seed, 1), dtype)
    pos = np.random.default_rng(seed).integers(0, 8000, (1, tokens)).astype(np.int32)
    inv = W.inv_freq_ladder(1e4, d)
    return case, k, v, pos, inv


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 80)])
def test_cache_write_identity_slots_equal_plain_op(dtype, d):
    case, k, v, pos, inv = _cache_case(57, 8, 2, d, dtype, d)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    kc = torch.full((57, 2, d), float("nan"), dtype=case.q.dtype, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    qo = qkr.qk_norm_rope_cache(gpu(case.q), gpu(k), gpu(v), gpu(case.q_weight), gpu(case.k_weight), kc, vc,
                                gpu(torch.arange(57, dtype=torch.int64)), case.eps, rope)
    pq, pk = qkr.qk_norm_rope(gpu(case.q), gpu(k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    assert torch.equal(qo, pq) and torch.equal(kc, pk) and torch.equal(vc, gpu(v))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_write_paged_sparse_slots(dtype):
    """A paged [blocks, block_size, H, D] cache, an injective random map with
    padding (-1) and out-of-range slots; unmapped rows keep their content."""
    tokens, qh, kvh, d = 300, 16, 8, 128
    case, k, v, pos, inv = _cache_case(tokens, qh, kvh, d, dtype, 77)
    blocks, bs = 40, 16
    num_slots = blocks * bs
    rng = np.random.default_rng(3)
    slots = rng.permutation(num_slots)[:tokens].astype(np.int64)
    slots[rng.choice(tokens, 20, replace=False)] = -1
    slots[[5, 6]] = [num_slots, 1 << 40]
    fill = -3.0
    kc = torch.full((blocks, bs, kvh, d), fill, dtype=case.q.dtype, device=DEV)
    vc = torch.full_like(kc, fill)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    qo = qkr.qk_norm_rope_cache(gpu(case.q), gpu(k), gpu(v), gpu(case.q_weight), gpu(case.k_weight), kc, vc,
                                gpu(torch.from_numpy(slots)), case.eps, rope)
    orope = oracle.Rope("1d", d, "neox", inv_freq=inv, positions=pos)
    kc0 = np.full((num_slots, kvh, d), fill, np.float32)
    rq, rk, rv = oracle.qk_norm_rope_cache(W.as_f32(case.q), W.as_f32(k), W.as_f32(v), W.as_f32(case.q_weight),
                                           W.as_f32(case.k_weight), case.eps, orope, slots, kc0, kc0.copy(), dtype)
    check(host(qo), rq, dtype, d, "neox", "q")
    gk = host(kc).reshape(num_slots, kvh, d)
    mapped = np.zeros(num_slots, bool)
    mapped[slots[(slots >= 0) & (slots < num_slots)]] = True
    assert np.array_equal(gk[~mapped], rk[~mapped])            # untouched rows, exactly
    check(gk[mapped], rk[mapped], dtype, d, "neox", "k cache")
    assert np.array_equal(host(vc).reshape(num_slots, kvh, d), rv)   # V copied bit for bit


@pytest.mark.parametrize("slot_map", ["random", "blocks"])
def test_cache_write_full_size(slot_map):
    """The timed cache-write configurations: 8192 tokens of the IMROPE workload
    (16 Q, 8 K/V heads x 128, bf16) into a paged cache of 2048 blocks x 16
    slots, one launch, through a random injective map of single slots or a
    block-ordered one (16 consecutive tokens per block, blocks in random
    order)."""
    case = W.imrope()
    T, H, KV, D = case.q.shape[0], case.q.shape[1], case.k.shape[1], 128
    blocks, bs = 2048, 16
    v = W.to_dtype(W.normal((T, KV, D), 0.0, 1.0, 61), "bf16")
    if slot_map == "blocks":
        order = np.random.default_rng(61).permutation(blocks)[:T // bs].astype(np.int64)
        slots = order[np.arange(T) // bs] * bs + np.arange(T) % bs
    else:
        slots = np.random.default_rng(61).permutation(blocks * bs)[:T].astype(np.int64)
    kc = torch.zeros((blocks, bs, KV, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    rope = qkr.Rope("imrope", D, "neox", inv_freq=gpu(torch.from_numpy(case.inv_freq)),
                    positions=gpu(torch.from_numpy(case.positions)), sections=case.sections)
    qo = qkr.qk_norm_rope_cache(gpu(case.q), gpu(case.k), gpu(v), gpu(case.q_weight), gpu(case.k_weight), kc, vc,
                                gpu(torch.from_numpy(slots)), case.eps, rope)
    # 16 Q heads fill both passes of a tile, 8 K and 8 V heads only one: with
    # two passes per tile a third of the passes would be idle, so one
    assert qkr.last_variant().startswith("rope:np1:"), qkr.last_variant()
    orope = oracle.Rope("imrope", D, "neox", inv_freq=case.inv_freq, sections=case.sections,
                        positions=case.positions)
    kc0 = np.zeros((blocks * bs, KV, D), np.float32)
    rq, rk, rv = oracle.qk_norm_rope_cache(W.as_f32(case.q), W.as_f32(case.k), W.as_f32(v), W.as_f32(case.q_weight),
                                           W.as_f32(case.k_weight), case.eps, orope, slots, kc0, kc0.copy(), "bf16")
    check(host(qo), rq, "bf16", D, "neox", "q")
    gk = host(kc).reshape(blocks * bs, KV, D)
    mapped = np.zeros(blocks * bs, bool)
    mapped[slots] = True
    assert np.array_equal(gk[~mapped], rk[~mapped])
    check(gk[mapped], rk[mapped], "bf16", D, "neox", "k cache")
    assert np.array_equal(host(vc).reshape(blocks * bs, KV, D), rv)


def test_cache_write_imrope_without_v_and_empty_cache():
    case = W.imrope(tokens=64)
    d = 128
    pos, inv = gpu(torch.from_numpy(case.positions)), gpu(torch.from_numpy(case.inv_freq))
    rope = qkr.Rope("imrope", d, "neox", inv_freq=inv, positions=pos, sections=case.sections)
    slots = torch.arange(64, dtype=torch.int64).flip(0)
    kc = torch.zeros((64, case.k.shape[1], d), dtype=torch.bfloat16, device=DEV)
    qo = qkr.qk_norm_rope_cache(gpu(case.q), gpu(case.k), None, gpu(case.q_weight), gpu(case.k_weight), kc, None,
                                gpu(slots), case.eps, rope)
    pq, pk = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    assert torch.equal(qo, pq) and torch.equal(kc, pk.flip(0))
    empty = torch.zeros((0, case.k.shape[1], d), dtype=torch.bfloat16, device=DEV)
    qo2 = qkr.qk_norm_rope_cache(gpu(case.q), gpu(case.k), None, gpu(case.q_weight), gpu(case.k_weight), empty,
                                 None, gpu(slots), case.eps, rope)
    assert torch.equal(qo2, pq)


# ---------------------------------------------------------------------------
# 64-bit addressing and graph capture of the cache-write and residual-add paths
# ---------------------------------------------------------------------------

def test_cache_write_past_4_gib():
    """Cache rows past 2^31 elements (4 GiB of bf16): 16 tokens mapped to the
    last slots of a 2^21 + 64 slot cache."""
    tokens, qh, kvh, d = 16, 4, 8, 128
    case, k, v, pos, inv = _cache_case(tokens, qh, kvh, d, "bf16", 91)
    num_slots = (1 << 21) + 64                               # 2 KiB per slot
    slots = np.arange(num_slots - tokens, num_slots, dtype=np.int64)[::-1].copy()
    slots[3] = 5                                             # and one near the start
    kc = torch.zeros((num_slots, kvh, d), dtype=torch.bfloat16, device=DEV)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    qkr.qk_norm_rope_cache(gpu(case.q), gpu(k), None, gpu(case.q_weight), gpu(case.k_weight), kc, None,
                           gpu(torch.from_numpy(slots)), case.eps, rope)
    orope = oracle.Rope("1d", d, "neox", inv_freq=inv, positions=pos)
    rk = oracle.qk_norm_rope(W.as_f32(k), W.as_f32(case.k_weight), case.eps, orope)
    got = host(kc[torch.from_numpy(slots).to(DEV)])
    assert_bf16_close(got, rk, d, "neox", "k rows past 4 GiB")
    head = kc[: 1 << 10]                                     # slots 0..1023: only slot 5 is mapped
    assert int(torch.count_nonzero(head)) == int(torch.count_nonzero(head[5])) == kvh * d
    del kc
    torch.cuda.empty_cache()


def test_add_rms_norm_row_offsets_past_4_gib():
    """Rows 2^20 elements apart: the last rows start past 2^32 bytes."""
    rows, width, stride = 2100, 1024, 1 << 20
    x, r, w = _addrms_case(rows, width, "bf16", 13)
    big = torch.empty((rows, stride), dtype=torch.bfloat16, device=DEV)
    big[:, :width].copy_(gpu(x))
    big[:, width:2 * width].copy_(gpu(r))
    xs, rs = big[:, :width], big[:, width:2 * width]
    y, s = qkr.add_rms_norm(xs, gpu(w), 1e-6, residual=rs)
    ref_s, ref_y = oracle.add_rms_norm(W.as_f32(x), W.as_f32(w), 1e-6, W.as_f32(r), "bf16", "bf16")
    assert np.array_equal(host(s), ref_s)
    assert_bf16_close(host(y), ref_y, what="rows past 4 GiB")
    del big
    torch.cuda.empty_cache()


def test_graph_capture_of_cache_write_and_residual_add():
    case, k, v, pos, inv = _cache_case(40, 8, 2, 128, "bf16", 95)
    rope = qkr.Rope("1d", 128, "neox", inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    slots = gpu(torch.from_numpy(np.random.default_rng(95).permutation(64)[:40].astype(np.int64)))
    q, kk, vv, wq, wk = gpu(case.q), gpu(k), gpu(v), gpu(case.q_weight), gpu(case.k_weight)
    x, r, w = (gpu(t) for t in _addrms_case(7, 2048, "bf16", 95))
    scale = gpu(torch.tensor([0.03], dtype=torch.float32))

    def run(kc, vc, qo, res, y8):
        qkr.qk_norm_rope_cache(q, kk, vv, wq, wk, kc, vc, slots, case.eps, rope, q_out=qo)
        res.copy_(r)
        qkr.add_rms_norm(x, w, 1e-6, residual=res, out_dtype="fp8_e4m3", scale=scale, out=y8)

    def fresh():
        return (torch.zeros((64, 2, 128), dtype=torch.bfloat16, device=DEV),
                torch.zeros((64, 2, 128), dtype=torch.bfloat16, device=DEV), torch.empty_like(q),
                torch.empty_like(r), torch.empty(r.shape, dtype=torch.float8_e4m3fn, device=DEV))

    ref = fresh()
    run(*ref)
    got = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*got)
    for _ in range(3):
        got[0].zero_()                                         # cache rows no token maps to stay as they are
        got[1].zero_()
        for t in got[2:]:
            t.view(torch.uint8).fill_(0x55)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        run(*fresh())                                          # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Eager numerics: the rounding points of an eager RMSNorm + RoPE chain
# ([Ovis] "Supplemental eager bitwise measurements"; [VecRMS] review thread)
# ---------------------------------------------------------------------------

def _differs(a, b):
    return float(np.mean(np.asarray(a) != np.asarray(b)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("t,variant", [(1, None), (37, "rms:rows"), (37, "rms:wide"), (37, "rms:split"),
                                       (4096, None)])
def test_eager_rms_norm(dtype, t, variant):
    case = W.rows(t, width=5120 if dtype == "bf16" else 2560, dtype=dtype, seed_stream=300 + t)
    qkr.set_variant_override(variant)
    try:
        y = qkr.rms_norm(gpu(case.x), gpu(case.weight), case.eps, numerics="eager")
        name = qkr.last_variant()
    finally:
        qkr.set_variant_override(None)
    assert name.endswith(":eager") and (variant is None or name.startswith(variant + ":")), name
    ref = oracle.rms_norm(W.as_f32(case.x), W.as_f32(case.weight), case.eps, dtype, numerics="eager")
    check(host(y), ref, dtype, what=f"eager rms {name}")
    if dtype == "bf16" and t > 1:
        contract = qkr.rms_norm(gpu(case.x), gpu(case.weight), case.eps)
        assert _differs(host(y), host(contract)) > 0.05      # a different rounding chain, really taken


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_eager_add_rms_norm(act):
    x, r, w = _addrms_case(300, 5120, act, 77)
    gr = gpu(r)
    y, s = qkr.add_rms_norm(gpu(x), gpu(w), 1e-6, residual=gr, numerics="eager")
    assert qkr.last_variant().endswith(":add:eager"), qkr.last_variant()
    rs, ry = oracle.add_rms_norm(W.as_f32(x), W.as_f32(w), 1e-6, W.as_f32(r), act, act, numerics="eager")
    assert np.array_equal(host(s), rs)
    check(host(y), ry, act, what="eager add_rms_norm")
    with pytest.raises(qkr.QkrError, match="UNSUPPORTED"):
        qkr.add_rms_norm(gpu(x), gpu(w), 1e-6, out_dtype="fp8_e4m3",
                         scale=gpu(torch.tensor([0.02], dtype=torch.float32)), numerics="eager")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("head_dim,pairing", [(128, "neox"), (128, "adjacent"), (64, "neox"), (80, "adjacent")])
def test_eager_qk_norm_rope_1d(dtype, head_dim, pairing):
    case = W.tiny(tokens=61, heads=7, head_dim=head_dim, dtype=dtype, seed_stream=400 + head_dim)
    pos = np.random.default_rng(head_dim + 4).integers(0, 8192, (1, 61)).astype(np.int32)
    inv = W.inv_freq_ladder(1e4, head_dim)
    rope = qkr.Rope("1d", head_dim, pairing, inv_freq=gpu(torch.from_numpy(inv)), positions=gpu(torch.from_numpy(pos)))
    qo, ko = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope,
                              numerics="eager")
    assert qkr.last_variant().endswith(":eager"), qkr.last_variant()
    orope = oracle.Rope("1d", head_dim, pairing, inv_freq=inv, positions=pos)
    for got, x, w, nm in ((qo, case.q, case.q_weight, "q"), (ko, case.k, case.k_weight, "k")):
        ref = oracle.qk_norm_rope(W.as_f32(x), W.as_f32(w), case.eps, orope, dtype, numerics="eager")
        check(host(got), ref, dtype, head_dim, pairing, f"eager {nm}")
    if dtype == "bf16":
        cq, _ = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
        assert _differs(host(qo), host(cq)) > 0.05


@pytest.mark.parametrize("dtype,head_dim,rotary_dim,pairing,heads,mode", [
    ("bf16", 80, 80, "neox", 16, "1d"), ("bf16", 48, 48, "adjacent", 26, "1d"), ("bf16", 112, 112, "neox", 11, "1d"),
    ("bf16", 96, 64, "adjacent", 13, "1d"), ("f32", 24, 16, "neox", 26, "1d"), ("f32", 48, 48, "adjacent", 9, "1d"),
    ("bf16", 80, 0, "neox", 16, "none"), ("f32", 40, 0, "adjacent", 16, "none"),
    ("bf16", 96, 0, "adjacent", 13, "none"), ("bf16", 112, 0, "neox", 11, "none"),
    ("bf16", 80, 80, "neox", 16, "planes"), ("bf16", 96, 96, "adjacent", 12, "planes"),
    ("bf16", 112, 112, "neox", 11, "planes"), ("f32", 40, 40, "neox", 16, "planes"),
])
def test_token_tiles_both_numerics_match_the_oracle(dtype, head_dim, rotary_dim, pairing, heads, mode):
    """Token tiles (3, 5, 6 and 7 lanes per row; rows by LDS DMA for norm
    only and for planes up to 6 lanes, through registers for positions and
    7-lane planes) and the tile kernel, each forced, with the contract and
    with the eager numerics, against the oracle of each; for bf16 the eager
    result differs visibly from the contracted one, so the eager rounding
    points are the ones taken."""
    tokens = 45
    case = W.tiny(tokens=tokens, heads=heads, head_dim=head_dim, dtype=dtype, seed_stream=head_dim + 613)
    rng = np.random.default_rng(head_dim + 9)
    half = rotary_dim // 2
    if mode == "1d":
        pos = rng.integers(0, 8000, (1, tokens)).astype(np.int32)
        inv = W.inv_freq_ladder(1e4, rotary_dim)
        rope = qkr.Rope("1d", rotary_dim, pairing, inv_freq=gpu(torch.from_numpy(inv)),
                        positions=gpu(torch.from_numpy(pos)))
        orope = oracle.Rope("1d", rotary_dim, pairing, inv_freq=inv, positions=pos)
    elif mode == "planes":
        ang = rng.uniform(0, 60, (3, tokens, half))
        cosp, sinp = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
        secs = (half // 4, half // 4, half - 2 * (half // 4), 0)
        rope = qkr.Rope("planes", rotary_dim, pairing, sections=secs, cos_planes=gpu(torch.from_numpy(cosp)),
                        sin_planes=gpu(torch.from_numpy(sinp)))
        orope = oracle.Rope("planes", rotary_dim, pairing, sections=secs, cos_planes=cosp, sin_planes=sinp)
    else:
        rope, orope = None, None
    refs = {n: [oracle.qk_norm_rope(W.as_f32(x), W.as_f32(w), case.eps, orope, dtype, numerics=n)
                for x, w in ((case.q, case.q_weight), (case.k, case.k_weight))] for n in ("contract", "eager")}
    args = (gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, rope)
    for variant in ("rope:token", "rope:tile"):
        (qo, ko), name = _with_variants([variant], lambda: qkr.qk_norm_rope(*args, numerics="eager"))
        assert name.startswith("rope:token:" if variant == "rope:token" else "rope:np"), name
        assert name.endswith(":eager"), name
        check(host(qo), refs["eager"][0], dtype, rotary_dim, pairing, f"eager q {name}")
        check(host(ko), refs["eager"][1], dtype, rotary_dim, pairing, f"eager k {name}")
        (cq, ck), cname = _with_variants([variant], lambda: qkr.qk_norm_rope(*args))
        assert cname + ":eager" == name, (cname, name)
        check(host(cq), refs["contract"][0], dtype, rotary_dim, pairing, f"q {cname}")
        check(host(ck), refs["contract"][1], dtype, rotary_dim, pairing, f"k {cname}")
        if dtype == "bf16":
            assert _differs(host(qo), host(cq)) > 0.05, name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_eager_rotation_is_unfused_bitwise(dtype):
    """Rows of +-1 with eps = 0 normalise exactly (rrms = 1), and planes mode
    hands every kernel the same cos/sin, so the eager output is fixed bit
    for bit by its rounding points: each fp32 product and sum rounded on its
    own.  With fp32 operands a fused multiply-add would change a visible
    share of the results, as the contract path's output shows."""
    tokens, heads, d = 300, 4, 128
    rng = np.random.default_rng(500)
    x = W.to_dtype(rng.choice([-1.0, 1.0], (tokens, heads, d)).astype(np.float32), dtype)
    w = W.to_dtype(rng.normal(1.0, 0.3, d).astype(np.float32), dtype)
    cosp = rng.uniform(-1, 1, (3, tokens, d // 2)).astype(np.float32)
    sinp = rng.uniform(-1, 1, (3, tokens, d // 2)).astype(np.float32)
    secs = (16, 24, 24, 0)
    rope = qkr.Rope("planes", d, "neox", sections=secs, cos_planes=gpu(torch.from_numpy(cosp)),
                    sin_planes=gpu(torch.from_numpy(sinp)))
    eager, _ = qkr.qk_norm_rope(gpu(x), None, gpu(w), None, 0.0, rope, numerics="eager")
    contract, _ = qkr.qk_norm_rope(gpu(x), None, gpu(w), None, 0.0, rope)
    orope = oracle.Rope("planes", d, "neox", sections=secs, cos_planes=cosp, sin_planes=sinp)
    ref = oracle.qk_norm_rope(W.as_f32(x), W.as_f32(w), 0.0, orope, dtype, numerics="eager")
    assert np.array_equal(host(eager), ref)
    if dtype == "f32":
        assert _differs(host(contract), ref) > 0.01


def test_eager_imrope_full_size_chunked():
    case = W.imrope()
    pos, inv = gpu(torch.from_numpy(case.positions)), gpu(torch.from_numpy(case.inv_freq))
    q, k = gpu(case.q), gpu(case.k)
    outs = []
    for b in range(0, 8192, case.chunk):
        rope = qkr.Rope("imrope", 128, "neox", inv_freq=inv, positions=pos, sections=case.sections, token_base=b)
        outs.append(qkr.qk_norm_rope(q[b:b + case.chunk], k[b:b + case.chunk], gpu(case.q_weight),
                                     gpu(case.k_weight), case.eps, rope, numerics="eager"))
    orope = oracle.Rope("imrope", 128, "neox", inv_freq=case.inv_freq, sections=case.sections,
                        positions=case.positions)
    for i, (x, w, nm) in enumerate(((case.q, case.q_weight, "q"), (case.k, case.k_weight, "k"))):
        got = torch.cat([o[i] for o in outs])
        ref = oracle.qk_norm_rope(W.as_f32(x), W.as_f32(w), case.eps, orope, "bf16", numerics="eager")
        assert_bf16_close(host(got), ref, 128, "neox", f"eager imrope {nm}")


@pytest.mark.parametrize("pairing", ["adjacent", "neox"])
def test_eager_joint_full_size(pairing):
    case = W.joint()
    g, rope = joint_gpu(case, pairing)
    q, k, v = qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope, numerics="eager")
    hd = case.head_dim

    def stream(s):
        return {"q": W.as_f32(s.view(0, case.heads, hd)), "k": W.as_f32(s.view(1, case.heads, hd)),
                "v": W.as_f32(s.view(2, case.heads, hd)), "q_weight": W.as_f32(s.q_weight),
                "k_weight": W.as_f32(s.k_weight)}

    orope = oracle.Rope("axes", hd, pairing, inv_freq=case.inv_freq, sections=case.sections, positions=case.positions)
    rq, rk, rv = oracle.joint_qk_norm_rope(stream(case.text), stream(case.image), case.eps, orope, "bf16",
                                           numerics="eager")
    assert_bf16_close(host(q), rq, 128, pairing, "eager joint q")
    assert_bf16_close(host(k), rk, 128, pairing, "eager joint k")
    assert np.array_equal(host(v), rv)


def test_eager_vit_fused_and_cache_write():
    case = W.vit()
    inv = [gpu(torch.from_numpy(a)) for a in (case.inv_t, case.inv_h, case.inv_w)]
    qo, ko = qkr.vit_qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, *inv,
                                  case.grid_thw, case.merge, numerics="eager")
    for got, x, w, nm in ((qo, case.q, case.q_weight, "q"), (ko, case.k, case.k_weight, "k")):
        ref = oracle.vit_qk_norm_rope(W.as_f32(x), W.as_f32(w), case.eps, case.inv_t, case.inv_h, case.inv_w,
                                      case.grid_thw, case.merge, numerics="eager")
        assert_bf16_close(host(got), ref, 2 * case.half_rot, "neox", f"eager vit {nm}")
    tokens, qh, kvh, d = 300, 16, 8, 128
    cc, k, v, pos, inv1 = _cache_case(tokens, qh, kvh, d, "bf16", 501)
    slots = np.random.default_rng(501).permutation(640)[:tokens].astype(np.int64)
    kc = torch.zeros((640, kvh, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    rope = qkr.Rope("1d", d, "neox", inv_freq=gpu(torch.from_numpy(inv1)), positions=gpu(torch.from_numpy(pos)))
    q_out = qkr.qk_norm_rope_cache(gpu(cc.q), gpu(k), gpu(v), gpu(cc.q_weight), gpu(cc.k_weight), kc, vc,
                                   gpu(torch.from_numpy(slots)), cc.eps, rope, numerics="eager")
    orope = oracle.Rope("1d", d, "neox", inv_freq=inv1, positions=pos)
    rq, rk, rv = oracle.qk_norm_rope_cache(W.as_f32(cc.q), W.as_f32(k), W.as_f32(v), W.as_f32(cc.q_weight),
                                           W.as_f32(cc.k_weight), cc.eps, orope, slots,
                                           np.zeros((640, kvh, d), np.float32), np.zeros((640, kvh, d), np.float32),
                                           "bf16", numerics="eager")
    assert_bf16_close(host(q_out), rq, d, "neox", "eager cache q")
    assert_bf16_close(host(kc)[slots], rk[slots], d, "neox", "eager cache k")
    assert np.array_equal(host(vc), rv)


@pytest.mark.parametrize("mode", ["1d", "imrope"])
@pytest.mark.parametrize("numerics", ["contract", "eager"])
def test_rounding_points_decide_the_bits(mode, numerics):
    """On the elements whose bf16 value depends on where the kernel rounds,
    the GPU takes the oracle's value for its numerics: not the value of a
    rotation of the unrounded normalised row ([Ovis] kernel review: the
    normalised value is rounded before the rotation), and not the other
    preset's value (x * rrms rounded before the weight, cos/sin in the
    activation type, no fused multiply-add)."""
    from test_parity_rules import _bf16, _case, _rotate
    case, x, w, rope, theta = _case(mode)
    extra = {"sections": case.sections} if mode == "imrope" else {}
    gr = qkr.Rope(mode, 128, "neox", inv_freq=gpu(torch.from_numpy(case.inv_freq)),
                  positions=gpu(torch.from_numpy(case.positions if mode == "imrope" else case.positions[:1])),
                  **extra)
    q, _ = qkr.qk_norm_rope(gpu(case.q), gpu(case.k), gpu(case.q_weight), gpu(case.k_weight), case.eps, gr,
                            numerics=numerics)
    got = host(q)
    ref = oracle.qk_norm_rope(x, w, case.eps, rope, "bf16", numerics=numerics)
    other = oracle.qk_norm_rope(x, w, case.eps, rope, "bf16",
                                numerics="eager" if numerics == "contract" else "contract")
    unrounded = _rotate(oracle.qk_norm_rope(x, w, case.eps, None, "f32"), theta, np.float64)
    assert_bf16_close(got, ref, 128, "neox", f"{mode} {numerics}")
    for name, slip in (("unrounded normalised value", unrounded), ("the other numerics", other)):
        d = ref != slip                                   # elements that tell the two apart
        assert d.mean() > 0.05, (name, d.mean())          # enough of them to decide
        took_ref = (got[d] == ref[d]).mean()
        took_slip = (got[d] == slip[d]).mean()
        assert took_ref > 0.995 and took_slip < 0.005, (name, d.sum(), took_ref, took_slip)
