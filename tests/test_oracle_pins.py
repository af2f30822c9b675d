"""Pins of the CPU oracle against things other than itself (CPU only).

Every expected value here is fixed by something independent of the oracle's
code: a closed form, an invariant of the mathematics, a library routine on a
special case, or a fixture under tests/golden/ written out by hand from the
pages.  Each test is chosen so that a plausible slip in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a missed offset) fails it.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import inv_freq_ladder

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(k):
    return np.random.default_rng([7, k])


# ----------------------------------------------------------------------------
# bf16 rounding
# ----------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_float32_values():
    """torch's float32 -> bfloat16 cast rounds to nearest even.  For inputs that
    are exactly float32, rounding the real value once to bf16 is the same
    operation, so the two must agree bit for bit, ties included."""
    rng = _rng(1)
    normal = rng.normal(0.0, 1.0, 4000)
    wide = rng.normal(0.0, 1.0, 2000) * np.exp2(rng.integers(-140, 126, 2000))
    # exact ties: a bf16 value plus half its spacing
    b = torch.from_numpy(rng.normal(0, 1, 2000).astype(np.float32)).to(torch.bfloat16)
    b = b.float().numpy().astype(np.float64)
    _, e = np.frexp(b)
    ties = b + np.ldexp(0.5, e - 8)
    edge = np.array([3.0e38, -3.3e38, np.float32(3.4028235e38), 1e-40, -1e-44, 0.0, -0.0])
    x = np.concatenate([normal, wide, ties, edge]).astype(np.float32)
    expect = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, expect, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(expect))


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("c", [0.5, -3.0, 1e-3, 7.25])
def test_rms_norm_constant_row_closed_form(c):
    """x_i = c for every i: mean(x^2) = c^2, so y_i = c / sqrt(c^2 + eps) * w_i."""
    width = 96
    eps = np.float32(1e-2)
    w = _rng(2).normal(1.0, 0.1, width).astype(np.float32)
    y = oracle.rms_norm(np.full((1, width), c, np.float32), w, float(eps), "f32")
    expect = c / np.sqrt(c * c + np.float64(eps)) * w.astype(np.float64)
    np.testing.assert_allclose(y[0], expect, rtol=1.5e-7, atol=0)


@pytest.mark.parametrize("width", [1, 7, 64, 5120])
def test_rms_norm_output_has_unit_rms_without_eps(width):
    """With eps = 0 the weight-divided output has root mean square exactly 1,
    whatever the row."""
    rng = _rng(3)
    x = rng.normal(0.0, 2.0, (5, width)).astype(np.float32)
    w = rng.normal(1.0, 0.1, width).astype(np.float32)
    y = oracle.rms_norm(x, w, 0.0, "f32")
    r = np.sqrt(np.mean((y.astype(np.float64) / w) ** 2, axis=1))
    np.testing.assert_allclose(r, 1.0, rtol=3e-7)


def test_rms_norm_scale_invariant_without_eps():
    """Scaling a row by a power of two changes no output bit when eps = 0."""
    rng = _rng(4)
    x = rng.normal(0.0, 1.0, (3, 256)).astype(np.float32)
    w = rng.normal(1.0, 0.1, 256).astype(np.float32)
    for dt in ("f32", "bf16"):
        a = oracle.rms_norm(x, w, 0.0, dt)
        b = oracle.rms_norm(x * np.float32(8.0), w, 0.0, dt)
        assert np.array_equal(a, b)


def test_rms_norm_bf16_output_is_on_bf16_grid_and_close():
    rng = _rng(5)
    x = rng.normal(0.0, 1.0, (4, 5120)).astype(np.float32)
    w = rng.normal(1.0, 0.1, 5120).astype(np.float32)
    y32 = oracle.rms_norm(x, w, 1e-6, "f32")
    y16 = oracle.rms_norm(x, w, 1e-6, "bf16")
    grid = torch.from_numpy(y16).to(torch.bfloat16).float().numpy()
    assert np.array_equal(grid, y16)
    assert np.max(np.abs(y16 - y32) / np.abs(y32)) <= 2.0 ** -8


# ----------------------------------------------------------------------------
# Rotation
# ----------------------------------------------------------------------------

def _rope_1d(positions, inv_freq, rotary_dim, pairing="neox", token_base=0):
    return oracle.Rope("1d", rotary_dim, pairing, inv_freq=inv_freq,
                       positions=np.asarray(positions, np.int32).reshape(1, -1),
                       token_base=token_base)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("pairing", ["neox", "adjacent"])
def test_position_zero_is_identity(out, pairing):
    """At position 0 every angle is 0 (cos 1, sin 0): the output is the
    norm-only output, bit for bit."""
    rng = _rng(6)
    x = rng.normal(0, 1, (3, 4, 64)).astype(np.float32)
    w = rng.normal(1, 0.1, 64).astype(np.float32)
    rope = _rope_1d(np.zeros(3), inv_freq_ladder(1e4, 64), 64, pairing)
    assert np.array_equal(oracle.qk_norm_rope(x, w, 1e-6, rope, out),
                          oracle.qk_norm_rope(x, w, 1e-6, None, out))


@pytest.mark.parametrize("pairing", ["neox", "adjacent"])
@pytest.mark.parametrize("rotary_dim", [64, 32])
def test_rotation_is_complex_multiplication(pairing, rotary_dim):
    """Rotating pair (a, b) by theta is multiplying a + ib by exp(i theta)
    (numpy's complex exponential).  NeoX pairs element p with p + R/2, the
    adjacent pairing 2p with 2p + 1; theta = fl32(fl32(pos) * inv_freq[p]);
    elements at or past R pass through."""
    rng = _rng(7)
    tokens, heads, d = 5, 3, 64
    x = rng.normal(0, 1, (tokens, heads, d)).astype(np.float32)
    w = rng.normal(1, 0.1, d).astype(np.float32)
    pos = rng.integers(0, 9000, tokens).astype(np.int32)
    inv = inv_freq_ladder(1e4, rotary_dim)
    out = oracle.qk_norm_rope(x, w, 1e-6, _rope_1d(pos, inv, rotary_dim, pairing), "f32")
    n = oracle.qk_norm_rope(x, w, 1e-6, None, "f32").astype(np.float64)
    theta = (pos.astype(np.float32)[:, None] * inv[None, :]).astype(np.float32)
    rot = np.exp(1j * theta.astype(np.float64))[:, None, :]
    half = rotary_dim // 2
    if pairing == "neox":
        i, j = np.arange(half), np.arange(half) + half
    else:
        i, j = 2 * np.arange(half), 2 * np.arange(half) + 1
    z = (n[..., i] + 1j * n[..., j]) * rot
    np.testing.assert_allclose(out[..., i], z.real, atol=2e-6, rtol=0)
    np.testing.assert_allclose(out[..., j], z.imag, atol=2e-6, rtol=0)
    np.testing.assert_allclose(out[..., rotary_dim:], n[..., rotary_dim:], atol=0, rtol=1e-7)


def test_relative_position_property():
    """<R(m) q, R(n) k> = <R(m - n) q, k>: the score depends only on the
    position difference.  inv_freq and positions are chosen so that every fp32
    angle product is exact."""
    rng = _rng(8)
    d = 64
    p = np.arange(d // 2)
    inv = ((1.0 + (p % 16) / 16.0) * np.exp2(-(p // 16))).astype(np.float32)
    q = rng.normal(0, 1, (1, 1, d)).astype(np.float32)
    k = rng.normal(0, 1, (1, 1, d)).astype(np.float32)
    w = rng.normal(1, 0.1, d).astype(np.float32)
    for pairing in ("neox", "adjacent"):
        def rot(x, pos):
            return oracle.qk_norm_rope(x, w, 1e-6, _rope_1d([pos], inv, d, pairing), "f32")[0, 0]
        for m, n in [(5, 3), (300, 17), (2, 40), (511, 0)]:
            a = np.dot(rot(q, m).astype(np.float64), rot(k, n))
            b = np.dot(rot(q, m - n).astype(np.float64), rot(k, 0))
            assert abs(a - b) <= 1e-5 * (1 + abs(a))


# ----------------------------------------------------------------------------
# Position axis maps
# ----------------------------------------------------------------------------

def _golden_imrope_cases():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "imrope_axes.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"sections": tuple(int(v) for v in tok[1:5]), "pairs": int(tok[6]), "axes": {}}
            cases.append(cur)
            continue
        idx = []
        for item in tok[1:]:
            if ":" in item:
                a, b, s = (int(v) for v in item.split(":"))
                idx += list(range(a, b, s))
            else:
                idx.append(int(item))
        cur["axes"]["thwe".index(tok[0])] = idx
    return cases


@pytest.mark.parametrize("case", _golden_imrope_cases(), ids=lambda c: str(c["sections"]))
def test_imrope_axis_map_matches_hand_derived_table(case):
    expect = np.full(case["pairs"], -1)
    for axis, pairs in case["axes"].items():
        expect[pairs] = axis
    assert (expect >= 0).all(), "fixture must cover every pair"
    rope = oracle.Rope("imrope", 2 * case["pairs"], sections=case["sections"])
    assert np.array_equal(oracle.axis_map(rope, case["pairs"]), expect)


def test_imrope_counts_for_24_20_20():
    rope = oracle.Rope("imrope", 128, sections=(24, 20, 20, 0))
    ax = oracle.axis_map(rope, 64)
    assert np.bincount(ax, minlength=4).tolist() == [22, 20, 20, 2]
    assert np.nonzero(ax == 3)[0].tolist() == [61, 62]


def test_axes_map_is_contiguous_runs():
    rope = oracle.Rope("axes", 128, sections=(8, 28, 28, 0))
    assert np.array_equal(oracle.axis_map(rope, 64), np.repeat([0, 1, 2], [8, 28, 28]))


def _imrope_setup(seed, tokens=37, heads=3, d=128):
    rng = _rng(seed)
    x = rng.normal(0, 1, (tokens, heads, d)).astype(np.float32)
    w = rng.normal(1, 0.1, d).astype(np.float32)
    pos = rng.integers(0, 8192, (4, tokens)).astype(np.int32)
    return x, w, pos, inv_freq_ladder(1e6, d)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_imrope_collapses_to_plain_rope(out):
    """All pairs on e ([0, 0, 0, R/2]) is plain RoPE over plane e; any sections
    with four equal planes is plain RoPE over that plane."""
    x, w, pos, inv = _imrope_setup(9)
    all_e = oracle.Rope("imrope", 128, inv_freq=inv, sections=(0, 0, 0, 64), positions=pos)
    assert np.array_equal(oracle.qk_norm_rope(x, w, 1e-6, all_e, out),
                          oracle.qk_norm_rope(x, w, 1e-6, _rope_1d(pos[3], inv, 128), out))
    same = np.repeat(pos[1:2], 4, axis=0)
    sect = oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0), positions=same)
    assert np.array_equal(oracle.qk_norm_rope(x, w, 1e-6, sect, out),
                          oracle.qk_norm_rope(x, w, 1e-6, _rope_1d(pos[1], inv, 128), out))


def test_imrope_non_collapsing_differs_from_plain_rope():
    """Sections that leave pairs on several axes, with independent planes, must
    not reproduce plain RoPE over any single plane."""
    x, w, pos, inv = _imrope_setup(10)
    sect = oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0), positions=pos)
    got = oracle.qk_norm_rope(x, w, 1e-6, sect, "f32")
    for plane in range(4):
        plain = oracle.qk_norm_rope(x, w, 1e-6, _rope_1d(pos[plane], inv, 128), "f32")
        assert np.max(np.abs(got - plain)) > 0.1


def test_imrope_pair_reads_its_own_plane():
    """Change only plane h at one token: exactly the pairs the fixture puts on
    h change, at that token only."""
    x, w, pos, inv = _imrope_setup(11)
    rope = oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0), positions=pos)
    base = oracle.qk_norm_rope(x, w, 1e-6, rope, "f32")
    pos2 = pos.copy()
    pos2[1, 5] += 1
    rope2 = oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0), positions=pos2)
    diff = oracle.qk_norm_rope(x, w, 1e-6, rope2, "f32") != base
    tok, _, elem = np.nonzero(diff)
    assert set(tok.tolist()) == {5}
    pairs = sorted(set((elem % 64).tolist()))
    assert pairs == list(range(1, 60, 3))


def test_chunked_launch_equals_one_launch():
    """A call over tokens [b, b + L) with token_base b, reading the whole-length
    planes, reproduces those rows of the single call; reading the planes as if
    they started at the chunk (the bug class the IMROPE page reports) does
    not."""
    x, w, pos, inv = _imrope_setup(12, tokens=64)
    full = oracle.qk_norm_rope(
        x, w, 1e-6, oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0),
                                positions=pos), "bf16")
    for b in (0, 16, 32, 48):
        rope = oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0),
                           positions=pos, token_base=b)
        assert np.array_equal(oracle.qk_norm_rope(x[b:b + 16], w, 1e-6, rope, "bf16"),
                              full[b:b + 16])
    wrong = oracle.Rope("imrope", 128, inv_freq=inv, sections=(24, 20, 20, 0), positions=pos)
    assert not np.array_equal(oracle.qk_norm_rope(x[16:32], w, 1e-6, wrong, "bf16"), full[16:32])


# ----------------------------------------------------------------------------
# Joint text/image op
# ----------------------------------------------------------------------------

def _joint_inputs(seed, batch=2, st=5, si=12, heads=3, d=64, grid=(3, 4)):
    rng = _rng(seed)

    def stream(n):
        return {"q": rng.normal(0, 1, (batch, n, heads, d)).astype(np.float32),
                "k": rng.normal(0, 1, (batch, n, heads, d)).astype(np.float32),
                "v": rng.normal(0, 1, (batch, n, heads, d)).astype(np.float32),
                "q_weight": rng.normal(1, 0.1, d).astype(np.float32),
                "k_weight": rng.normal(1, 0.1, d).astype(np.float32)}

    txt, img = stream(st), stream(si)
    pos = np.zeros((3, st + si), np.int32)
    k = np.arange(si)
    pos[1, st:] = k // grid[1]
    pos[2, st:] = k % grid[1]
    inv = np.concatenate([inv_freq_ladder(1e4, 8), inv_freq_ladder(1e4, 28), inv_freq_ladder(1e4, 28)])
    rope = oracle.Rope("axes", d, "adjacent", inv_freq=inv, sections=(4, 14, 14, 0), positions=pos)
    return txt, img, rope, pos, inv


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_joint_is_text_first_concat_of_streams(out):
    txt, img, rope, pos, inv = _joint_inputs(13)
    st = txt["q"].shape[1]
    q, k, v = oracle.joint_qk_norm_rope(txt, img, 1e-6, rope, out)
    # V is routed unchanged, text first.
    assert np.array_equal(v, np.concatenate([txt["v"], img["v"]], axis=1))
    for b in range(q.shape[0]):
        # text rows sit at position (0, 0, 0): norm-only with the text weights
        assert np.array_equal(q[b, :st], oracle.qk_norm_rope(txt["q"][b], txt["q_weight"], 1e-6, None, out))
        assert np.array_equal(k[b, :st], oracle.qk_norm_rope(txt["k"][b], txt["k_weight"], 1e-6, None, out))
        # image rows: the image stream with its own weights at joint positions
        r = oracle.Rope("axes", rope.rotary_dim, "adjacent", inv_freq=inv, sections=(4, 14, 14, 0),
                        positions=pos, token_base=st)
        assert np.array_equal(q[b, st:], oracle.qk_norm_rope(img["q"][b], img["q_weight"], 1e-6, r, out))
        assert np.array_equal(k[b, st:], oracle.qk_norm_rope(img["k"][b], img["k_weight"], 1e-6, r, out))


def test_joint_t_axis_pairs_of_image_rows_are_unrotated():
    """Image positions are (0, row, col): the t-axis pairs see angle 0 and keep
    their normalised values."""
    txt, img, rope, pos, inv = _joint_inputs(14, batch=1)
    st = txt["q"].shape[1]
    q, _, _ = oracle.joint_qk_norm_rope(txt, img, 1e-6, rope, "f32")
    n = oracle.qk_norm_rope(img["q"][0], img["q_weight"], 1e-6, None, "f32")
    t_elems = np.arange(8)            # adjacent pairs 0..3 -> elements 0..7
    assert np.array_equal(q[0, st:][..., t_elems], n[..., t_elems])
    assert not np.array_equal(q[0, st:][..., 8:], n[..., 8:])


# ----------------------------------------------------------------------------
# ViT positions and planes
# ----------------------------------------------------------------------------

def test_vit_positions_match_hand_derived_fixture():
    rows = np.loadtxt(os.path.join(GOLDEN, "vit_positions.txt"), dtype=np.int64)
    pos = oracle.vit_positions([[1, 4, 6], [2, 2, 4]], 2)
    assert pos.shape == (3, rows.shape[0])
    assert np.array_equal(pos.T, rows[:, 1:])


def test_vit_positions_merge_one_is_raster_order():
    grids = [[2, 3, 5], [1, 4, 4]]
    pos = oracle.vit_positions(grids, 1)
    expect = []
    for t, h, w in grids:
        n = np.arange(t * h * w)
        expect.append(np.stack([n // (h * w), (n % (h * w)) // w, n % w]))
    assert np.array_equal(pos, np.concatenate(expect, axis=1))


def _merge_permuted_ids(t, h, w, m):
    """The ViT position-id permute written as array reshapes: lay (row, col) ids
    on the h x w grid, cut it into m x m blocks, order blocks row-major and the
    cells inside each block row-major."""
    hh = np.broadcast_to(np.arange(h)[:, None], (h, w))
    ww = np.broadcast_to(np.arange(w)[None, :], (h, w))

    def permute(a):
        return a.reshape(h // m, m, w // m, m).transpose(0, 2, 1, 3).reshape(-1)

    frame = np.stack([permute(hh), permute(ww)])
    tt = np.repeat(np.arange(t), h * w)
    return np.concatenate([tt[None], np.tile(frame, (1, t))])


def test_vit_positions_match_block_permute_on_workload_grids():
    grids = [[1, 64, 64], [2, 32, 48], [1, 28, 28]]
    pos = oracle.vit_positions(grids, 2)
    expect = np.concatenate([_merge_permuted_ids(t, h, w, 2) for t, h, w in grids], axis=1)
    assert np.array_equal(pos, expect)


def test_vit_positions_are_a_bijection_per_frame():
    grids = [[3, 6, 4], [1, 8, 10]]
    pos = oracle.vit_positions(grids, 2)
    start = 0
    for t, h, w in grids:
        for f in range(t):
            sl = slice(start + f * h * w, start + (f + 1) * h * w)
            assert (pos[0, sl] == f).all()
            cells = set(zip(pos[1, sl].tolist(), pos[2, sl].tolist()))
            assert cells == {(i, j) for i in range(h) for j in range(w)}
        start += t * h * w


def test_vit_planes_invariants():
    grids = [[1, 8, 8], [2, 4, 6]]
    inv_t, inv_h, inv_w = inv_freq_ladder(1e4, 16), inv_freq_ladder(1e4, 32), inv_freq_ladder(1e4, 32)
    cos, sin = oracle.vit_cos_sin(inv_t, inv_h, inv_w, grids, 2)
    own = [slice(0, 8), slice(8, 24), slice(24, 40)]
    for a in range(3):
        c, s = cos[a][:, own[a]].astype(np.float64), sin[a][:, own[a]].astype(np.float64)
        np.testing.assert_allclose(c * c + s * s, 1.0, atol=3e-7)
        rest = np.ones(40, bool)
        rest[own[a]] = False
        assert np.isnan(cos[a][:, rest]).all() and np.isnan(sin[a][:, rest]).all()
    # frame 0 of grid 0 has t = 0: its t columns are exactly (1, 0)
    assert (cos[0, :64, :8] == 1.0).all() and (sin[0, :64, :8] == 0.0).all()


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_vit_planes_apply_equals_axes_rope_from_positions(out):
    """Rotating with the setup's planes is rotating with the ViT positions in
    AXES mode over the concatenated per-axis inv_freq: the two routes differ
    only by the planes' fp32 rounding of cos and sin."""
    grids = [[1, 8, 8], [2, 4, 6]]
    inv = [inv_freq_ladder(1e4, 16), inv_freq_ladder(1e4, 32), inv_freq_ladder(1e4, 32)]
    cos, sin = oracle.vit_cos_sin(*inv, grids, 2)
    pos = oracle.vit_positions(grids, 2)
    rng = _rng(15)
    n = pos.shape[1]
    x = rng.normal(0, 1, (n, 4, 80)).astype(np.float32)
    w = rng.normal(1, 0.1, 80).astype(np.float32)
    planes = oracle.Rope("planes", 80, sections=(8, 16, 16, 0), cos_planes=cos, sin_planes=sin)
    axes = oracle.Rope("axes", 80, inv_freq=np.concatenate(inv), sections=(8, 16, 16, 0),
                       positions=pos)
    a = oracle.qk_norm_rope(x, w, 1e-6, planes, out)
    b = oracle.qk_norm_rope(x, w, 1e-6, axes, out)
    if out == "f32":
        np.testing.assert_allclose(a, b, atol=1e-6, rtol=0)
    else:
        # at most one bf16 step apart, measured against the pair's magnitude
        assert np.max(np.abs(a - b)) <= 2.0 ** -7 * np.max(np.abs(b))
        assert np.mean(a == b) > 0.99


@pytest.mark.parametrize("pairing", ["neox", "adjacent"])
def test_bf16_contract_rounds_normalised_value_then_result(pairing):
    """bf16 contract: the rotation acts on the bf16-rounded normalised value
    and its result is rounded once.  Rebuild that from the norm-only bf16
    output with numpy's complex exponential and round with torch's cast; the
    double-precision results agree except on exact ties."""
    rng = _rng(16)
    tokens, heads, d = 9, 4, 128
    x = rng.normal(0, 1, (tokens, heads, d)).astype(np.float32)
    w = rng.normal(1, 0.1, d).astype(np.float32)
    pos = rng.integers(0, 8192, tokens).astype(np.int32)
    inv = inv_freq_ladder(1e4, d)
    got = oracle.qk_norm_rope(x, w, 1e-6, _rope_1d(pos, inv, d, pairing), "bf16")
    n = oracle.qk_norm_rope(x, w, 1e-6, None, "bf16").astype(np.float64)
    theta = (pos.astype(np.float32)[:, None] * inv[None, :]).astype(np.float32)
    rot = np.exp(1j * theta.astype(np.float64))[:, None, :]
    half = d // 2
    i, j = ((np.arange(half), np.arange(half) + half) if pairing == "neox"
            else (2 * np.arange(half), 2 * np.arange(half) + 1))
    z = (n[..., i] + 1j * n[..., j]) * rot
    expect = np.empty_like(n)
    expect[..., i], expect[..., j] = z.real, z.imag
    # float64 -> float32 -> bf16 could double-round; only ties of the float32
    # step matter and they are vanishingly rare for these values.
    expect = torch.from_numpy(expect.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.mean(got != expect) < 1e-3


# ----------------------------------------------------------------------------
# ViT setup and rotation in one step
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("pairing", ["neox", "adjacent"])
def test_vit_fused_equals_setup_then_planes_apply(pairing):
    """Computing each token's positions from the grids inside the rotation
    equals writing the cos/sin planes and rotating with them, up to the
    planes' fp32 rounding of cos and sin."""
    grids = [[1, 8, 8], [2, 4, 6], [1, 2, 2]]
    # distinct h and w ladders, so a mix-up of the two axes shows
    inv = [inv_freq_ladder(1e4, 16), inv_freq_ladder(1e4, 32), inv_freq_ladder(2e3, 32)]
    cos, sin = oracle.vit_cos_sin(*inv, grids, 2)
    rng = _rng(17)
    n = cos.shape[1]
    x = rng.normal(0, 1, (n, 3, 96)).astype(np.float32)      # 80 rotary dims + 16 pass-through
    w = rng.normal(1, 0.1, 96).astype(np.float32)
    planes = oracle.Rope("planes", 80, pairing, sections=(8, 16, 16, 0), cos_planes=cos, sin_planes=sin)
    a = oracle.qk_norm_rope(x, w, 1e-6, planes, "f32")
    b = oracle.vit_qk_norm_rope(x, w, 1e-6, *inv, grids, 2, pairing, "f32")
    np.testing.assert_allclose(b, a, atol=1e-6, rtol=0)
    # frame 0 of grid 0 has t = 0: its t pairs keep their normalised values
    nrm = oracle.qk_norm_rope(x, w, 1e-6, None, "f32")
    # elements of the 8 t pairs: NeoX p and p + 40, adjacent 2p and 2p + 1
    t_elems = np.concatenate([np.arange(8), 40 + np.arange(8)]) if pairing == "neox" else np.arange(16)
    assert np.array_equal(b[:64][..., t_elems], nrm[:64][..., t_elems])
    assert np.array_equal(b[..., 80:], nrm[..., 80:])


# ---------------------------------------------------------------------------
# residual add + RMSNorm, static FP8 E4M3 output
# ---------------------------------------------------------------------------

def _fp8_torch(values):
    """torch's float -> float8_e4m3fn conversion (round half to even) of
    values inside the finite range."""
    t = torch.tensor(np.asarray(values, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_every_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.fp8_e4m3_decode(codes)
    assert np.array_equal(oracle.fp8_e4m3_encode(vals), codes)
    assert np.isnan(oracle.fp8_e4m3_decode([0x7F, 0xFF])).all()
    pos = np.sort(vals[vals > 0])
    assert pos[0] == 2.0 ** -9 and pos[-1] == 448.0 and len(pos) == 126


def test_fp8_matches_torch_on_grid_midpoints_and_random_values():
    codes = np.arange(0, 0x7F, dtype=np.uint8)              # 0 .. 448, increasing
    vals = oracle.fp8_e4m3_decode(codes)
    mids = (vals[:-1] + vals[1:]) / 2                         # exact ties: must go to the even code
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rng = np.random.default_rng(7)
    rand = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-2 ** -5, 2 ** -5, 4000),
                           np.exp2(rng.uniform(-12, 8.8, 4000)) * rng.choice([-1, 1], 4000)])
    for v in (mids, -mids, near, rand.astype(np.float32)):
        v = np.asarray(v, dtype=np.float32)
        v = v[np.abs(v) < 448]
        assert np.array_equal(oracle.fp8_e4m3_encode(v), _fp8_torch(v))
    # every exact tie went to the code with an even mantissa
    assert (oracle.fp8_e4m3_encode(mids.astype(np.float32)) & 1 == 0).all()


def test_fp8_saturates_at_448():
    big = np.array([448.0, 448.5, 463.9, 464.0, 1e4, 3.4e38])
    assert (oracle.fp8_e4m3_encode(big) == 0x7E).all()
    assert (oracle.fp8_e4m3_encode(-big) == 0xFE).all()
    assert oracle.fp8_e4m3_encode([-0.0])[0] == 0x80 and oracle.fp8_e4m3_encode([0.0])[0] == 0x00


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_add_rms_norm_without_residual_is_rms_norm(act):
    x = _act(np.random.default_rng(3).normal(0, 2, (5, 96)), act)
    w = _act(np.random.default_rng(4).normal(1, 0.1, 96), act)
    for out in ("bf16", "f32"):
        s, y = oracle.add_rms_norm(x, w, 1e-6, None, act, out)
        assert np.array_equal(s, x)
        assert np.array_equal(y, oracle.rms_norm(x, w, 1e-6, out))
        s0, y0 = oracle.add_rms_norm(x, w, 1e-6, np.zeros_like(x), act, out)
        assert np.array_equal(s0, x) and np.array_equal(y0, y)


def _act(a, act):
    a = np.asarray(a, dtype=np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).float().numpy() if act == "bf16" else a


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_add_rms_norm_residual_stream_and_norm_input(act):
    """s is the sum rounded once to the activation type (torch: fp32 sum of
    the two operands, then its bf16 cast), and y is the norm of that s."""
    rng = np.random.default_rng(5)
    x = _act(rng.normal(0, 1, (7, 128)) * np.exp2(rng.integers(-20, 20, (7, 128))), act)
    r = _act(rng.normal(0, 1, (7, 128)) * np.exp2(rng.integers(-20, 20, (7, 128))), act)
    w = _act(rng.normal(1, 0.1, 128), act)
    s, y = oracle.add_rms_norm(x, w, 1e-6, r, act, act)
    ref = torch.from_numpy(x) + torch.from_numpy(r)
    if act == "bf16":
        ref = ref.to(torch.bfloat16).float()
    assert np.array_equal(s, ref.numpy())
    assert np.array_equal(y, oracle.rms_norm(ref.numpy(), w, 1e-6, act))
    s2, y2 = oracle.add_rms_norm(r, w, 1e-6, x, act, act)     # the add commutes
    assert np.array_equal(s2, s) and np.array_equal(y2, y)


@pytest.mark.parametrize("scale", [1.0, 0.005, 3.5])
def test_add_rms_norm_fp8_codes(scale):
    """code = e4m3(fl32(fl32(y) / scale)): y from the fp32-output norm of the
    rounded sum, the fp32 quotient by numpy, the encoding by torch where it is
    in range, saturation at +-448 otherwise."""
    rng = np.random.default_rng(int(scale * 1000))
    x = _act(rng.normal(0, 1, (6, 64)), "bf16")
    r = _act(rng.normal(0, 1, (6, 64)), "bf16")
    w = _act(rng.normal(1, 0.3, 64), "bf16")
    s, q = oracle.add_rms_norm(x, w, 1e-6, r, "bf16", "fp8_e4m3", scale)
    y32 = oracle.rms_norm(s, w, 1e-6, "f32")
    quo = (y32 / np.float32(scale)).astype(np.float32)
    inside = np.abs(quo) < 448
    assert np.array_equal(q[inside], _fp8_torch(quo[inside]))
    assert (q[~inside] == np.where(quo[~inside] > 0, 0x7E, 0xFE)).all()
    if scale == 0.005:
        assert (~inside).any() and inside.any()


# ---------------------------------------------------------------------------
# K (and V) written into cache rows picked per token
# ---------------------------------------------------------------------------

def _cache_case(tokens=23, qh=6, kvh=2, d=64, seed=31):
    rng = _rng(seed)
    q = rng.normal(0, 1, (tokens, qh, d)).astype(np.float32)
    k = rng.normal(0, 1, (tokens, kvh, d)).astype(np.float32)
    v = rng.normal(0, 1, (tokens, kvh, d)).astype(np.float32)
    wq = rng.normal(1, 0.1, d).astype(np.float32)
    wk = rng.normal(1, 0.1, d).astype(np.float32)
    pos = rng.integers(0, 3000, (1, tokens)).astype(np.int32)
    rope = oracle.Rope("1d", d, "neox", inv_freq=inv_freq_ladder(1e4, d), positions=pos)
    return q, k, v, wq, wk, rope


def test_cache_write_with_identity_slots_is_the_plain_op():
    q, k, v, wq, wk, rope = _cache_case()
    n = q.shape[0]
    kc0 = np.full((n,) + k.shape[1:], np.nan, np.float32)
    qo, kc, vc = oracle.qk_norm_rope_cache(q, k, v, wq, wk, 1e-6, rope, np.arange(n), kc0, kc0.copy())
    assert np.array_equal(qo, oracle.qk_norm_rope(q, wq, 1e-6, rope))
    assert np.array_equal(kc, oracle.qk_norm_rope(k, wk, 1e-6, rope))
    assert np.array_equal(vc, v)


def test_cache_write_reversed_and_sparse_slots():
    q, k, v, wq, wk, rope = _cache_case(seed=32)
    n = q.shape[0]
    kn = oracle.qk_norm_rope(k, wk, 1e-6, rope)
    kc0 = np.full((n,) + k.shape[1:], -7.0, np.float32)
    _, kc, vc = oracle.qk_norm_rope_cache(q, k, v, wq, wk, 1e-6, rope, np.arange(n)[::-1], kc0, kc0.copy())
    assert np.array_equal(kc, kn[::-1]) and np.array_equal(vc, v[::-1])
    # a larger cache, an injective random map with padding (-1) and out-of-range slots
    rng = _rng(33)
    num_slots = 101
    slots = rng.permutation(num_slots)[:n].astype(np.int64)
    slots[[2, 9, 15]] = -1
    slots[[4, 20]] = [num_slots, 10 ** 12]
    slots[0] = num_slots - 1
    kc0 = np.full((num_slots,) + k.shape[1:], -7.0, np.float32)
    _, kc, vc = oracle.qk_norm_rope_cache(q, k, v, wq, wk, 1e-6, rope, slots, kc0, kc0.copy())
    ok = (slots >= 0) & (slots < num_slots)
    ref_k, ref_v = kc0.copy(), kc0.copy()
    ref_k[slots[ok]] = kn[ok]                                # numpy's scatter
    ref_v[slots[ok]] = v[ok]
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)
    _, kc_nov, vc_nov = oracle.qk_norm_rope_cache(q, k, None, wq, wk, 1e-6, rope, slots, kc0, None)
    assert np.array_equal(kc_nov, ref_k) and vc_nov is None


# ----------------------------------------------------------------------------
# Eager numerics: the rounding points of an eager RMSNorm + RoPE chain
# ([VecRMS] review thread: the RMSNorm output is ((scalar_t)(x * s_variance))
# * weight; [Ovis] "Supplemental eager bitwise measurements": floating-point
# fusion off, a RoPE table in the activation type).  The reconstructions below
# run the same chain through torch's bf16 arithmetic and casts and numpy's
# float32 arithmetic, not through the oracle's own rounding code.
# ----------------------------------------------------------------------------

def _rrms32(x, eps):
    """fp32 value of 1 / sqrt(mean(x^2) + eps), from a double computation."""
    xd = x.astype(np.float64)
    return (1.0 / np.sqrt(np.mean(xd * xd, axis=-1) + np.float64(np.float32(eps)))).astype(np.float32)


def _eager_norm_torch(x, w, eps, act):
    """(act)((act)(x * s_variance) * w) with s_variance the fp32 rrms."""
    t = (x * _rrms32(x, eps)[..., None]).astype(np.float32)              # one fp32 product
    if act == "f32":
        return (t * w).astype(np.float32)
    tb = torch.from_numpy(t).to(torch.bfloat16)                          # (scalar_t)(x * s_variance)
    wb = torch.from_numpy(w).to(torch.bfloat16)
    return (tb * wb).float().numpy()                                     # bf16 * bf16 -> bf16


def _bf16_inputs(shape, k, mean=0.0, std=1.0):
    a = _rng(k).normal(mean, std, shape).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_eager_rms_norm_equals_torch_cast_chain(act):
    x = _bf16_inputs((64, 1024), 90) if act == "bf16" else _rng(90).normal(0, 1, (64, 1024)).astype(np.float32)
    w = _bf16_inputs((1024,), 91, 1.0, 0.1) if act == "bf16" else _rng(91).normal(1, 0.1, 1024).astype(np.float32)
    got = oracle.rms_norm(x, w, 1e-6, act, numerics="eager")
    assert np.array_equal(got, _eager_norm_torch(x, w, 1e-6, act))
    # the eager chain rounds twice: a visible share of elements differs from
    # the contract's single rounding, each by at most a couple of steps
    one = oracle.rms_norm(x, w, 1e-6, act)
    frac = np.mean(got != one)
    assert (0.05 < frac < 0.6) if act == "bf16" else (frac > 0.05)
    np.testing.assert_allclose(got, one, rtol=2 ** -6 if act == "bf16" else 2 ** -22)


def _eager_rotation(n, c, s, pairing, rotary_dim):
    """Eager rotation of rows n by per-(token, pair) cos/sin tables c, s
    (already in the table's type, as float32): fp32 products and sums as
    separate numpy float32 operations (no fused multiply-add)."""
    out = n.copy()
    half = rotary_dim // 2
    p = np.arange(half)
    i, j = (p, p + half) if pairing == "neox" else (2 * p, 2 * p + 1)
    a, b = n[..., i], n[..., j]
    cc, ss = c[:, None, :], s[:, None, :]
    out[..., i] = (a * cc).astype(np.float32) - (b * ss).astype(np.float32)
    out[..., j] = (b * cc).astype(np.float32) + (a * ss).astype(np.float32)
    return out


@pytest.mark.parametrize("act,pairing", [("bf16", "neox"), ("bf16", "adjacent"), ("f32", "neox")])
def test_eager_rope_equals_torch_chain(act, pairing):
    tokens, heads, d = 96, 6, 128
    if act == "bf16":
        x, w = _bf16_inputs((tokens, heads, d), 92), _bf16_inputs((d,), 93, 1.0, 0.1)
    else:
        x, w = _rng(92).normal(0, 1, (tokens, heads, d)).astype(np.float32), \
            _rng(93).normal(1, 0.1, d).astype(np.float32)
    pos = _rng(94).integers(0, 8192, (1, tokens)).astype(np.int32)
    inv = inv_freq_ladder(1e4, d)
    rope = oracle.Rope("1d", d, pairing, inv_freq=inv, positions=pos)
    got = oracle.qk_norm_rope(x, w, 1e-6, rope, act, numerics="eager")

    n = _eager_norm_torch(x, w, 1e-6, act)
    theta = (pos[0, :, None].astype(np.float32) * inv[None, :]).astype(np.float32)
    c32 = np.cos(theta.astype(np.float64)).astype(np.float32)       # fp32 table values
    s32 = np.sin(theta.astype(np.float64)).astype(np.float32)
    if act == "bf16":
        c32 = torch.from_numpy(c32).to(torch.bfloat16).float().numpy()
        s32 = torch.from_numpy(s32).to(torch.bfloat16).float().numpy()
    o = _eager_rotation(n, c32, s32, pairing, d)
    expect = torch.from_numpy(o).to(torch.bfloat16).float().numpy() if act == "bf16" else o
    assert np.array_equal(got, expect)
    if act == "f32":
        # with a fused multiply-add the first element of a pair would be
        # fl32(a c - fl32(b s)): the fp32 products are not exact here, and
        # the eager result must differ from that on a visible share
        half = d // 2
        a, b = n[..., :half].astype(np.float64), n[..., half:].astype(np.float64)
        fused = (a * c32[:, None, :] - (n[..., half:] * s32[:, None, :]).astype(np.float32)).astype(np.float32)
        assert np.mean(fused != got[..., :half]) > 0.01


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_eager_position_zero_and_norm_only_agree(act):
    """At position 0 cos is 1 and sin 0 in every type, so the eager rotation
    returns the eager norm bit for bit; the eager norm of a row is the eager
    row RMSNorm of it."""
    x, w = _bf16_inputs((20, 4, 64), 95), _bf16_inputs((64,), 96, 1.0, 0.1)
    zeros = np.zeros((1, 20), np.int32)
    rot = oracle.qk_norm_rope(x, w, 1e-6, oracle.Rope("1d", 64, "neox", inv_freq=inv_freq_ladder(1e4, 64),
                                                      positions=zeros), act, numerics="eager")
    plain = oracle.qk_norm_rope(x, w, 1e-6, None, act, numerics="eager")
    assert np.array_equal(rot, plain)
    rows = oracle.rms_norm(x.reshape(-1, 64), w, 1e-6, act, numerics="eager")
    assert np.array_equal(plain.reshape(-1, 64), rows)


def test_eager_numerics_carry_through_joint_cache_and_vit():
    """The joint, cache-write and ViT entries apply the same eager rounding
    points as the plain op on their rows."""
    heads, d = 3, 128
    txt = {k: _bf16_inputs((1, 5, heads, d), 97 + i) for i, k in enumerate("qkv")}
    img = {k: _bf16_inputs((1, 7, heads, d), 100 + i) for i, k in enumerate("qkv")}
    for st, k in ((txt, 103), (img, 105)):
        st["q_weight"], st["k_weight"] = _bf16_inputs((d,), k, 1, 0.1), _bf16_inputs((d,), k + 1, 1, 0.1)
    pos = _rng(107).integers(0, 64, (3, 12)).astype(np.int32)
    inv = inv_freq_ladder(1e4, d)
    rope = oracle.Rope("axes", d, "adjacent", inv_freq=inv, sections=(8, 28, 28, 0), positions=pos)
    q, k, _ = oracle.joint_qk_norm_rope(txt, img, 1e-6, rope, "bf16", numerics="eager")
    ri = oracle.Rope("axes", d, "adjacent", inv_freq=inv, sections=(8, 28, 28, 0), positions=pos, token_base=5)
    assert np.array_equal(q[0, 5:], oracle.qk_norm_rope(img["q"][0], img["q_weight"], 1e-6, ri, "bf16",
                                                        numerics="eager"))
    slots = np.arange(5, dtype=np.int64)[::-1].copy()
    r1 = oracle.Rope("1d", d, "neox", inv_freq=inv, positions=pos[:1])
    qo, kc, _ = oracle.qk_norm_rope_cache(txt["q"][0], txt["k"][0], None, txt["q_weight"], txt["k_weight"], 1e-6,
                                          r1, slots, np.zeros((5, heads, d), np.float32), None, "bf16",
                                          numerics="eager")
    ek = oracle.qk_norm_rope(txt["k"][0], txt["k_weight"], 1e-6, r1, "bf16", numerics="eager")
    assert np.array_equal(kc, ek[::-1])
    grids = [[1, 4, 4]]
    vx = _bf16_inputs((16, 2, 80), 108)
    vw = _bf16_inputs((80,), 109, 1, 0.1)
    it, ih, iw = inv_freq_ladder(1e4, 16), inv_freq_ladder(1e4, 32), inv_freq_ladder(1e4, 32)
    fused = oracle.vit_qk_norm_rope(vx, vw, 1e-6, it, ih, iw, grids, 2, numerics="eager")
    vpos = oracle.vit_positions(grids, 2)
    ra = oracle.Rope("axes", 80, "neox", inv_freq=np.concatenate([it, ih, iw]), sections=(8, 16, 16, 0),
                     positions=vpos)
    assert np.array_equal(fused, oracle.qk_norm_rope(vx, vw, 1e-6, ra, "bf16", numerics="eager"))
