"""The C ABI on the host (CPU only, no compute calls).

- libqkrope loads and exports every symbol include/qkrope.h declares;
- every refusal returns its status code before any HIP call (the pointers
  below are never dereferenced), so these run on a machine without a GPU;
  no test here makes a call that would pass validation with a stand-in
  pointer (it would launch);
- the library's own index functions, compiled for the host from the same
  source as the device build, agree exactly with the oracle.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import transformer_qk_rmsnorm_amd as qkr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qkrope.h")

OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3
FAKE = 0x7f0000000000          # 16-byte aligned stand-in for a device pointer
ODD = FAKE + 8                 # 8-byte aligned only


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qkr_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = declared_symbols()
    assert len(syms) >= 12
    L = qkr.lib()
    for s in syms:
        assert hasattr(L, s), f"{s} declared in qkrope.h but not exported"
    assert set(syms) == set(qkr._SIGNATURES), "binding signatures and header disagree"


def test_status_strings():
    for code, name in [(0, "QKR_OK"), (1, "QKR_ERR_INVALID_ARGUMENT"), (2, "QKR_ERR_UNSUPPORTED"),
                       (3, "QKR_ERR_MISALIGNED"), (4, "QKR_ERR_HIP")]:
        assert qkr.status_of(code) == name


# ---------------------------------------------------------------------------
# rms_norm refusals
# ---------------------------------------------------------------------------

def rms(x=FAKE, xs=5120, y=FAKE, ys=5120, w=FAKE, rows=4, width=5120, eps=1e-6, dtype=qkr.BF16):
    return qkr.lib().qkr_rms_norm(x, xs, y, ys, w, rows, width, eps, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=7), INVALID),
    (dict(dtype=qkr.BF16 | 0x200), INVALID),                            # unknown numerics bits
    (dict(dtype=qkr.BF16 | 0x10000), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(width=0), INVALID),
    (dict(rows=-1), INVALID),
    (dict(width=5121, xs=5121, ys=5121), MISALIGNED),
    (dict(x=None), INVALID),
    (dict(w=None), INVALID),
    (dict(x=ODD), MISALIGNED),
    (dict(xs=5000), INVALID),
    (dict(ys=5128 + 4), MISALIGNED),
    (dict(width=40960, xs=40960, ys=40960), UNSUPPORTED),
])
def test_rms_norm_refusals(kwargs, code):
    assert rms(**kwargs) == code
    assert qkr.last_error() != ""


def test_rms_norm_zero_rows_is_a_noop():
    assert rms(rows=0, x=None, y=None, w=None) == OK


# ---------------------------------------------------------------------------
# add_rms_norm refusals (every call below fails validation before any device
# access: the pointers are stand-ins)
# ---------------------------------------------------------------------------

XA, RA, YA = FAKE, FAKE + (1 << 30), FAKE + (1 << 31)


def addrms(x=XA, xs=5120, r=RA, rs=5120, s=RA, ss=5120, y=YA, ys=5120, kind=0, scale=None, w=FAKE, rows=4,
           width=5120, eps=1e-6, dtype=qkr.BF16):
    return qkr.lib().qkr_add_rms_norm(x, xs, r, rs, s, ss, y, ys, kind, scale, w, rows, width, eps, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=7), INVALID), (dict(kind=5), INVALID), (dict(eps=-1.0), INVALID), (dict(width=0), INVALID),
    (dict(width=5121), MISALIGNED), (dict(rows=-1), INVALID), (dict(s=None), INVALID), (dict(r=None), INVALID),
    (dict(kind=1), INVALID), (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(w=ODD), MISALIGNED),
    (dict(x=ODD), MISALIGNED), (dict(r=ODD, s=ODD), MISALIGNED), (dict(y=XA), INVALID),
    (dict(y=RA + 64), INVALID), (dict(s=XA + 16), INVALID), (dict(s=RA + 32), INVALID),
    (dict(s=RA, ss=6144), INVALID), (dict(ys=5000), MISALIGNED), (dict(xs=5124), MISALIGNED),
    (dict(kind=1, scale=FAKE, y=YA + 4), MISALIGNED), (dict(kind=1, scale=FAKE + 2), MISALIGNED),
    (dict(kind=1, scale=FAKE, ys=5124), MISALIGNED), (dict(width=16 * 256 * 8 + 8), UNSUPPORTED),
    (dict(kind=1, scale=FAKE, dtype=qkr.BF16 | qkr.NUMERICS["eager"]), UNSUPPORTED),   # FP8 has no eager chain
    (dict(dtype=qkr.F32 | 0x300), INVALID),
])
def test_add_rms_norm_refusals(kwargs, code):
    assert addrms(**kwargs) == code
    assert qkr.last_error() != ""


def test_add_rms_norm_refuses_row_sets_shifted_by_less_than_a_row():
    """x, the residual and the residual output interleaved in one buffer (row
    stride 3 x width, 2 KiB rows) share no element (the GPU tests run that
    layout); a row set shifted into another by less than a row is refused."""
    w = 1024
    x, r = XA, XA + 2 * w
    assert addrms(x=x, xs=3 * w, r=r, rs=3 * w, s=x + 1024, ss=3 * w, width=w) == INVALID
    assert addrms(x=x, xs=3 * w, r=r, rs=3 * w, s=r + 16, ss=3 * w, width=w) == INVALID
    assert addrms(x=x, xs=3 * w, r=r, rs=3 * w, s=r, ss=3 * w, y=x + 2 * 2 * w - 16, ys=3 * w, width=w) == INVALID


def test_add_rms_norm_zero_rows_is_a_noop():
    assert addrms(rows=0, x=None, r=None, s=None, y=None, w=None) == OK
    assert qkr.lib().qkr_debug_fp8_e4m3(None, 0, None, None, None) == OK
    assert qkr.lib().qkr_debug_fp8_e4m3(None, 5, None, None, None) == INVALID


# ---------------------------------------------------------------------------
# qk_norm_rope refusals
# ---------------------------------------------------------------------------

def view(ptr=FAKE, sb=0, st=24 * 128, sh=128):
    return qkr._View(ptr, sb, st, sh)


def rope_c(mode=2, pairing=0, rotary_dim=128, sections=(24, 20, 20, 0), inv=FAKE, pos=FAKE,
           pos_stride=8192, token_base=0, cosp=None, sinp=None, planes_tokens=0):
    return qkr._Rope(mode, pairing, rotary_dim, (ctypes.c_int32 * 4)(*sections), inv, pos, pos_stride,
                     token_base, cosp, sinp, planes_tokens)


def qknr(batch=1, tokens=2048, head_dim=128, dtype=qkr.BF16, eps=1e-6, q=None, qo=None, qh=16, qw=FAKE,
         k=None, ko=None, kh=8, kw=FAKE, rope="default"):
    q = q or view(st=16 * 128)
    qo = qo or view(st=16 * 128)
    k = k or view(st=8 * 128)
    ko = ko or view(st=8 * 128)
    r = rope_c() if rope == "default" else rope
    return qkr.lib().qkr_qk_norm_rope(batch, tokens, head_dim, dtype, eps, ctypes.byref(q), ctypes.byref(qo), qh,
                                      qw, ctypes.byref(k), ctypes.byref(ko), kh, kw,
                                      ctypes.byref(r) if r is not None else None, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dtype=3), INVALID),
    (dict(dtype=qkr.NUMERICS["eager"] | 2), INVALID),
    (dict(dtype=qkr.BF16 | 0x400), INVALID),
    (dict(head_dim=0), INVALID),
    (dict(head_dim=512), INVALID),
    (dict(head_dim=100), MISALIGNED),                                 # 200 B rows
    (dict(tokens=-1), INVALID),
    (dict(qh=-2), INVALID),
    (dict(q=view(ptr=None, st=2048)), INVALID),
    (dict(q=view(ptr=ODD, st=2048)), MISALIGNED),
    (dict(q=view(st=2048 + 4)), MISALIGNED),
    (dict(k=view(st=-1024)), INVALID),
    (dict(qw=None), INVALID),
    (dict(kw=ODD), MISALIGNED),
    (dict(rope=rope_c(rotary_dim=127)), INVALID),                      # odd
    (dict(rope=rope_c(rotary_dim=130)), INVALID),                      # > head_dim
    (dict(rope=rope_c(pairing=5)), INVALID),
    (dict(rope=rope_c(mode=9)), INVALID),
    (dict(rope=rope_c(rotary_dim=120, sections=(20, 20, 20, 0))), UNSUPPORTED),  # NeoX half 60 not 8-aligned
    (dict(rope=rope_c(sections=(24, 20, 19, 0))), INVALID),            # sum 63 < R/2
    (dict(rope=rope_c(sections=(60, 60, 10, 0))), INVALID),            # sum 130 > R
    (dict(rope=rope_c(sections=(0, 0, 0, 0))), INVALID),               # missing sections refused
    (dict(rope=rope_c(sections=(30, 20, 20, -6))), INVALID),
    (dict(rope=rope_c(mode=1, sections=(8, 28, 27, 0))), INVALID),     # axes must sum to R/2
    (dict(rope=rope_c(mode=1, sections=(8, 28, 24, 4))), INVALID),     # axes take three sections
    (dict(rope=rope_c(inv=None)), INVALID),
    (dict(rope=rope_c(pos=None)), INVALID),
    (dict(rope=rope_c(pos_stride=2047)), INVALID),                     # positions shorter than the call
    (dict(rope=rope_c(token_base=6145)), INVALID),                     # token_base + tokens > pos_stride
    (dict(rope=rope_c(token_base=-1)), INVALID),
    (dict(rope=rope_c(mode=3, sections=(16, 24, 24, 0))), INVALID),    # planes mode without planes
    (dict(rope=rope_c(mode=3, sections=(16, 24, 24, 0), cosp=FAKE, sinp=FAKE, planes_tokens=100)), INVALID),
    (dict(rope=rope_c(mode=3, sections=(16, 24, 24, 0), cosp=FAKE + 2, sinp=FAKE, planes_tokens=9000)),
     MISALIGNED),
])
def test_qk_norm_rope_refusals(kwargs, code):
    assert qknr(**kwargs) == code, qkr.last_error()
    assert qkr.last_error() != ""


def test_qk_norm_rope_empty_calls_are_noops():
    assert qknr(tokens=0) == OK
    assert qknr(batch=0) == OK
    assert qknr(qh=0, kh=0, qw=None, kw=None) == OK
    assert qkr.last_error() == ""


def test_adjacent_pairing_takes_any_even_rotary_dim():
    # a valid geometry gets past validation; with no tokens nothing launches
    assert qknr(tokens=0, rope=rope_c(pairing=1, rotary_dim=122, sections=(61, 0, 0, 0), pos_stride=0)) == OK


def test_joint_refusals():
    L = qkr.lib()

    def stream(tokens, ptr=FAKE, w=FAKE):
        v = view(ptr=ptr, st=9216, sh=128)
        return qkr._Stream(v, v, v, tokens, w, w)

    out = view(st=24 * 128)
    r = rope_c(mode=1, pairing=1, sections=(8, 28, 28, 0), pos_stride=4608)

    def call(text, image, rope=r, heads=24, head_dim=128):
        return L.qkr_joint_qk_norm_rope(1, heads, head_dim, qkr.BF16, 1e-6, ctypes.byref(text),
                                        ctypes.byref(image), ctypes.byref(out), ctypes.byref(out),
                                        ctypes.byref(out), ctypes.byref(rope), None)

    assert call(stream(512), stream(4096, w=None)) == INVALID
    assert call(stream(-1), stream(4096)) == INVALID
    assert call(stream(512, ptr=ODD), stream(4096)) == MISALIGNED
    short = rope_c(mode=1, pairing=1, sections=(8, 28, 28, 0), pos_stride=4607)
    assert call(stream(512), stream(4096), rope=short) == INVALID     # positions cover joint tokens
    assert L.qkr_joint_qk_norm_rope(1, 24, 128, qkr.BF16, 1e-6, None, None, None, None, None, None,
                                    None) == INVALID
    assert call(stream(0), stream(0)) == OK


def test_mrope_setup_refusals():
    L = qkr.lib()

    def call(grids, merge=2, n=None, halves=(8, 16, 16), cos=FAKE, sin=FAKE, inv=FAKE):
        flat = [v for g in grids for v in g]
        arr = (ctypes.c_int32 * max(len(flat), 1))(*flat)
        if n is None:
            n = sum(t * h * w for t, h, w in grids)
        return L.qkr_mrope_cos_sin_setup(inv, halves[0], inv, halves[1], inv, halves[2], arr, len(grids), merge,
                                         cos, sin, n, None)

    assert call([[1, 64, 63]]) == INVALID          # w not a multiple of merge
    assert call([[1, 64, 64]], merge=0) == INVALID
    assert call([[0, 64, 64]]) == INVALID
    assert call([[1, 64, 64]], n=4095) == INVALID
    assert call([]) == INVALID
    assert call([[1, 64, 64]], cos=None) == INVALID
    assert call([[1, 64, 64]], cos=FAKE + 2) == MISALIGNED
    assert call([[1, 64, 64]], halves=(0, 0, 0)) == INVALID
    assert call([[1, 64, 64]], inv=None) == INVALID


def test_variant_override_names():
    for name in ("rms:rows", "rms:split", "rms:wide", "rope:np1", "rope:np2", "rope:np3", "rope:np4",
                 "rope:lpr4", "rope:lpr8", "rope:lpr16", "rope:lpr32", "rope:stage0", "rope:stage1", "nt:0",
                 "nt:1", "rope:token", "rope:tile"):
        qkr.set_variant_override(name)
    qkr.set_variant_override(None)
    with pytest.raises(qkr.QkrError):
        qkr.set_variant_override("rms:fastest")


@pytest.mark.parametrize("variant,call", [
    ("rms:split", lambda: addrms()),                                    # the split rows cannot take the add
    ("rms:rows", lambda: rms(width=16384, xs=16384, ys=16384)),         # 2048 vectors: more than one wave holds
    ("rms:split", lambda: rms(width=16384, xs=16384, ys=16384)),
    ("rope:lpr4", lambda: qknr()),                                      # 16 vectors need 8 lanes per row
    ("rope:stage1", lambda: qknr(head_dim=256, q=view(st=16 * 256, sh=256), qo=view(st=16 * 256, sh=256),
                                 k=view(st=8 * 256, sh=256), ko=view(st=8 * 256, sh=256),
                                 rope=rope_c(rotary_dim=256, sections=(48, 40, 40, 0)))),   # 16 lanes per row
    ("rope:token", lambda: qknr()),                                     # 16 vectors: 8 lanes, a power of two
    ("rope:token", lambda: qknr(head_dim=80, qh=24, kh=24, q=view(st=24 * 80, sh=80), qo=view(st=24 * 80, sh=80),
                                k=view(st=24 * 80, sh=80), ko=view(st=24 * 80, sh=80),
                                rope=rope_c(rotary_dim=80, sections=(14, 13, 13, 0)))),   # 480 vectors > 320
    ("rope:token,rope:np2", lambda: qknr(head_dim=80, q=view(st=16 * 80, sh=80), qo=view(st=16 * 80, sh=80),
                                         k=view(st=8 * 80, sh=80), ko=view(st=8 * 80, sh=80),
                                         rope=rope_c(rotary_dim=80, sections=(14, 13, 13, 0)))),   # a tile knob
])
def test_forced_variant_that_cannot_run_is_refused_before_any_launch(variant, call):
    """A forced variant is never swapped for another: the call returns
    QKR_ERR_UNSUPPORTED from the host planner (stand-in pointers, no GPU)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("stand-in pointers: run where no GPU is visible")
    for name in variant.split(","):
        qkr.set_variant_override(name)
    try:
        assert call() == UNSUPPORTED, qkr.last_error()
        assert "forced variant" in qkr.last_error()
    finally:
        qkr.set_variant_override(None)


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 5120, dtype=torch.bfloat16)
    w = torch.ones(5120, dtype=torch.bfloat16)
    with pytest.raises(qkr.QkrError, match="GPU tensor"):
        qkr.rms_norm(x, w)
    q = torch.zeros(4, 2, 64)
    with pytest.raises(qkr.QkrError, match="GPU tensor"):
        qkr.qk_norm_rope(q, q, w[:64].float(), w[:64].float())


# ---------------------------------------------------------------------------
# index maps: the library's host build vs the oracle (exact)
# ---------------------------------------------------------------------------

SECTION_CASES = [
    ("imrope", (24, 20, 20, 0), 64), ("imrope", (16, 24, 24, 0), 64), ("imrope", (20, 24, 16, 4), 64),
    ("imrope", (0, 0, 0, 64), 64), ("imrope", (11, 12, 13, 14), 40), ("imrope", (3, 3, 2, 0), 8),
    ("imrope", (40, 40, 40, 8), 64), ("imrope", (1, 1, 1, 1), 2),
    ("axes", (8, 28, 28, 0), 64), ("axes", (8, 16, 16, 0), 40), ("axes", (0, 32, 32, 0), 64),
    ("planes", (8, 16, 16, 0), 40), ("1d", (0, 0, 0, 0), 64),
]


@pytest.mark.parametrize("mode,sections,pairs", SECTION_CASES)
def test_axis_map_host_matches_oracle(mode, sections, pairs):
    expect = oracle.axis_map(oracle.Rope(mode, 2 * pairs, sections=sections), pairs)
    got = np.array(qkr.axis_map_host(mode, sections, pairs))
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("grids,merge", [
    ([[1, 64, 64], [2, 32, 48], [1, 28, 28]], 2),
    ([[1, 4, 6], [2, 2, 4]], 2),
    ([[3, 6, 9]], 3),
    ([[2, 5, 7], [1, 1, 1], [4, 3, 2]], 1),
    ([[1, 8, 8]] * 70, 2),                         # more grids than one launch carries
])
def test_vit_positions_host_matches_oracle(grids, merge):
    expect = oracle.vit_positions(grids, merge)
    got = np.array(qkr.vit_positions_host(grids, merge))
    assert np.array_equal(got, expect)


def test_vit_fused_refusals():
    L = qkr.lib()

    def call(grids, merge=2, tokens=None, halves=(8, 16, 16), head_dim=80, pairing=0, inv=FAKE, qw=FAKE):
        flat = [v for g in grids for v in g]
        arr = (ctypes.c_int32 * max(len(flat), 1))(*flat)
        if tokens is None:
            tokens = sum(t * h * w for t, h, w in grids)
        v = view(st=16 * head_dim, sh=head_dim)
        return L.qkr_vit_qk_norm_rope(tokens, head_dim, qkr.BF16, 1e-6, ctypes.byref(v), ctypes.byref(v), 16, qw,
                                      ctypes.byref(v), ctypes.byref(v), 16, FAKE, pairing, inv, halves[0], inv,
                                      halves[1], inv, halves[2], arr, len(grids), merge, None)

    assert call([[1, 64, 63]]) == INVALID                 # w not a multiple of merge
    assert call([[1, 64, 64]], tokens=4095) == INVALID    # tokens != sum t*h*w
    assert call([[1, 64, 64]], halves=(8, 16, 24)) == INVALID   # 2 * 48 > head_dim 80
    assert call([[1, 64, 64]], halves=(4, 16, 16)) == UNSUPPORTED  # NeoX half 36 not whole vectors
    assert call([[1, 64, 64]], inv=None) == INVALID
    assert call([[1, 64, 64]], qw=None) == INVALID
    assert call([[1, 64, 64]], pairing=7) == INVALID
    assert call([]) == INVALID


# ---------------------------------------------------------------------------
# qk_norm_rope_cache refusals
# ---------------------------------------------------------------------------

def qkcache(tokens=64, head_dim=128, dtype=qkr.BF16, eps=1e-6, qh=16, kvh=8, qw=FAKE, kw=FAKE, v="view",
            vc="view", slots=FAKE, num_slots=4096, kc=None, rope="default"):
    q, qo, k = view(st=16 * 128), view(st=16 * 128), view(st=8 * 128)
    kc = kc or view(st=8 * 128)
    vv = view(st=8 * 128) if v == "view" else v
    vcc = view(st=8 * 128) if vc == "view" else vc
    r = rope_c(mode=0, sections=(0, 0, 0, 0)) if rope == "default" else rope
    return qkr.lib().qkr_qk_norm_rope_cache(tokens, head_dim, dtype, eps, ctypes.byref(q), ctypes.byref(qo), qh, qw,
                                            ctypes.byref(k), ctypes.byref(vv) if vv is not None else None, kvh, kw,
                                            ctypes.byref(kc), ctypes.byref(vcc) if vcc is not None else None, slots,
                                            num_slots, ctypes.byref(r) if r is not None else None, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(slots=None), INVALID), (dict(slots=FAKE + 4), MISALIGNED), (dict(v=None), INVALID),
    (dict(vc=None), INVALID), (dict(num_slots=-1), INVALID), (dict(tokens=-1), INVALID),
    (dict(kc=view(ptr=FAKE + 8, st=8 * 128)), MISALIGNED), (dict(kc=view(ptr=None)), INVALID),
    (dict(kw=None), INVALID), (dict(head_dim=100), MISALIGNED), (dict(dtype=9), INVALID),
    (dict(rope=rope_c(mode=0, rotary_dim=129, sections=(0, 0, 0, 0))), INVALID),
    (dict(tokens=1 << 31), UNSUPPORTED),
])
def test_qk_norm_rope_cache_refusals(kwargs, code):
    assert qkcache(**kwargs) == code
    assert qkr.last_error() != ""


def test_qk_norm_rope_cache_empty_calls_are_noops():
    assert qkcache(tokens=0, slots=None) == OK
    assert qkcache(qh=0, kvh=0, qw=None, kw=None, slots=None) == OK


# ---------------------------------------------------------------------------
# size arithmetic: counts whose products leave 64 bits are refused, never
# wrapped into a small launch
# ---------------------------------------------------------------------------

BIG = 1 << 62


def test_row_counts_beyond_the_grid_are_refused():
    # rows x blocks-per-row wraps to 0 in 64 bits when rows = 2^62 and a row takes 4 blocks
    assert rms(rows=BIG, width=2048, xs=2048, ys=2048) == UNSUPPORTED
    assert rms(rows=(1 << 31), width=64, xs=64, ys=64) == UNSUPPORTED
    assert addrms(rows=BIG) == UNSUPPORTED
    # the row set (rows - 1) x stride leaves the address space before any overlap check runs
    assert rms(rows=1 << 20, xs=1 << 40) == UNSUPPORTED
    assert addrms(rows=1 << 20, ys=1 << 40) == UNSUPPORTED
    assert qkr.lib().qkr_debug_fp8_e4m3(FAKE, 1 << 31, None, FAKE, None) == UNSUPPORTED


@pytest.mark.parametrize("kwargs", [
    dict(qh=(1 << 31) - 1, kh=2),                        # q_heads + k_heads wraps in 32 bits
    dict(qh=(1 << 30), kh=(1 << 30)),
    dict(batch=(1 << 31) - 1, tokens=(1 << 31) - 1, qh=1 << 20, kh=0),   # product wraps in 64 bits
    dict(tokens=1 << 31),
    dict(tokens=BIG, batch=0),                           # an empty batch does not hide the token bound
    dict(q=view(st=1 << 50)),                            # stride past the address space
    dict(q=view(sb=-(1 << 60), st=16 * 128)),            # unused strides are bounded too
    dict(tokens=1 << 20, q=view(st=1 << 32)),            # (tokens - 1) x stride spans > 2^48 bytes
])
def test_qk_norm_rope_size_refusals(kwargs):
    assert qknr(**kwargs) == UNSUPPORTED, qkr.last_error()


@pytest.mark.parametrize("rope,code", [
    # sections whose 32-bit sum wraps onto rotary_dim / 2
    (rope_c(mode=1, sections=((1 << 31) - 1, (1 << 31) - 1, 66, 0)), INVALID),
    # token_base + tokens leaves 64 bits
    (rope_c(token_base=(1 << 63) - 100), INVALID),
    (rope_c(mode=3, sections=(16, 24, 24, 0), cosp=FAKE, sinp=FAKE, planes_tokens=4096,
            token_base=(1 << 63) - 100), INVALID),
    (rope_c(pos_stride=1 << 60), UNSUPPORTED),           # position planes past the address space
    (rope_c(mode=3, sections=(16, 24, 24, 0), cosp=FAKE, sinp=FAKE, planes_tokens=1 << 50), UNSUPPORTED),
])
def test_rope_size_refusals(rope, code):
    assert qknr(rope=rope) == code, qkr.last_error()


def test_axis_map_sections_that_wrap_are_refused():
    out = (ctypes.c_int32 * 4)()
    m = (1 << 31) - 1
    for sections in ((m, m, 3, 0), (m, 1, 0, 0), (1 << 21, 0, 0, 0), (4, -1, 4, 0)):
        # (m, m, 3, 0) sums to 1 in 32 bits; 3 x 2^21 still fits but exceeds the stated range
        big = rope_c(mode=2, sections=sections)
        assert qkr.lib().qkr_axis_map_host(ctypes.byref(big), 4, out) == INVALID, sections
        assert qkr.lib().qkr_debug_axis_map(ctypes.byref(big), 4, FAKE, None) == INVALID, sections


def test_cache_and_joint_size_refusals():
    assert qkcache(kvh=(1 << 30), qh=(1 << 30)) == UNSUPPORTED                  # 2 x kv_heads in 32 bits
    assert qkcache(tokens=1 << 20, kvh=1 << 19, qh=0, qw=None) == UNSUPPORTED   # 2^20 x 2^20 rows
    assert qkcache(num_slots=1 << 40) == UNSUPPORTED                            # cache spans > 2^48 bytes
    L = qkr.lib()

    def stream(tokens):
        v = view(st=9216, sh=128)
        return qkr._Stream(v, v, v, tokens, FAKE, FAKE)

    out = view(st=24 * 128)
    r = rope_c(mode=1, pairing=1, sections=(8, 28, 28, 0), pos_stride=4608)

    def call(text, image, heads=24, batch=1):
        return L.qkr_joint_qk_norm_rope(batch, heads, 128, qkr.BF16, 1e-6, ctypes.byref(text), ctypes.byref(image),
                                        ctypes.byref(out), ctypes.byref(out), ctypes.byref(out), ctypes.byref(r),
                                        None)

    assert call(stream((1 << 63) - 1), stream(2)) == UNSUPPORTED    # text + image tokens leave 64 bits
    assert call(stream(1 << 30), stream(1 << 30), heads=1 << 18, batch=1 << 30) == UNSUPPORTED


def test_grid_products_that_leave_64_bits_are_refused():
    L = qkr.lib()
    m = (1 << 31) - 1
    # t x h x w = (2^31 - 1)^3 and its sum over grids wrap in 64 bits
    flat = [m, m - 1, m - 1] * 3
    arr = (ctypes.c_int32 * len(flat))(*flat)
    assert L.qkr_vit_positions_host(arr, 3, 1, None, 0) == UNSUPPORTED
    assert L.qkr_mrope_cos_sin_setup(FAKE, 8, FAKE, 16, FAKE, 16, arr, 3, 1, FAKE, FAKE, 0, None) == UNSUPPORTED
    # one grid of 2^30 tokens with 64 columns: 2^36 setup threads
    one = (ctypes.c_int32 * 3)(1, 1 << 15, 1 << 15)
    assert L.qkr_mrope_cos_sin_setup(FAKE, 16, FAKE, 16, FAKE, 32, one, 1, 1, FAKE, FAKE, 1 << 30,
                                     None) == UNSUPPORTED
    # ViT fused: head counts whose 32-bit sum wraps
    v = view(st=16 * 80, sh=80)
    g = (ctypes.c_int32 * 3)(1, 64, 64)
    assert L.qkr_vit_qk_norm_rope(4096, 80, qkr.BF16, 1e-6, ctypes.byref(v), ctypes.byref(v), (1 << 31) - 1, FAKE,
                                  ctypes.byref(v), ctypes.byref(v), 2, FAKE, 0, FAKE, 8, FAKE, 16, FAKE, 16, g, 1, 2,
                                  None) == UNSUPPORTED
    # ViT fused: axis halves whose 32-bit sum wraps past head_dim / 2
    assert L.qkr_vit_qk_norm_rope(4096, 80, qkr.BF16, 1e-6, ctypes.byref(v), ctypes.byref(v), 16, FAKE,
                                  ctypes.byref(v), ctypes.byref(v), 16, FAKE, 0, FAKE, (1 << 31) - 1, FAKE,
                                  (1 << 31) - 1, FAKE, 8, g, 1, 2, None) == INVALID


def test_missing_library_fails_loudly():
    """With no built library the binding raises at once (no fallback path):
    loading it and calling an entry point both raise QkrError."""
    import subprocess
    import sys
    code = ("import transformer_qk_rmsnorm_amd as qkr\n"
            "qkr.LIB_PATH = '/nonexistent/libqkrope.so'\n"
            "for f in (qkr.lib, lambda: qkr.status_of(0)):\n"
            "    try:\n"
            "        f()\n"
            "    except qkr.QkrError as e:\n"
            "        assert 'is not built' in str(e), e\n"
            "    else:\n"
            "        raise SystemExit('no error')\n"
            "print('raised')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "raised" in r.stdout, r.stdout + r.stderr


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and a
    JSON message, before touching a GPU."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
