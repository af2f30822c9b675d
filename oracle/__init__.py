"""CPU oracle for per-row RMSNorm fused with rotary position embedding.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It wraps
``liboracle.so`` (plain C in ``oracle.c``, double precision, written from the
pages) with numpy marshalling and shares no code with the HIP library.

Arrays in and out are numpy: activations/weights as float32 (a bf16 tensor is
passed decoded to float32, which is exact), positions and grids as int32.
``out_dtype`` is ``"f32"`` or ``"bf16"``; a bf16 result is returned as float32
values that lie on the bf16 grid.

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, invariants, library special cases and the hand-derived fixtures in
tests/golden/.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB lets the mutation test load a deliberately broken build of
# oracle.c to show that the pins catch it; it is never set otherwise.
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

POS_1D, POS_AXES, POS_IMROPE, POS_PLANES = 0, 1, 2, 3
PAIR_NEOX, PAIR_ADJACENT = 0, 1
_MODES = {"1d": POS_1D, "axes": POS_AXES, "imrope": POS_IMROPE, "planes": POS_PLANES}
_PAIRS = {"neox": PAIR_NEOX, "adjacent": PAIR_ADJACENT}
_OUT = {"f32": 0, "bf16": 1}
_NUMERICS = {"contract": 0, "eager": 1}

_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)


class _Rope(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("pairing", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("inv_freq", _f32p),
        ("sections", ctypes.c_int32 * 4),
        ("positions", _i32p),
        ("pos_stride", ctypes.c_int64),
        ("token_base", ctypes.c_int64),
        ("cos_planes", _f32p),
        ("sin_planes", _f32p),
        ("planes_tokens", ctypes.c_int64),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_round_bf16.restype = ctypes.c_double
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_rms_norm.restype = None
        lib.oracle_rms_norm.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, _f32p,
                                        ctypes.c_float, ctypes.c_int32, ctypes.c_int32, _f32p]
        lib.oracle_fp8_e4m3_decode.restype = ctypes.c_double
        lib.oracle_fp8_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_add_rms_norm.restype = None
        lib.oracle_add_rms_norm.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_int32, _f32p, ctypes.c_float,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _f32p,
                                            _f32p, ctypes.POINTER(ctypes.c_uint8)]
        lib.oracle_qk_norm_rope_cache.restype = None
        lib.oracle_qk_norm_rope_cache.argtypes = [_f32p, ctypes.c_int32, _f32p, _f32p, ctypes.c_int32,
                                                  ctypes.c_int64, ctypes.c_int32, _f32p, _f32p, ctypes.c_float,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Rope),
                                                  ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, _f32p, _f32p,
                                                  _f32p]
        lib.oracle_axis.restype = ctypes.c_int32
        lib.oracle_axis.argtypes = [ctypes.POINTER(_Rope), ctypes.c_int32]
        lib.oracle_qk_norm_rope.restype = None
        lib.oracle_qk_norm_rope.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            _f32p, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(_Rope), _f32p]
        lib.oracle_joint_qk_norm_rope.restype = None
        lib.oracle_joint_qk_norm_rope.argtypes = (
            [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
            + [_f32p] * 3 + [ctypes.c_int64] + [_f32p] * 2
            + [_f32p] * 3 + [ctypes.c_int64] + [_f32p] * 2
            + [ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Rope)] + [_f32p] * 3)
        lib.oracle_vit_positions.restype = None
        lib.oracle_vit_positions.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, _i32p,
                                             ctypes.c_int64]
        lib.oracle_vit_qk_norm_rope.restype = None
        lib.oracle_vit_qk_norm_rope.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _f32p,
                                                ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                _f32p, ctypes.c_int32, _f32p, ctypes.c_int32, _f32p,
                                                ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32, _f32p]
        lib.oracle_vit_cos_sin.restype = None
        lib.oracle_vit_cos_sin.argtypes = [_f32p, ctypes.c_int32, _f32p, ctypes.c_int32,
                                           _f32p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                           ctypes.c_int32, _f32p, _f32p, ctypes.c_int64]
        _lib = lib
    return _lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_f32p)


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


class Rope:
    """RoPE parameters for the oracle.

    mode: "1d" | "axes" | "imrope" | "planes"; pairing: "neox" | "adjacent".
    inv_freq: float32 [R/2] (not planes).  sections: 4 ints (axes/planes: pairs
    per axis t, h, w; imrope: s0..s3).  positions: int32 [n_planes, pos_stride]
    (not planes).  token_base: first token of the call inside every plane.
    cos_planes/sin_planes: float32 [3, planes_tokens, R/2] (planes mode).
    """

    def __init__(self, mode, rotary_dim, pairing="neox", inv_freq=None, sections=(0, 0, 0, 0),
                 positions=None, token_base=0, cos_planes=None, sin_planes=None):
        self.mode = mode
        self.pairing = pairing
        self.rotary_dim = int(rotary_dim)
        self.inv_freq = None if inv_freq is None else np.ascontiguousarray(inv_freq, np.float32)
        self.sections = tuple(int(s) for s in sections)
        self.positions = None if positions is None else np.ascontiguousarray(positions, np.int32)
        self.token_base = int(token_base)
        self.cos_planes = None if cos_planes is None else np.ascontiguousarray(cos_planes, np.float32)
        self.sin_planes = None if sin_planes is None else np.ascontiguousarray(sin_planes, np.float32)

    def _c(self):
        r = _Rope()
        r.mode = _MODES[self.mode]
        r.pairing = _PAIRS[self.pairing]
        r.rotary_dim = self.rotary_dim
        r.sections = (ctypes.c_int32 * 4)(*self.sections)
        if self.inv_freq is not None:
            r.inv_freq = self.inv_freq.ctypes.data_as(_f32p)
        if self.positions is not None:
            pos = self.positions.reshape(-1, self.positions.shape[-1])
            r.positions = pos.ctypes.data_as(_i32p)
            r.pos_stride = pos.shape[-1]
        r.token_base = self.token_base
        if self.cos_planes is not None:
            r.cos_planes = self.cos_planes.ctypes.data_as(_f32p)
            r.sin_planes = self.sin_planes.ctypes.data_as(_f32p)
            r.planes_tokens = self.cos_planes.shape[1]
        return r


def round_bf16(v) -> np.ndarray:
    """Nearest bf16 value (ties to even) of every element, as float64."""
    lib = _load()
    v = np.asarray(v, dtype=np.float64)
    return np.vectorize(lib.oracle_round_bf16, otypes=[np.float64])(v) if v.size else v.copy()


def rms_norm(x, weight, eps, out_dtype="bf16", numerics="contract"):
    """Plain row RMSNorm of x [rows, width].  numerics "contract" (one
    rounding) or "eager" (the eager chain's rounding points)."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(weight)
    rows, width = x.shape
    y = np.empty_like(x)
    lib.oracle_rms_norm(xp, rows, width, wp, eps, _OUT[out_dtype], _NUMERICS[numerics], y.ctypes.data_as(_f32p))
    return y


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (uint8 array)."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_fp8_e4m3_decode(int(v)) for v in c.ravel()]).reshape(c.shape)


def fp8_e4m3_encode(values) -> np.ndarray:
    """OCP FP8 E4M3 codes of finite reals (round half to even, saturating)."""
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.oracle_fp8_e4m3_encode(float(a)) for a in v.ravel()], dtype=np.uint8).reshape(v.shape)


def add_rms_norm(x, weight, eps, residual=None, act_dtype="bf16", out_dtype="bf16", scale=1.0,
                 numerics="contract"):
    """Residual add + RMSNorm of x [rows, width]: returns (s, y) where s is the
    new residual stream and y the output (float array, or uint8 FP8 E4M3
    codes for out_dtype "fp8_e4m3", which has no eager numerics)."""
    if numerics != "contract" and out_dtype == "fp8_e4m3":
        raise ValueError("the FP8 output is defined for the contract numerics only")
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(weight)
    rows, width = x.shape
    if residual is not None:
        r, rp = _f32(residual)
        if r.shape != x.shape:
            raise ValueError("residual must match x")
    else:
        r, rp = None, None
    s = np.empty_like(x)
    fp8 = out_dtype == "fp8_e4m3"
    y = np.empty(x.shape, np.uint8 if fp8 else np.float32)
    out_kind = 2 if fp8 else _OUT[out_dtype]
    lib.oracle_add_rms_norm(xp, rp, rows, width, wp, eps, _OUT[act_dtype], out_kind, _NUMERICS[numerics], scale,
                            s.ctypes.data_as(_f32p), None if fp8 else y.ctypes.data_as(_f32p),
                            y.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)) if fp8 else None)
    return s, y


def axis_map(rope: Rope, n_pairs: int) -> np.ndarray:
    """Position axis (0=t, 1=h, 2=w, 3=e) read by each of n_pairs pairs."""
    lib = _load()
    r = rope._c()
    return np.array([lib.oracle_axis(ctypes.byref(r), p) for p in range(n_pairs)], np.int32)


def qk_norm_rope(x, weight, eps, rope=None, out_dtype="bf16", numerics="contract"):
    """Per-(token, head) RMSNorm + RoPE of x [tokens, heads, head_dim]."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(weight)
    tokens, heads, head_dim = x.shape
    out = np.empty_like(x)
    rp = ctypes.byref(rope._c()) if rope is not None else None
    lib.oracle_qk_norm_rope(xp, tokens, heads, head_dim, wp, eps, _OUT[out_dtype], _NUMERICS[numerics], rp,
                            out.ctypes.data_as(_f32p))
    return out


def qk_norm_rope_cache(q, k, v, q_weight, k_weight, eps, rope, slots, k_cache, v_cache, out_dtype="bf16",
                       numerics="contract"):
    """Q out [tokens, Hq, D] plus the caches [num_slots, Hkv, D] after writing
    token t's rotated K and its V into row slots[t] (copies of the given
    caches are updated and returned: (q_out, k_cache, v_cache))."""
    lib = _load()
    q, qp = _f32(q)
    k, kp = _f32(k)
    tokens, qh, d = q.shape
    kvh = k.shape[1]
    if v is not None:
        v, vp = _f32(v)
    else:
        vp = None
    wq, wqp = _f32(q_weight)
    wk, wkp = _f32(k_weight)
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    kc = np.array(k_cache, dtype=np.float32, copy=True)
    vc = np.array(v_cache, dtype=np.float32, copy=True) if v_cache is not None else None
    qo = np.empty_like(q)
    r = rope._c() if rope is not None else None
    lib.oracle_qk_norm_rope_cache(qp, qh, kp, vp, kvh, tokens, d, wqp, wkp, eps, _OUT[out_dtype], _NUMERICS[numerics],
                                  ctypes.byref(r) if r is not None else None,
                                  sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), kc.shape[0],
                                  qo.ctypes.data_as(_f32p), kc.ctypes.data_as(_f32p),
                                  vc.ctypes.data_as(_f32p) if vc is not None else None)
    return qo, kc, vc


def joint_qk_norm_rope(txt, img, eps, rope, out_dtype="bf16", numerics="contract"):
    """Joint text/image op.

    txt / img: dicts with q, k, v float32 [batch, tokens_s, heads, head_dim]
    and q_weight, k_weight float32 [head_dim].  Returns (q, k, v) float32
    [batch, tokens_txt + tokens_img, heads, head_dim].
    """
    lib = _load()
    keep = []

    def arr(a):
        a, p = _f32(a)
        keep.append(a)
        return a, p

    qt, qtp = arr(txt["q"]); _, ktp = arr(txt["k"]); _, vtp = arr(txt["v"])
    _, qwtp = arr(txt["q_weight"]); _, kwtp = arr(txt["k_weight"])
    qi, qip = arr(img["q"]); _, kip = arr(img["k"]); _, vip = arr(img["v"])
    _, qwip = arr(img["q_weight"]); _, kwip = arr(img["k_weight"])
    batch, st, heads, d = qt.shape
    si = qi.shape[1]
    shape = (batch, st + si, heads, d)
    qo, ko, vo = (np.empty(shape, np.float32) for _ in range(3))
    r = rope._c()
    lib.oracle_joint_qk_norm_rope(batch, heads, d, qtp, ktp, vtp, st, qwtp, kwtp,
                                  qip, kip, vip, si, qwip, kwip, eps, _OUT[out_dtype], _NUMERICS[numerics],
                                  ctypes.byref(r), qo.ctypes.data_as(_f32p),
                                  ko.ctypes.data_as(_f32p), vo.ctypes.data_as(_f32p))
    return qo, ko, vo


def vit_positions(grid_thw, merge) -> np.ndarray:
    """(3, N) int32 (t, h, w) position of every ViT patch token."""
    lib = _load()
    g, gp = _i32(np.asarray(grid_thw).reshape(-1, 3))
    n = int(sum(int(t) * int(h) * int(w) for t, h, w in g))
    pos = np.empty((3, n), np.int32)
    lib.oracle_vit_positions(gp, g.shape[0], merge, pos.ctypes.data_as(_i32p), n)
    return pos


def vit_cos_sin(inv_t, inv_h, inv_w, grid_thw, merge, fill=np.nan):
    """(cos, sin) float32 planes [3, N, half_t + half_h + half_w].

    Columns outside each plane's own section keep ``fill``.
    """
    lib = _load()
    it, itp = _f32(inv_t)
    ih, ihp = _f32(inv_h)
    iw, iwp = _f32(inv_w)
    g, gp = _i32(np.asarray(grid_thw).reshape(-1, 3))
    n = int(sum(int(t) * int(h) * int(w) for t, h, w in g))
    half = it.size + ih.size + iw.size
    cos = np.full((3, n, half), fill, np.float32)
    sin = np.full((3, n, half), fill, np.float32)
    lib.oracle_vit_cos_sin(itp, it.size, ihp, ih.size, iwp, iw.size, gp, g.shape[0], merge,
                           cos.ctypes.data_as(_f32p), sin.ctypes.data_as(_f32p), n)
    return cos, sin


def vit_qk_norm_rope(x, weight, eps, inv_t, inv_h, inv_w, grid_thw, merge, pairing="neox", out_dtype="bf16",
                     numerics="contract"):
    """Per-head RMSNorm + RoPE of x [N, heads, head_dim] with (t, h, w)
    positions computed from the ViT grids (no cos/sin planes)."""
    lib = _load()
    x, xp = _f32(x)
    w, wp = _f32(weight)
    it, itp = _f32(inv_t)
    ih, ihp = _f32(inv_h)
    iw, iwp = _f32(inv_w)
    g, gp = _i32(np.asarray(grid_thw).reshape(-1, 3))
    n, heads, d = x.shape
    out = np.empty_like(x)
    lib.oracle_vit_qk_norm_rope(xp, n, heads, d, wp, eps, _OUT[out_dtype], _NUMERICS[numerics], _PAIRS[pairing],
                                itp, it.size, ihp,
                                ih.size, iwp, iw.size, gp, g.shape[0], merge, out.ctypes.data_as(_f32p))
    return out
