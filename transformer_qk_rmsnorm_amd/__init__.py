"""Python binding of libqkrope: fused per-head QK RMSNorm + RoPE on MI355X.

Argument marshalling only.  Every operation runs in the gfx950 kernels of
``libqkrope.so`` through its C ABI (``include/qkrope.h``); PyTorch supplies
device memory, fresh output tensors and the current HIP stream.  There is no
fallback: if the library is missing, or a tensor is not on the GPU, the call
raises.

Functions (same names as the C entry points, without the ``qkr_`` prefix;
the prefixed spellings are aliases; every entry point with a dtype takes
``numerics="contract"`` (default) or ``"eager"``):
    rms_norm(x, weight, eps)                         -> y
    qk_norm_rope(q, k, q_weight, k_weight, eps, rope) -> (q_out, k_out)
    joint_qk_norm_rope(text, image, eps, rope)        -> (q, k, v)
    mrope_cos_sin_setup(inv_t, inv_h, inv_w, grid_thw, spatial_merge) -> (cos, sin)
    vit_qk_norm_rope(q, k, q_weight, k_weight, eps, inv_t, inv_h, inv_w, grid_thw, spatial_merge)
                                                      -> (q_out, k_out)
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkrope.so")

F32, BF16 = 0, 1
NUMERICS = {"contract": 0, "eager": 0x100}
MODES = {"1d": 0, "axes": 1, "imrope": 2, "planes": 3}
PAIRINGS = {"neox": 0, "adjacent": 1}
_PLANES_NEEDED = {"1d": 1, "axes": 3, "imrope": 4}


class QkrError(RuntimeError):
    """A refusal or launch failure reported by libqkrope."""


class _View(ctypes.Structure):
    _fields_ = [("ptr_dev", ctypes.c_void_p), ("stride_batch", ctypes.c_int64),
                ("stride_tok", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class _Rope(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("pairing", ctypes.c_int32), ("rotary_dim", ctypes.c_int32),
                ("sections", ctypes.c_int32 * 4), ("inv_freq_dev", ctypes.c_void_p),
                ("positions_dev", ctypes.c_void_p), ("pos_stride", ctypes.c_int64),
                ("token_base", ctypes.c_int64), ("cos_planes_dev", ctypes.c_void_p),
                ("sin_planes_dev", ctypes.c_void_p), ("planes_tokens", ctypes.c_int64)]


class _Stream(ctypes.Structure):
    _fields_ = [("q", _View), ("k", _View), ("v", _View), ("tokens", ctypes.c_int64),
                ("q_weight_dev", ctypes.c_void_p), ("k_weight_dev", ctypes.c_void_p)]


_P = ctypes.POINTER
_lib_handle = None

# Every symbol include/qkrope.h declares, with its ctypes signature.
_SIGNATURES = {
    "qkr_rms_norm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                    ctypes.c_int32, ctypes.c_void_p]),
    "qkr_add_rms_norm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]),
    "qkr_debug_fp8_e4m3": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "qkr_qk_norm_rope_cache": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                              _P(_View), _P(_View), ctypes.c_int32, ctypes.c_void_p, _P(_View),
                                              _P(_View), ctypes.c_int32, ctypes.c_void_p, _P(_View), _P(_View),
                                              ctypes.c_void_p, ctypes.c_int64, _P(_Rope), ctypes.c_void_p]),
    "qkr_qk_norm_rope": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_float, _P(_View), _P(_View), ctypes.c_int32, ctypes.c_void_p,
                                        _P(_View), _P(_View), ctypes.c_int32, ctypes.c_void_p, _P(_Rope),
                                        ctypes.c_void_p]),
    "qkr_joint_qk_norm_rope": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_float, _P(_Stream), _P(_Stream), _P(_View), _P(_View),
                                              _P(_View), _P(_Rope), ctypes.c_void_p]),
    "qkr_mrope_cos_sin_setup": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_int32, _P(ctypes.c_int32),
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_int64, ctypes.c_void_p]),
    "qkr_vit_qk_norm_rope": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                            _P(_View), _P(_View), ctypes.c_int32, ctypes.c_void_p,
                                            _P(_View), _P(_View), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_int32, _P(ctypes.c_int32), ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p]),
    "qkr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qkr_last_error": (ctypes.c_char_p, []),
    "qkr_set_variant_override": (ctypes.c_int, [ctypes.c_char_p]),
    "qkr_debug_last_variant": (ctypes.c_char_p, []),
    "qkr_last_variant": (ctypes.c_char_p, []),
    "qkr_debug_axis_map": (ctypes.c_int, [_P(_Rope), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "qkr_debug_vit_positions": (ctypes.c_int, [_P(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "qkr_axis_map_host": (ctypes.c_int, [_P(_Rope), ctypes.c_int32, _P(ctypes.c_int32)]),
    "qkr_vit_positions_host": (ctypes.c_int, [_P(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32,
                                              _P(ctypes.c_int32), ctypes.c_int64]),
}


def lib():
    """The loaded libqkrope (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise QkrError(f"{LIB_PATH} is not built: run `python -m transformer_qk_rmsnorm_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = handle
    return _lib_handle


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise QkrError(f"{what}: {L.qkr_status_string(status).decode()}: {L.qkr_last_error().decode()}")


def status_of(status: int) -> str:
    return lib().qkr_status_string(status).decode()


def last_error() -> str:
    return lib().qkr_last_error().decode()


def last_variant() -> str:
    return lib().qkr_debug_last_variant().decode()


def set_variant_override(name: Optional[str]):
    _check(lib().qkr_set_variant_override(None if name is None else name.encode()), "set_variant_override")


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor, numerics: str = "contract") -> int:
    """The C dtype argument: the element type OR-ed with the numerics bits."""
    if numerics not in NUMERICS:
        raise QkrError(f"unknown numerics {numerics!r} (contract or eager)")
    if t.dtype == torch.float32:
        return F32 | NUMERICS[numerics]
    if t.dtype == torch.bfloat16:
        return BF16 | NUMERICS[numerics]
    raise QkrError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _on_gpu(name: str, t: torch.Tensor, device: torch.device):
    if not t.is_cuda:
        raise QkrError(f"{name} must be a GPU tensor (got {t.device})")
    if t.device != device:
        raise QkrError(f"{name} is on {t.device}, expected {device}")


def _unit_stride(t: torch.Tensor, dim: int) -> bool:
    """Whether dimension `dim` is laid out contiguously.  An empty tensor has
    no elements to lay out (torch may give it any strides), and a dimension of
    length 1 has no stride to speak of."""
    return t.numel() == 0 or t.shape[dim] <= 1 or t.stride(dim) == 1


def _rows4(name: str, t: torch.Tensor) -> torch.Tensor:
    """[tokens, heads, D] or [batch, tokens, heads, D] -> 4-D view."""
    if t.dim() == 3:
        t = t.unsqueeze(0)
    if t.dim() != 4:
        raise QkrError(f"{name} must be [tokens, heads, head_dim] or [batch, tokens, heads, head_dim]")
    if not _unit_stride(t, -1):
        raise QkrError(f"{name}: the head_dim dimension must be contiguous")
    return t


def _view(t: Optional[torch.Tensor]) -> _View:
    if t is None:
        return _View(None, 0, 0, 0)
    return _View(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


@dataclass
class Rope:
    """Rotary parameters (device tensors for the per-call data).

    mode: "1d" | "axes" | "imrope" | "planes"; pairing: "neox" | "adjacent".
    inv_freq: float32 [R/2].  positions: int32 [planes, L] with planes 1 (1d),
    3 (axes) or 4 (imrope) and L >= token_base + tokens.  sections: pairs per
    axis (axes/planes) or IMROPE s0..s3.  cos_planes / sin_planes: float32
    [3, T, R/2] from mrope_cos_sin_setup (planes mode).
    """
    mode: str
    rotary_dim: int
    pairing: str = "neox"
    inv_freq: Optional[torch.Tensor] = None
    positions: Optional[torch.Tensor] = None
    sections: Sequence[int] = (0, 0, 0, 0)
    token_base: int = 0
    cos_planes: Optional[torch.Tensor] = None
    sin_planes: Optional[torch.Tensor] = None

    def to_c(self, device: torch.device, tokens: int) -> _Rope:
        if self.mode not in MODES or self.pairing not in PAIRINGS:
            raise QkrError(f"unknown mode {self.mode!r} or pairing {self.pairing!r}")
        secs = tuple(int(s) for s in self.sections) + (0,) * (4 - len(self.sections))
        r = _Rope(MODES[self.mode], PAIRINGS[self.pairing], int(self.rotary_dim), (ctypes.c_int32 * 4)(*secs[:4]),
                  None, None, 0, int(self.token_base), None, None, 0)
        half = int(self.rotary_dim) // 2
        if self.rotary_dim == 0:
            return r
        if self.mode == "planes":
            for nm, p in (("cos_planes", self.cos_planes), ("sin_planes", self.sin_planes)):
                if p is None:
                    raise QkrError(f"planes mode needs {nm}")
                _on_gpu(nm, p, device)
                if p.dtype != torch.float32 or not p.is_contiguous() or p.dim() != 3 or p.shape[0] != 3 \
                        or p.shape[2] != half:
                    raise QkrError(f"{nm} must be contiguous float32 [3, tokens, rotary_dim/2={half}]")
            if self.cos_planes.shape != self.sin_planes.shape:
                raise QkrError("cos_planes and sin_planes differ in shape")
            r.cos_planes_dev = self.cos_planes.data_ptr()
            r.sin_planes_dev = self.sin_planes.data_ptr()
            r.planes_tokens = self.cos_planes.shape[1]
            return r
        if self.inv_freq is None or self.positions is None:
            raise QkrError(f"mode {self.mode} needs inv_freq and positions")
        _on_gpu("inv_freq", self.inv_freq, device)
        _on_gpu("positions", self.positions, device)
        if self.inv_freq.dtype != torch.float32 or not self.inv_freq.is_contiguous() \
                or self.inv_freq.numel() < half:
            raise QkrError(f"inv_freq must be contiguous float32 with >= {half} entries")
        pos = self.positions
        if pos.dtype != torch.int32 or pos.dim() != 2 or not _unit_stride(pos, 1):
            raise QkrError("positions must be int32 [planes, tokens] with contiguous rows")
        need = _PLANES_NEEDED[self.mode]
        if pos.shape[0] < need:
            raise QkrError(f"mode {self.mode} needs {need} position planes, got {pos.shape[0]}")
        if pos.shape[1] < self.token_base + tokens:
            raise QkrError(f"positions hold {pos.shape[1]} tokens, the call reads up to "
                           f"{self.token_base + tokens}")
        if need > 1 and pos.stride(0) < pos.shape[1]:
            raise QkrError("position planes overlap")
        r.inv_freq_dev = self.inv_freq.data_ptr()
        r.positions_dev = pos.data_ptr()
        # One plane read (1d): its length bounds the reads, whatever the planes' stride.
        r.pos_stride = pos.stride(0) if need > 1 else pos.shape[1]
        return r


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6,
             out: Optional[torch.Tensor] = None, numerics: str = "contract") -> torch.Tensor:
    """Row RMSNorm of x [rows, width] (qkr_rms_norm).  numerics "contract"
    (one rounding) or "eager" (the eager chain's rounding points)."""
    dev = x.device
    _on_gpu("x", x, dev)
    _on_gpu("weight", weight, dev)
    if x.dim() != 2 or not _unit_stride(x, 1):
        raise QkrError("x must be [rows, width] with contiguous rows")
    if weight.dtype != x.dtype or not weight.is_contiguous() or weight.numel() != x.shape[1]:
        raise QkrError("weight must be contiguous [width] of x's dtype")
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not _unit_stride(y, 1):
        raise QkrError("out must match x")
    _on_gpu("out", y, dev)
    st = lib().qkr_rms_norm(x.data_ptr(), x.stride(0), y.data_ptr(), y.stride(0), weight.data_ptr(),
                            x.shape[0], x.shape[1], float(eps), _dtype_code(x, numerics), _stream(dev))
    _check(st, "rms_norm")
    return y


def add_rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6,
                 residual: Optional[torch.Tensor] = None, residual_out: Optional[torch.Tensor] = None,
                 out_dtype: Optional[str] = None, scale: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, numerics: str = "contract"):
    """Residual add + RMSNorm of x [rows, width] (qkr_add_rms_norm).

    With `residual`, s = x + residual rounded to x's dtype is written to
    `residual_out` (default: `residual` itself, updated in place) and
    normalised.  out_dtype None: y in x's dtype; "fp8_e4m3": y as OCP E4M3
    codes (torch.float8_e4m3fn) of y / scale, `scale` a one-element float32
    device tensor.  Returns (y, residual_out)."""
    dev = x.device
    _on_gpu("x", x, dev)
    _on_gpu("weight", weight, dev)
    if x.dim() != 2 or not _unit_stride(x, 1):
        raise QkrError("x must be [rows, width] with contiguous rows")
    if weight.dtype != x.dtype or not weight.is_contiguous() or weight.numel() != x.shape[1]:
        raise QkrError("weight must be contiguous [width] of x's dtype")

    def rows_like(name, t):
        _on_gpu(name, t, dev)
        if t.shape != x.shape or t.dtype != x.dtype or not _unit_stride(t, 1):
            raise QkrError(f"{name} must match x")

    if residual is not None:
        rows_like("residual", residual)
        residual_out = residual if residual_out is None else residual_out
        rows_like("residual_out", residual_out)
    elif residual_out is not None:
        raise QkrError("residual_out needs a residual")
    fp8 = out_dtype == "fp8_e4m3"
    if out_dtype not in (None, "fp8_e4m3"):
        raise QkrError(f"unknown out_dtype {out_dtype!r}")
    ydt = torch.float8_e4m3fn if fp8 else x.dtype
    y = torch.empty(x.shape, dtype=ydt, device=dev) if out is None else out
    if y.shape != x.shape or y.dtype != ydt or not _unit_stride(y, 1):
        raise QkrError(f"out must be {tuple(x.shape)} of {ydt}")
    _on_gpu("out", y, dev)
    if fp8:
        if scale is None:
            raise QkrError("FP8 output needs scale")
        _on_gpu("scale", scale, dev)
        if scale.dtype != torch.float32 or scale.numel() != 1:
            raise QkrError("scale must be a one-element float32 tensor")
    st = lib().qkr_add_rms_norm(x.data_ptr(), x.stride(0),
                                residual.data_ptr() if residual is not None else None,
                                residual.stride(0) if residual is not None else 0,
                                residual_out.data_ptr() if residual is not None else None,
                                residual_out.stride(0) if residual is not None else 0,
                                y.data_ptr(), y.stride(0), 1 if fp8 else 0,
                                scale.data_ptr() if fp8 else None, weight.data_ptr(),
                                x.shape[0], x.shape[1], float(eps), _dtype_code(x, numerics), _stream(dev))
    _check(st, "add_rms_norm")
    return y, residual_out


def debug_fp8_e4m3(x: torch.Tensor, scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The row kernel's FP8 E4M3 quantiser applied to a float32 device tensor:
    uint8 codes of x / scale (or of x when scale is None)."""
    _on_gpu("x", x, x.device)
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise QkrError("x must be contiguous float32")
    if scale is not None:
        _on_gpu("scale", scale, x.device)
        if scale.dtype != torch.float32 or scale.numel() != 1:
            raise QkrError("scale must be a one-element float32 tensor")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().qkr_debug_fp8_e4m3(x.data_ptr(), x.numel(), scale.data_ptr() if scale is not None else None,
                                    out.data_ptr(), _stream(x.device)), "debug_fp8_e4m3")
    return out


def qk_norm_rope(q: Optional[torch.Tensor], k: Optional[torch.Tensor], q_weight: Optional[torch.Tensor],
                 k_weight: Optional[torch.Tensor], eps: float = 1e-6, rope: Optional[Rope] = None,
                 q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                 numerics: str = "contract"):
    """Per-head RMSNorm + RoPE of q [.., tokens, Hq, D] and k [.., tokens, Hk, D]."""
    ref = q if q is not None else k
    if ref is None:
        raise QkrError("need q or k")
    dev = ref.device
    squeeze = ref.dim() == 3
    q4 = _rows4("q", q) if q is not None else None
    k4 = _rows4("k", k) if k is not None else None
    r4 = q4 if q4 is not None else k4
    batch, tokens, _, d = r4.shape
    outs = []
    for nm, t4, w, o in (("q", q4, q_weight, q_out), ("k", k4, k_weight, k_out)):
        if t4 is None:
            outs.append(None)
            continue
        _on_gpu(nm, t4, dev)
        if t4.dtype != r4.dtype or t4.shape[0] != batch or t4.shape[1] != tokens or t4.shape[3] != d:
            raise QkrError(f"{nm} does not match the other tensor's batch/tokens/head_dim/dtype")
        if w is None:
            raise QkrError(f"{nm}_weight is required")
        _on_gpu(f"{nm}_weight", w, dev)
        if w.dtype != t4.dtype or not w.is_contiguous() or w.numel() != d:
            raise QkrError(f"{nm}_weight must be contiguous [head_dim] of the activation dtype")
        o4 = torch.empty(t4.shape, dtype=t4.dtype, device=dev) if o is None else _rows4(f"{nm}_out", o)
        if o4.shape != t4.shape or o4.dtype != t4.dtype:
            raise QkrError(f"{nm}_out must match {nm}")
        _on_gpu(f"{nm}_out", o4, dev)
        outs.append(o4)
    qo4, ko4 = outs
    cr = rope.to_c(dev, tokens) if rope is not None else None
    L = lib()
    st = L.qkr_qk_norm_rope(batch, tokens, d, _dtype_code(r4, numerics), float(eps),
                            ctypes.byref(_view(q4)), ctypes.byref(_view(qo4)), q4.shape[2] if q4 is not None else 0,
                            q_weight.data_ptr() if q4 is not None else None,
                            ctypes.byref(_view(k4)), ctypes.byref(_view(ko4)), k4.shape[2] if k4 is not None else 0,
                            k_weight.data_ptr() if k4 is not None else None,
                            ctypes.byref(cr) if cr is not None else None, _stream(dev))
    _check(st, "qk_norm_rope")
    if squeeze:
        qo4 = qo4[0] if qo4 is not None else None
        ko4 = ko4[0] if ko4 is not None else None
    return qo4, ko4


def _slots_view(name: str, cache: torch.Tensor, heads: int, d: int) -> torch.Tensor:
    """[num_slots, heads, d] view of a cache given as [slots, H, D] or as a
    paged [blocks, block_size, H, D] tensor."""
    if cache.dim() == 4:
        if cache.stride(0) != cache.shape[1] * cache.stride(1):
            raise QkrError(f"{name}: blocks and block slots must be evenly strided to be seen as slots")
        cache = cache.view(cache.shape[0] * cache.shape[1], cache.shape[2], cache.shape[3]) \
            if cache.is_contiguous() else cache.flatten(0, 1)
    if cache.dim() != 3 or cache.shape[1] != heads or cache.shape[2] != d or cache.stride(2) != 1:
        raise QkrError(f"{name} must be [slots, {heads}, {d}] (or paged [blocks, block_size, {heads}, {d}])")
    return cache


def qk_norm_rope_cache(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], q_weight: torch.Tensor,
                       k_weight: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                       slot_mapping: torch.Tensor, eps: float = 1e-6, rope: Optional[Rope] = None,
                       q_out: Optional[torch.Tensor] = None, numerics: str = "contract") -> torch.Tensor:
    """Q/K RMSNorm + RoPE of q [tokens, Hq, D] and k [tokens, Hkv, D] with K
    (and V, copied) written into the cache rows slot_mapping [tokens] (int64)
    picks (qkr_qk_norm_rope_cache).  Returns q_out; the caches are updated in
    place."""
    dev = q.device
    for nm, t in (("q", q), ("k", k), ("q_weight", q_weight), ("k_weight", k_weight), ("k_cache", k_cache),
                  ("slot_mapping", slot_mapping)):
        _on_gpu(nm, t, dev)
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise QkrError("q and k must be [tokens, heads, head_dim] with equal tokens and head_dim")
    if k.dtype != q.dtype:
        raise QkrError("q and k must share a dtype")
    for nm, t in (("q", q), ("k", k), ("v", v), ("q_out", q_out)):
        if t is not None and not _unit_stride(t, -1):
            raise QkrError(f"{nm}: the head_dim dimension must be contiguous")
    tokens, hq, d = q.shape
    hkv = k.shape[1]
    if (v is None) != (v_cache is None):
        raise QkrError("v and v_cache come together")
    if v is not None:
        _on_gpu("v", v, dev)
        _on_gpu("v_cache", v_cache, dev)
        if v.shape != k.shape or v.dtype != q.dtype:
            raise QkrError("v must match k")
    for nm, w in (("q_weight", q_weight), ("k_weight", k_weight)):
        if w.dtype != q.dtype or not w.is_contiguous() or w.numel() != d:
            raise QkrError(f"{nm} must be contiguous [head_dim] of the activation dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 or slot_mapping.numel() != tokens \
            or not slot_mapping.is_contiguous():
        raise QkrError("slot_mapping must be contiguous int64 [tokens]")
    kc = _slots_view("k_cache", k_cache, hkv, d)
    if kc.dtype != q.dtype:
        raise QkrError("k_cache must have the activation dtype")
    vc = None
    if v_cache is not None:
        vc = _slots_view("v_cache", v_cache, hkv, d)
        if vc.shape != kc.shape or vc.dtype != q.dtype:
            raise QkrError("v_cache must match k_cache")
    qo = torch.empty_like(q, memory_format=torch.contiguous_format) if q_out is None else q_out
    if qo.shape != q.shape or qo.dtype != q.dtype:
        raise QkrError("q_out must match q")
    _on_gpu("q_out", qo, dev)
    cr = rope.to_c(dev, tokens) if rope is not None else None
    def v4(t):
        return ctypes.byref(_view(t.unsqueeze(0)))

    st = lib().qkr_qk_norm_rope_cache(tokens, d, _dtype_code(q, numerics), float(eps), v4(q), v4(qo), hq,
                                      q_weight.data_ptr(), v4(k), v4(v) if v is not None else None, hkv,
                                      k_weight.data_ptr(), v4(kc), v4(vc) if vc is not None else None,
                                      slot_mapping.data_ptr(), kc.shape[0],
                                      ctypes.byref(cr) if cr is not None else None, _stream(dev))
    _check(st, "qk_norm_rope_cache")
    return qo


def joint_qk_norm_rope(text: dict, image: dict, eps: float = 1e-6, rope: Optional[Rope] = None,
                       out: Optional[Sequence[torch.Tensor]] = None, numerics: str = "contract"):
    """Joint text/image QK RMSNorm + concatenation (text first) + RoPE.

    text / image: dicts with q, k, v [batch, tokens_s, heads, head_dim] views
    (e.g. chunks of a packed QKV projection) and q_weight, k_weight [head_dim].
    Returns joint (q, k, v) [batch, tokens_txt + tokens_img, heads, head_dim].
    """
    q0 = _rows4("text.q", text["q"])
    dev = q0.device
    batch, _, heads, d = q0.shape
    streams = []
    for sname, s in (("text", text), ("image", image)):
        views = {}
        for nm in ("q", "k", "v"):
            t = _rows4(f"{sname}.{nm}", s[nm])
            _on_gpu(f"{sname}.{nm}", t, dev)
            if t.dtype != q0.dtype or t.shape[0] != batch or t.shape[2] != heads or t.shape[3] != d:
                raise QkrError(f"{sname}.{nm} does not match text.q's batch/heads/head_dim/dtype")
            views[nm] = t
        if not (views["q"].shape[1] == views["k"].shape[1] == views["v"].shape[1]):
            raise QkrError(f"{sname}: q, k, v token counts differ")
        for nm in ("q_weight", "k_weight"):
            w = s[nm]
            _on_gpu(f"{sname}.{nm}", w, dev)
            if w.dtype != q0.dtype or not w.is_contiguous() or w.numel() != d:
                raise QkrError(f"{sname}.{nm} must be contiguous [head_dim] of the activation dtype")
        streams.append(_Stream(_view(views["q"]), _view(views["k"]), _view(views["v"]), views["q"].shape[1],
                               s["q_weight"].data_ptr(), s["k_weight"].data_ptr()))
    joint = streams[0].tokens + streams[1].tokens
    shape = (batch, joint, heads, d)
    if out is None:
        outs = [torch.empty(shape, dtype=q0.dtype, device=dev) for _ in range(3)]
    else:
        outs = [_rows4("out", o) for o in out]
        for o in outs:
            _on_gpu("out", o, dev)
            if tuple(o.shape) != shape or o.dtype != q0.dtype:
                raise QkrError(f"outputs must be {shape} of the activation dtype")
    cr = rope.to_c(dev, joint) if rope is not None else None
    st = lib().qkr_joint_qk_norm_rope(batch, heads, d, _dtype_code(q0, numerics), float(eps), ctypes.byref(streams[0]),
                                      ctypes.byref(streams[1]), ctypes.byref(_view(outs[0])),
                                      ctypes.byref(_view(outs[1])), ctypes.byref(_view(outs[2])),
                                      ctypes.byref(cr) if cr is not None else None, _stream(dev))
    _check(st, "joint_qk_norm_rope")
    return tuple(outs)


def _grid_array(grid_thw):
    flat = [int(v) for g in grid_thw for v in g]
    if len(flat) % 3 != 0 or not flat:
        raise QkrError("grid_thw must be a non-empty list of [t, h, w]")
    return (ctypes.c_int32 * len(flat))(*flat), len(flat) // 3, sum(
        flat[i] * flat[i + 1] * flat[i + 2] for i in range(0, len(flat), 3))


def mrope_cos_sin_setup(inv_t: torch.Tensor, inv_h: torch.Tensor, inv_w: torch.Tensor, grid_thw,
                        spatial_merge: int, out: Optional[Sequence[torch.Tensor]] = None):
    """(cos, sin) float32 [3, N, half_t + half_h + half_w] for ViT patch grids.

    Plane a holds only axis a's columns; the other columns are left as they
    were (uninitialised in fresh outputs)."""
    dev = inv_t.device
    for nm, t in (("inv_t", inv_t), ("inv_h", inv_h), ("inv_w", inv_w)):
        _on_gpu(nm, t, dev)
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 1:
            raise QkrError(f"{nm} must be contiguous float32 [half]")
    arr, g, n = _grid_array(grid_thw)
    half = inv_t.numel() + inv_h.numel() + inv_w.numel()
    if out is None:
        cos = torch.empty((3, n, half), dtype=torch.float32, device=dev)
        sin = torch.empty((3, n, half), dtype=torch.float32, device=dev)
    else:
        cos, sin = out
        for nm, t in (("cos", cos), ("sin", sin)):
            _on_gpu(nm, t, dev)
            if tuple(t.shape) != (3, n, half) or t.dtype != torch.float32 or not t.is_contiguous():
                raise QkrError(f"{nm} must be contiguous float32 {(3, n, half)}")
    st = lib().qkr_mrope_cos_sin_setup(inv_t.data_ptr(), inv_t.numel(), inv_h.data_ptr(), inv_h.numel(),
                                       inv_w.data_ptr(), inv_w.numel(), arr, g, int(spatial_merge),
                                       cos.data_ptr(), sin.data_ptr(), n, _stream(dev))
    _check(st, "mrope_cos_sin_setup")
    return cos, sin


def vit_qk_norm_rope(q: Optional[torch.Tensor], k: Optional[torch.Tensor], q_weight: Optional[torch.Tensor],
                     k_weight: Optional[torch.Tensor], eps: float, inv_t: torch.Tensor, inv_h: torch.Tensor,
                     inv_w: torch.Tensor, grid_thw, spatial_merge: int, pairing: str = "neox",
                     q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                     numerics: str = "contract"):
    """ViT per-head RMSNorm + RoPE of q, k [N, heads, head_dim] with (t, h, w)
    positions computed from the patch grids in the kernel (no cos/sin planes)."""
    ref = q if q is not None else k
    if ref is None:
        raise QkrError("need q or k")
    dev = ref.device
    for nm, t in (("inv_t", inv_t), ("inv_h", inv_h), ("inv_w", inv_w)):
        _on_gpu(nm, t, dev)
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 1:
            raise QkrError(f"{nm} must be contiguous float32 [half]")
    if pairing not in PAIRINGS:
        raise QkrError(f"unknown pairing {pairing!r}")
    outs, views = [], []
    for nm, t, w, o in (("q", q, q_weight, q_out), ("k", k, k_weight, k_out)):
        if t is None:
            outs.append(None)
            views.append((None, None, 0, None))
            continue
        if t.dim() != 3 or not _unit_stride(t, -1):
            raise QkrError(f"{nm} must be [tokens, heads, head_dim] with a contiguous last dimension")
        _on_gpu(nm, t, dev)
        if t.dtype != ref.dtype or t.shape[0] != ref.shape[0] or t.shape[2] != ref.shape[2]:
            raise QkrError(f"{nm} does not match the other tensor's tokens/head_dim/dtype")
        if w is None:
            raise QkrError(f"{nm}_weight is required")
        _on_gpu(f"{nm}_weight", w, dev)
        if w.dtype != t.dtype or not w.is_contiguous() or w.numel() != t.shape[2]:
            raise QkrError(f"{nm}_weight must be contiguous [head_dim] of the activation dtype")
        oo = torch.empty(t.shape, dtype=t.dtype, device=dev) if o is None else o
        if oo.shape != t.shape or oo.dtype != t.dtype or not _unit_stride(oo, -1):
            raise QkrError(f"{nm}_out must match {nm}, with a contiguous last dimension")
        _on_gpu(f"{nm}_out", oo, dev)
        outs.append(oo)
        views.append((t, oo, t.shape[1], w))

    def view3(x):
        return _View(None, 0, 0, 0) if x is None else _View(x.data_ptr(), 0, x.stride(0), x.stride(1))

    arr, g, n = _grid_array(grid_thw)
    (qi, qo, qh, qw), (ki, ko, kh, kw) = views
    st = lib().qkr_vit_qk_norm_rope(ref.shape[0], ref.shape[2], _dtype_code(ref, numerics), float(eps),
                                    ctypes.byref(view3(qi)), ctypes.byref(view3(qo)), qh,
                                    qw.data_ptr() if qw is not None else None,
                                    ctypes.byref(view3(ki)), ctypes.byref(view3(ko)), kh,
                                    kw.data_ptr() if kw is not None else None, PAIRINGS[pairing],
                                    inv_t.data_ptr(), inv_t.numel(), inv_h.data_ptr(), inv_h.numel(),
                                    inv_w.data_ptr(), inv_w.numel(), arr, g, int(spatial_merge), _stream(dev))
    _check(st, "vit_qk_norm_rope")
    return outs[0], outs[1]


# ----------------------------------------------------------------------------
# index-map introspection
# ----------------------------------------------------------------------------

def debug_axis_map(mode: str, sections, n_pairs: int, device="cuda") -> torch.Tensor:
    """Axis of each pair from the kernels' own device function."""
    out = torch.empty(n_pairs, dtype=torch.int32, device=device)
    r = _Rope(MODES[mode], 0, 2 * n_pairs, (ctypes.c_int32 * 4)(*(tuple(sections) + (0,) * 4)[:4]),
              None, None, 0, 0, None, None, 0)
    _check(lib().qkr_debug_axis_map(ctypes.byref(r), n_pairs, out.data_ptr(), _stream(out.device)),
           "debug_axis_map")
    return out


def debug_vit_positions(grid_thw, spatial_merge: int, device="cuda") -> torch.Tensor:
    arr, g, n = _grid_array(grid_thw)
    out = torch.empty((3, n), dtype=torch.int32, device=device)
    _check(lib().qkr_debug_vit_positions(arr, g, int(spatial_merge), out.data_ptr(), n, _stream(out.device)),
           "debug_vit_positions")
    return out


def axis_map_host(mode: str, sections, n_pairs: int):
    """Host build of the kernels' axis function (no GPU needed)."""
    out = (ctypes.c_int32 * max(n_pairs, 1))()
    r = _Rope(MODES[mode], 0, 2 * n_pairs, (ctypes.c_int32 * 4)(*(tuple(sections) + (0,) * 4)[:4]),
              None, None, 0, 0, None, None, 0)
    _check(lib().qkr_axis_map_host(ctypes.byref(r), n_pairs, out), "axis_map_host")
    return list(out)[:n_pairs]


def vit_positions_host(grid_thw, spatial_merge: int):
    """Host build of the kernels' ViT position function: [3][N] list."""
    arr, g, n = _grid_array(grid_thw)
    out = (ctypes.c_int32 * (3 * n))()
    _check(lib().qkr_vit_positions_host(arr, g, int(spatial_merge), out, n), "vit_positions_host")
    flat = list(out)
    return [flat[0:n], flat[n:2 * n], flat[2 * n:3 * n]]


qkr_rms_norm = rms_norm
qkr_add_rms_norm = add_rms_norm
qkr_qk_norm_rope = qk_norm_rope
qkr_qk_norm_rope_cache = qk_norm_rope_cache
qkr_joint_qk_norm_rope = joint_qk_norm_rope
qkr_mrope_cos_sin_setup = mrope_cos_sin_setup
qkr_vit_qk_norm_rope = vit_qk_norm_rope
