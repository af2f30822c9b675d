"""Seeded synthetic inputs for the five workloads (shared by tests, smoke and bench).

This module only draws and lays out input data: it holds none of the method's
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
it.  Random values are drawn in float32 with numpy and converted to bf16 by
torch (round to nearest even); the oracle receives the decoded bf16 values, the
GPU the bf16 bits, so both read identical numbers.

Workloads (shapes follow the pages' own cases):
  tiny    Q, K fp32 [4, 2, 64], NeoX 1-D RoPE, theta 1e4, positions 0..3.
  rows    plain row RMSNorm, bf16 [t, 5120], t in {1, 32, 4096} (decode and
          prefill rows of the Vulkan RmsNorm page, the 4096-token regime of the
          vectorized-variance page).
  joint   text 512 + image 4096 tokens, 24 heads x 128, Q/K/V as chunked views
          of a packed bf16 [1, S, 3*24*128] projection; 3-axis RoPE with
          [8, 28, 28] pairs per axis, positions (0, row, col) on a 64 x 64
          grid and (0, 0, 0) for text (the Ovis-Image double-block operator
          case).
  imrope  8192 tokens, 16 Q + 8 K heads x 128 bf16, sections [24, 20, 20, 0],
          four planes of i.i.d. uniform int positions in [0, 8192), theta 1e6,
          launched in 2048-token chunks (the Qwen3-VL text rotation).
  vit     grids [[1,64,64],[2,32,48],[1,28,28]], merge 2, inv_freq lengths
          8/16/16, Q, K bf16 [7952, 16, 80] (the ViT mrope setup + apply).
"""
from dataclasses import dataclass, field

import numpy as np
import torch

SEED = 20261008
EPS = 1e-6


def _rng(*stream):
    return np.random.default_rng([SEED, *stream])


def normal(shape, mean, std, *stream) -> np.ndarray:
    return _rng(*stream).normal(mean, std, size=shape).astype(np.float32)


def to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> CPU torch tensor of dtype ("f32" or "bf16")."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def as_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 decode of a CPU tensor (for the oracle)."""
    return t.detach().to("cpu").float().numpy()


def inv_freq_ladder(theta: float, dim: int) -> np.ndarray:
    """Standard RoPE inverse frequencies theta^(-2j/dim), j < dim/2, float32."""
    j = np.arange(dim // 2, dtype=np.float64)
    return (theta ** (-2.0 * j / dim)).astype(np.float32)


# ---------------------------------------------------------------- tiny -----
@dataclass
class Tiny:
    q: torch.Tensor
    k: torch.Tensor
    q_weight: torch.Tensor
    k_weight: torch.Tensor
    inv_freq: np.ndarray
    positions: np.ndarray   # int32 [1, tokens]
    rotary_dim: int
    dtype: str = "f32"
    eps: float = EPS


def tiny(tokens=4, heads=2, head_dim=64, dtype="f32", seed_stream=0) -> Tiny:
    s = (1, seed_stream)
    return Tiny(
        q=to_dtype(normal((tokens, heads, head_dim), 0.0, 1.0, *s, 0), dtype),
        k=to_dtype(normal((tokens, heads, head_dim), 0.0, 1.0, *s, 1), dtype),
        q_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, 2), dtype),
        k_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, 3), dtype),
        inv_freq=inv_freq_ladder(1e4, head_dim),
        positions=np.arange(tokens, dtype=np.int32)[None, :],
        rotary_dim=head_dim,
        dtype=dtype,
    )


# ---------------------------------------------------------------- rows -----
@dataclass
class Rows:
    x: torch.Tensor
    weight: torch.Tensor
    eps: float = EPS


def rows(t: int, width: int = 5120, dtype: str = "bf16", seed_stream=0) -> Rows:
    s = (2, t, width, seed_stream)
    return Rows(x=to_dtype(normal((t, width), 0.0, 1.0, *s, 0), dtype),
                weight=to_dtype(normal((width,), 1.0, 0.1, *s, 1), dtype))


# --------------------------------------------------------------- joint -----
@dataclass
class Stream:
    qkv: torch.Tensor        # packed [batch, tokens, 3*heads*head_dim]
    q_weight: torch.Tensor
    k_weight: torch.Tensor

    def view(self, which: int, heads: int, head_dim: int) -> torch.Tensor:
        """Q (0), K (1) or V (2) as a strided [batch, tokens, heads, head_dim] view."""
        b, s, _ = self.qkv.shape
        return self.qkv.view(b, s, 3, heads, head_dim)[:, :, which]


@dataclass
class Joint:
    text: Stream
    image: Stream
    heads: int
    head_dim: int
    positions: np.ndarray    # int32 [3, tokens_txt + tokens_img]
    sections: tuple          # pairs per axis (t, h, w, 0)
    inv_freq: np.ndarray     # float32 [head_dim/2], axis ladders concatenated
    eps: float = EPS


def joint(tokens_txt=512, grid=(64, 64), heads=24, head_dim=128, axes_pairs=(8, 28, 28),
          batch=1, dtype="bf16", theta=1e4, seed_stream=0) -> Joint:
    s = (3, tokens_txt, grid[0], grid[1], heads, head_dim, batch, seed_stream)
    tokens_img = grid[0] * grid[1]
    hd = heads * head_dim

    def stream(k, n):
        return Stream(qkv=to_dtype(normal((batch, n, 3 * hd), 0.0, 1.0, *s, k, 0), dtype),
                      q_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, k, 1), dtype),
                      k_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, k, 2), dtype))

    img = np.arange(tokens_img, dtype=np.int32)
    pos = np.zeros((3, tokens_txt + tokens_img), np.int32)
    pos[1, tokens_txt:] = img // grid[1]
    pos[2, tokens_txt:] = img % grid[1]
    inv = np.concatenate([inv_freq_ladder(theta, 2 * p) for p in axes_pairs])
    return Joint(text=stream(0, tokens_txt), image=stream(1, tokens_img), heads=heads,
                 head_dim=head_dim, positions=pos, sections=tuple(axes_pairs) + (0,),
                 inv_freq=inv)


# -------------------------------------------------------------- imrope -----
@dataclass
class Imrope:
    q: torch.Tensor
    k: torch.Tensor
    q_weight: torch.Tensor
    k_weight: torch.Tensor
    positions: np.ndarray    # int32 [4, tokens]
    sections: tuple
    inv_freq: np.ndarray
    chunk: int
    eps: float = EPS


def imrope(tokens=8192, q_heads=16, k_heads=8, head_dim=128, sections=(24, 20, 20, 0),
           theta=1e6, chunk=2048, dtype="bf16", seed_stream=0) -> Imrope:
    s = (4, tokens, q_heads, k_heads, head_dim, seed_stream)
    pos = _rng(*s, 4).integers(0, 8192, size=(4, tokens), dtype=np.int32)
    return Imrope(q=to_dtype(normal((tokens, q_heads, head_dim), 0.0, 1.0, *s, 0), dtype),
                  k=to_dtype(normal((tokens, k_heads, head_dim), 0.0, 1.0, *s, 1), dtype),
                  q_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, 2), dtype),
                  k_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, 3), dtype),
                  positions=pos, sections=tuple(sections),
                  inv_freq=inv_freq_ladder(theta, head_dim), chunk=chunk)


# ----------------------------------------------------------------- vit -----
@dataclass
class Vit:
    grid_thw: list
    merge: int
    inv_t: np.ndarray
    inv_h: np.ndarray
    inv_w: np.ndarray
    q: torch.Tensor
    k: torch.Tensor
    q_weight: torch.Tensor
    k_weight: torch.Tensor
    eps: float = EPS

    @property
    def n_tokens(self) -> int:
        return sum(t * h * w for t, h, w in self.grid_thw)

    @property
    def half_rot(self) -> int:
        return self.inv_t.size + self.inv_h.size + self.inv_w.size


def vit(grid_thw=((1, 64, 64), (2, 32, 48), (1, 28, 28)), merge=2, halves=(8, 16, 16),
        heads=16, head_dim=80, theta=1e4, dtype="bf16", seed_stream=0) -> Vit:
    grid_thw = [list(map(int, g)) for g in grid_thw]
    n = sum(t * h * w for t, h, w in grid_thw)
    s = (5, n, heads, head_dim, seed_stream)
    return Vit(grid_thw=grid_thw, merge=merge,
               inv_t=inv_freq_ladder(theta, 2 * halves[0]),
               inv_h=inv_freq_ladder(theta, 2 * halves[1]),
               inv_w=inv_freq_ladder(theta, 2 * halves[2]),
               q=to_dtype(normal((n, heads, head_dim), 0.0, 1.0, *s, 0), dtype),
               k=to_dtype(normal((n, heads, head_dim), 0.0, 1.0, *s, 1), dtype),
               q_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, 2), dtype),
               k_weight=to_dtype(normal((head_dim,), 1.0, 0.1, *s, 3), dtype))
