"""Layouts the Python binding must refuse or accept, on GPU tensors.

The kernels read and write every row as contiguous head_dim elements, so a
view whose last dimension is strided is refused before the library is called
(nothing launches).  A 1-D rotation reads one position plane, so positions
given as the first of several overlapping planes (an expanded tensor) are
accepted and give the same bits as a plain one-plane tensor.
"""
import pytest
import torch

import transformer_qk_rmsnorm_amd as qkr
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def bf(*shape):
    g = torch.Generator(device=DEV).manual_seed(W.SEED)
    return torch.randn(*shape, device=DEV, generator=g).to(BF)


def strided(*shape):
    """A bf16 view of `shape` whose last dimension has stride 2."""
    return bf(*shape, 2)[..., 0]


def test_cache_refuses_a_strided_head_dim():
    t, hq, hkv, d = 8, 4, 2, 64
    w = torch.ones(d, dtype=BF, device=DEV)
    slots = torch.arange(t, dtype=torch.int64, device=DEV)
    base = dict(q=bf(t, hq, d), k=bf(t, hkv, d), v=bf(t, hkv, d))
    for name, bad in (("q", strided(t, hq, d)), ("k", strided(t, hkv, d)), ("v", strided(t, hkv, d)),
                      ("q_out", strided(t, hq, d))):
        args = dict(base)
        q_out = bad if name == "q_out" else None
        if name != "q_out":
            args[name] = bad
        kc, vc = bf(32, hkv, d), bf(32, hkv, d)
        kc0, vc0 = kc.clone(), vc.clone()
        with pytest.raises(qkr.QkrError, match="contiguous"):
            qkr.qk_norm_rope_cache(args["q"], args["k"], args["v"], w, w, kc, vc, slots, W.EPS, None, q_out=q_out)
        torch.cuda.synchronize()
        assert torch.equal(kc, kc0) and torch.equal(vc, vc0), f"{name}: a refused call wrote the cache"


def test_vit_refuses_a_strided_output():
    grid, merge, d = [[1, 4, 4]], 2, 64
    n, h = 16, 2
    w = torch.ones(d, dtype=BF, device=DEV)
    inv = [torch.full((m,), 0.5, dtype=torch.float32, device=DEV) for m in (4, 6, 6)]
    q, k = bf(n, h, d), bf(n, h, d)
    for kwargs in (dict(q_out=strided(n, h, d)), dict(k_out=strided(n, h, d))):
        with pytest.raises(qkr.QkrError, match="contiguous"):
            qkr.vit_qk_norm_rope(q, k, w, w, W.EPS, *inv, grid, merge, **kwargs)


def test_one_d_positions_from_overlapping_planes():
    t, h, d, length = 40, 4, 128, 64
    q, k = bf(t, h, d), bf(t, h, d)
    w = torch.ones(d, dtype=BF, device=DEV)
    inv = torch.from_numpy(W.inv_freq_ladder(1e4, d)).to(DEV)
    plain = torch.randint(0, 4096, (1, length), dtype=torch.int32, device=DEV)
    expanded = plain.expand(3, length)                 # stride(0) == 0: three views of one plane
    assert expanded.stride(0) == 0
    out = []
    for pos in (plain, expanded):
        rope = qkr.Rope("1d", d, "neox", inv_freq=inv, positions=pos, token_base=5)
        out.append(qkr.qk_norm_rope(q, k, w, w, W.EPS, rope))
    torch.cuda.synchronize()
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
