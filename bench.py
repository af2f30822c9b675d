#!/usr/bin/env python3
"""Benchmark of the fused QK RMSNorm + RoPE hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload joint|joint-neox|imrope|vit|vit-fused|rows1|rows32|
                                                 rows4096|addrms4096|addrms4096-fp8|addrms1|cache|tiny|copy]

Prints one JSON line.  A step is one pass of the workload's hot path over one
batch of synthetic input already resident in HBM (default workload: the joint
text/image QK RMSNorm + concatenation + 3-axis RoPE, 512 text + 4096 image
tokens, 24 heads x 128, bf16; one launch per step).  Consecutive steps rotate
over several input/output buffer sets whose total exceeds the 256 MB
last-level (Infinity) cache, so every step streams from HBM.

value   = algorithmic bytes per step / time per step (GB/s), whole job.
roofline.achieved = algorithmic bytes per launch of the dominant kernel /
          its average launch duration: HIP events recorded on the stream the
          kernels run on bracket the timed region (exactly K steps replayed
          from captured graphs, launches back to back), divided by the
          launches it holds.
cpu_baseline: the CPU oracle on a bounded sample of the same workload, on
          the host cores (single-threaded C).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 << 20         # MI355X Infinity Cache
METRIC = "fused QK-norm+RoPE µs/call and achieved HBM GB/s (% of peak), 1 MI355X"


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="joint",
                    choices=["joint", "joint-neox", "imrope", "vit", "vit-fused", "rows1", "rows32", "rows4096",
                             "addrms4096", "addrms4096-fp8", "addrms1", "cache", "tiny", "copy"])
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0: enough to exceed the cache)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget (0: skip)")
    ap.add_argument("--variant", default=None,
                    help="comma-separated kernel variant overrides (qkr_set_variant_override)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured HIP graph")
    return ap.parse_args()


class Workload:
    """name, description, bytes per step, dominant-kernel bytes per launch,
    launches of it per step, make_set() -> state, step(state) launches the
    path, cpu_step() runs the oracle on one step's input."""


def build_joint(pairing):
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.joint()
    H, D = case.heads, case.head_dim
    st, si = case.text.qkv.shape[1], case.image.qkv.shape[1]
    joint = st + si
    dev = torch.device("cuda")
    pos = torch.from_numpy(case.positions).to(dev)
    inv = torch.from_numpy(case.inv_freq).to(dev)
    rope = qkr.Rope("axes", D, pairing, inv_freq=inv, positions=pos, sections=case.sections)

    def make_set():
        g = {}
        for nm, s in (("text", case.text), ("image", case.image)):
            qkv = s.qkv.to(dev)
            v = qkv.view(qkv.shape[0], qkv.shape[1], 3, H, D)
            g[nm] = {"q": v[:, :, 0], "k": v[:, :, 1], "v": v[:, :, 2], "q_weight": s.q_weight.to(dev),
                     "k_weight": s.k_weight.to(dev), "_qkv": qkv}
        outs = [torch.empty((1, joint, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
        return g, outs

    def step(state):
        g, outs = state
        qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope, out=outs)

    qkv_bytes = joint * 3 * H * D * 2
    nbytes = 2 * qkv_bytes + case.positions.nbytes + 4 * D * 2 + case.inv_freq.nbytes

    def cpu_step():
        import oracle

        def stream(s):
            return {"q": W.as_f32(s.view(0, H, D)), "k": W.as_f32(s.view(1, H, D)), "v": W.as_f32(s.view(2, H, D)),
                    "q_weight": W.as_f32(s.q_weight), "k_weight": W.as_f32(s.k_weight)}

        tx, im = stream(case.text), stream(case.image)
        orope = oracle.Rope("axes", D, pairing, inv_freq=case.inv_freq, sections=case.sections,
                            positions=case.positions)

        def run():
            oracle.joint_qk_norm_rope(tx, im, case.eps, orope, "bf16")
        return run

    w = Workload()
    w.name = f"joint text/image QK RMSNorm + cat + 3-axis RoPE ({pairing})"
    w.config = {"workload": w.name, "text_tokens": st, "image_tokens": si, "heads": H, "head_dim": D,
                "axes_pairs": list(case.sections[:3]), "theta": 1e4, "eps": case.eps, "batch": 1}
    w.step_bytes = nbytes
    w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = "the full joint step (512 text + 4096 image tokens, Q/K/V)"
    return w


def build_imrope():
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.imrope()
    dev = torch.device("cuda")
    T, chunk = case.q.shape[0], case.chunk
    pos = torch.from_numpy(case.positions).to(dev)
    inv = torch.from_numpy(case.inv_freq).to(dev)
    ropes = [qkr.Rope("imrope", 128, "neox", inv_freq=inv, positions=pos, sections=case.sections, token_base=b)
             for b in range(0, T, chunk)]
    qw, kw = case.q_weight.to(dev), case.k_weight.to(dev)

    def make_set():
        q, k = case.q.to(dev), case.k.to(dev)
        return q, k, torch.empty_like(q), torch.empty_like(k)

    def step(state):
        q, k, qo, ko = state
        for r in ropes:
            b = r.token_base
            qkr.qk_norm_rope(q[b:b + chunk], k[b:b + chunk], qw, kw, case.eps, r, q_out=qo[b:b + chunk],
                             k_out=ko[b:b + chunk])

    rows = case.q.shape[1] + case.k.shape[1]
    chunk_bytes = 2 * chunk * rows * 128 * 2 + 4 * chunk * 4 + 2 * 128 * 2 + case.inv_freq.nbytes

    def cpu_step():
        import oracle
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)
        orope = oracle.Rope("imrope", 128, "neox", inv_freq=case.inv_freq, sections=case.sections,
                            positions=case.positions)

        def run():
            oracle.qk_norm_rope(qf, wq, case.eps, orope)
            oracle.qk_norm_rope(kf, wk, case.eps, orope)
        return run

    w = Workload()
    w.name = "IMROPE after per-head QK RMSNorm, 2048-token chunks"
    w.config = {"workload": w.name, "tokens": T, "chunk": chunk, "q_heads": case.q.shape[1],
                "k_heads": case.k.shape[1], "head_dim": 128, "sections": list(case.sections), "theta": 1e6}
    w.step_bytes = chunk_bytes * (T // chunk)
    w.launch_bytes = chunk_bytes
    w.launches = T // chunk
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = "all 8192 tokens (4 chunks), Q and K"
    return w


def build_vit():
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.vit()
    dev = torch.device("cuda")
    n, half = case.n_tokens, case.half_rot
    inv = [torch.from_numpy(a).to(dev) for a in (case.inv_t, case.inv_h, case.inv_w)]
    secs = (case.inv_t.size, case.inv_h.size, case.inv_w.size, 0)
    qw, kw = case.q_weight.to(dev), case.k_weight.to(dev)

    def make_set():
        q, k = case.q.to(dev), case.k.to(dev)
        cos = torch.empty((3, n, half), device=dev)
        sin = torch.empty((3, n, half), device=dev)
        return q, k, torch.empty_like(q), torch.empty_like(k), cos, sin

    def step(state):
        q, k, qo, ko, cos, sin = state
        qkr.mrope_cos_sin_setup(*inv, case.grid_thw, case.merge, out=(cos, sin))
        rope = qkr.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=cos, sin_planes=sin)
        qkr.qk_norm_rope(q, k, qw, kw, case.eps, rope, q_out=qo, k_out=ko)

    heads = case.q.shape[1]
    planes = 2 * n * half * 4
    apply_bytes = 4 * n * heads * 2 * half * 2 + planes + 2 * 2 * half * 2

    def cpu_step():
        import oracle
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)

        def run():
            c, s = oracle.vit_cos_sin(case.inv_t, case.inv_h, case.inv_w, case.grid_thw, case.merge)
            orope = oracle.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=c, sin_planes=s)
            oracle.qk_norm_rope(qf, wq, case.eps, orope)
            oracle.qk_norm_rope(kf, wk, case.eps, orope)
        return run

    w = Workload()
    w.name = "ViT mrope cos/sin setup + apply after per-head QK RMSNorm"
    w.config = {"workload": w.name, "grid_thw": case.grid_thw, "spatial_merge": case.merge, "tokens": n,
                "heads": heads, "head_dim": 2 * half, "halves": list(secs[:3])}
    w.step_bytes = planes + apply_bytes
    w.launch_bytes = apply_bytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = "setup + apply over all 7952 tokens"
    return w


def build_vit_fused():
    """ViT workload with the setup folded into the rotation (no planes)."""
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.vit()
    dev = torch.device("cuda")
    n, half = case.n_tokens, case.half_rot
    inv = [torch.from_numpy(a).to(dev) for a in (case.inv_t, case.inv_h, case.inv_w)]
    qw, kw = case.q_weight.to(dev), case.k_weight.to(dev)

    def make_set():
        q, k = case.q.to(dev), case.k.to(dev)
        return q, k, torch.empty_like(q), torch.empty_like(k)

    def step(state):
        q, k, qo, ko = state
        qkr.vit_qk_norm_rope(q, k, qw, kw, case.eps, *inv, case.grid_thw, case.merge, q_out=qo, k_out=ko)

    heads = case.q.shape[1]
    nbytes = 4 * n * heads * 2 * half * 2 + 2 * 2 * half * 2 + 4 * half

    def cpu_step():
        import oracle
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)

        def run():
            oracle.vit_qk_norm_rope(qf, wq, case.eps, case.inv_t, case.inv_h, case.inv_w, case.grid_thw, case.merge)
            oracle.vit_qk_norm_rope(kf, wk, case.eps, case.inv_t, case.inv_h, case.inv_w, case.grid_thw, case.merge)
        return run

    w = Workload()
    w.name = "ViT QK RMSNorm + mrope with positions from the grids (setup folded in)"
    w.config = {"workload": w.name, "grid_thw": case.grid_thw, "spatial_merge": case.merge, "tokens": n,
                "heads": heads, "head_dim": 2 * half, "halves": [case.inv_t.size, case.inv_h.size, case.inv_w.size]}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = "all 7952 tokens, Q and K"
    return w


def build_rows(t):
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.rows(t)
    dev = torch.device("cuda")
    wgt = case.weight.to(dev)

    def make_set():
        x = case.x.to(dev)
        return x, torch.empty_like(x)

    def step(state):
        x, y = state
        qkr.rms_norm(x, wgt, case.eps, out=y)

    width = case.x.shape[1]
    nbytes = 2 * t * width * 2 + width * 2

    def cpu_step():
        import oracle
        xf, wf = W.as_f32(case.x), W.as_f32(case.weight)

        def run():
            oracle.rms_norm(xf, wf, case.eps, "bf16")
        return run

    w = Workload()
    w.name = f"plain row RMSNorm bf16 [{t}, {width}]"
    w.config = {"workload": w.name, "rows": t, "width": width, "eps": case.eps}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = f"the full [{t}, {width}] input"
    return w


def build_cache():
    """IMROPE QK norm + RoPE of 8192 tokens (16 Q, 8 K/V heads x 128, bf16) with
    K and V written into a paged cache (2048 blocks x 16 slots) through a
    random injective slot mapping, one launch."""
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.imrope()
    dev = torch.device("cuda")
    T, H, KV, D = case.q.shape[0], case.q.shape[1], case.k.shape[1], 128
    blocks, bs = 2048, 16
    v_host = W.to_dtype(W.normal((T, KV, D), 0.0, 1.0, 61), "bf16")
    slots_host = torch.from_numpy(np.random.default_rng(61).permutation(blocks * bs)[:T].astype(np.int64))
    pos = torch.from_numpy(case.positions).to(dev)
    inv = torch.from_numpy(case.inv_freq).to(dev)
    rope = qkr.Rope("imrope", D, "neox", inv_freq=inv, positions=pos, sections=case.sections)
    qw, kw = case.q_weight.to(dev), case.k_weight.to(dev)
    slots = slots_host.to(dev)

    def make_set():
        q, k, v = case.q.to(dev), case.k.to(dev), v_host.to(dev)
        kc = torch.zeros((blocks, bs, KV, D), dtype=torch.bfloat16, device=dev)
        return q, k, v, kc, torch.zeros_like(kc), torch.empty_like(q)

    def step(state):
        q, k, v, kc, vc, qo = state
        qkr.qk_norm_rope_cache(q, k, v, qw, kw, kc, vc, slots, case.eps, rope, q_out=qo)

    nbytes = 2 * T * (H + 2 * KV) * D * 2 + T * 8 + case.positions.nbytes + 2 * D * 2 + case.inv_freq.nbytes

    def cpu_step():
        import oracle
        orope = oracle.Rope("imrope", D, "neox", inv_freq=case.inv_freq, positions=case.positions,
                            sections=case.sections)
        q, k, v = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(v_host)
        wq, wk = W.as_f32(case.q_weight), W.as_f32(case.k_weight)
        kc0 = np.zeros((blocks * bs, KV, D), np.float32)
        sl = slots_host.numpy()

        def run():
            oracle.qk_norm_rope_cache(q, k, v, wq, wk, case.eps, orope, sl, kc0, kc0)
        return run

    w = Workload()
    w.name = "IMROPE QK RMSNorm + RoPE with K/V written into a paged cache by slot mapping"
    w.config = {"workload": w.name, "tokens": T, "q_heads": H, "kv_heads": KV, "head_dim": D,
                "sections": list(case.sections), "cache_blocks": blocks, "block_size": bs}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = "all 8192 tokens"
    return w


def build_addrms(t, fp8):
    """Residual add + RMSNorm of bf16 [t, 5120] rows, bf16 or static FP8 E4M3 output."""
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.rows(t)
    res = W.rows(t, seed_stream=1).x
    dev = torch.device("cuda")
    wgt = case.weight.to(dev)
    scale = torch.tensor([0.02], dtype=torch.float32, device=dev)

    def make_set():
        x, r = case.x.to(dev), res.to(dev)
        y = torch.empty(x.shape, dtype=torch.float8_e4m3fn if fp8 else x.dtype, device=dev)
        return x, r, torch.empty_like(x), y

    def step(state):
        x, r, s_out, y = state
        qkr.add_rms_norm(x, wgt, case.eps, residual=r, residual_out=s_out, out_dtype="fp8_e4m3" if fp8 else None,
                         scale=scale, out=y)

    width = case.x.shape[1]
    nbytes = t * width * (2 + 2 + 2 + (1 if fp8 else 2)) + width * 2 + (4 if fp8 else 0)

    def cpu_step():
        import oracle
        xf, rf, wf = W.as_f32(case.x), W.as_f32(res), W.as_f32(case.weight)

        def run():
            oracle.add_rms_norm(xf, wf, case.eps, rf, "bf16", "fp8_e4m3" if fp8 else "bf16", 0.02)
        return run

    w = Workload()
    w.name = f"residual add + RMSNorm bf16 [{t}, {width}] -> {'FP8 E4M3 (static scale)' if fp8 else 'bf16'}"
    w.config = {"workload": w.name, "rows": t, "width": width, "eps": case.eps, "out": "fp8_e4m3" if fp8 else "bf16"}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "bf16"
    w.sample = f"the full [{t}, {width}] input"
    return w


def build_tiny():
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.tiny()
    dev = torch.device("cuda")
    rope = qkr.Rope("1d", 64, "neox", inv_freq=torch.from_numpy(case.inv_freq).to(dev),
                    positions=torch.from_numpy(case.positions).to(dev))
    ws = case.q_weight.to(dev), case.k_weight.to(dev)

    def make_set():
        q, k = case.q.to(dev), case.k.to(dev)
        return q, k, torch.empty_like(q), torch.empty_like(k)

    def step(state):
        q, k, qo, ko = state
        qkr.qk_norm_rope(q, k, ws[0], ws[1], case.eps, rope, q_out=qo, k_out=ko)

    nbytes = 2 * 2 * q_numel(case) * 4 + 2 * 64 * 4 + 4 * 4 + 32 * 4

    def cpu_step():
        import oracle
        orope = oracle.Rope("1d", 64, "neox", inv_freq=case.inv_freq, positions=case.positions)
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)

        def run():
            oracle.qk_norm_rope(qf, wq, case.eps, orope, "f32")
            oracle.qk_norm_rope(kf, wk, case.eps, orope, "f32")
        return run

    w = Workload()
    w.name = "tiny fp32 QK RMSNorm + NeoX RoPE [4, 2, 64]"
    w.config = {"workload": w.name, "tokens": 4, "heads": 2, "head_dim": 64}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_step = make_set, step, cpu_step
    w.dtype = "f32"
    w.sample = "the full [4, 2, 64] input"
    return w


def q_numel(case):
    return case.q.numel()


def build_copy():
    """Calibration only: a plain device copy of 256 MiB (read + write), the
    reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    nbytes = 256 << 20
    dev = torch.device("cuda")

    def make_set():
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        return src, torch.empty_like(src)

    def step(state):
        src, dst = state
        dst.copy_(src)

    w = Workload()
    w.name = "plain device copy, 256 MiB (counter calibration)"
    w.config = {"workload": w.name, "bytes_copied": nbytes}
    w.step_bytes = w.launch_bytes = 2 * nbytes
    w.launches = 1
    w.make_set, w.step = make_set, step
    w.cpu_step = None
    w.dtype = "f32"
    w.sample = "none"
    return w


KERNEL_SOURCES = ["transformer_qk_rmsnorm_amd/csrc/" + f for f in
                  ("qkr_kernels.hip", "qkr_rope_part.hip", "qkr_rope_kernel.hpp", "qkr_device.hpp",
                   "qkr_internal.hpp", "qkr_fastdiv.hpp")]


def kernel_source_hash():
    """Hash of the kernel sources' code with comments removed: the counters
    depend on the code, so a comment edit keeps them valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(text.encode("utf-8"))
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch from the committed counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by
    what the counter reads for a plain copy of known size), or None when no
    summary exists or the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["write_scale"])
        return round(fetch + write)
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, seconds):
    run = w.cpu_step()
    run()   # warm (page in, first-touch)
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbs = w.step_bytes * reps / el / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "us_per_step": round(el / reps * 1e6, 1),
            "sample": f"{reps} x {w.sample}, single-threaded C oracle"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: every row of the path is per-row "
                                   "independent and shards without communication; run with --gpus 1"}))
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one process, one GPU; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_qk_rmsnorm_amd as qkr

    builders = {"joint": lambda: build_joint("adjacent"), "joint-neox": lambda: build_joint("neox"),
                "imrope": build_imrope, "vit": build_vit, "vit-fused": build_vit_fused, "rows1": lambda: build_rows(1),
                "rows32": lambda: build_rows(32), "rows4096": lambda: build_rows(4096), "tiny": build_tiny,
                "addrms4096": lambda: build_addrms(4096, False), "addrms4096-fp8": lambda: build_addrms(4096, True),
                "addrms1": lambda: build_addrms(1, False), "cache": build_cache,
                "copy": build_copy}
    w = builders[args.workload]()
    nsets = args.sets or max(3, -(-2 * MALL_BYTES // max(w.step_bytes, 1)))
    nsets = min(nsets, 64)
    sets = [w.make_set() for _ in range(nsets)]
    for name in (args.variant.split(",") if args.variant else []):
        qkr.set_variant_override(name)
    stream = torch.cuda.current_stream()

    for i in range(args.warmup):
        w.step(sets[i % nsets])
    torch.cuda.synchronize()
    variant = qkr.last_variant()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if args.eager:
        K = args.steps
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(K):
            w.step(sets[i % nsets])
        t_end.record(stream)
    else:
        # Exactly K steps cycling over the buffer sets, captured in graphs of
        # up to 1024 kernel launches (plus one graph for the remainder);
        # replaying a graph runs its launches back to back with no host work
        # in between.  Each replay boundary costs several microseconds of idle
        # GPU, so the graphs are long; a single graph of 4096 launches measured
        # slower per launch (IMROPE chunk 6.39 us against 5.93-5.97 us with
        # 200 to 2000 launches split over graphs of up to 1024).
        K = args.steps
        chunk = max(1, min(K, 1024 // w.launches))
        plan = [chunk] * (K // chunk) + ([K % chunk] if K % chunk else [])
        graphs = {}
        for n in sorted(set(plan)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    w.step(sets[i % nsets])
            g.replay()
            graphs[n] = g
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        t_start.record(stream)
        for n in plan:
            graphs[n].replay()
        t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    launch_us = ms_per_step * 1e3 / w.launches

    value = w.step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = w.launch_bytes / (launch_us * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(launch_us, 3),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, workloads.py)",
        "config": dict(w.config, buffer_sets=nsets, variant=variant, bytes_per_step=w.step_bytes,
                       launch="eager" if args.eager else "hipGraph replay"),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.workload),
                     "bytes_per_launch": w.launch_bytes, "kernel": variant},
    }
    if args.cpu_seconds > 0 and w.cpu_step is not None:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
