#!/usr/bin/env python3
"""Benchmark of the fused QK RMSNorm + RoPE hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--numerics contract|eager]
                    [--workload joint|joint-neox|imrope|vit|vit-fused|rows1|rows32|rows4096|
                                addrms4096|addrms4096-fp8|addrms1|cache|tiny|copy]

Prints one JSON line.  A step is one pass of the workload's hot path over one
batch of synthetic input already resident in HBM (default workload: the joint
text/image QK RMSNorm + concatenation + 3-axis RoPE, 512 text + 4096 image
tokens, 24 heads x 128, bf16; one launch per step).  Consecutive steps rotate
over several input/output buffer sets whose total exceeds the 256 MB
last-level (Infinity) cache, so every step streams from HBM.

value   = algorithmic bytes per step / time per step (GB/s), whole job, over
          exactly K steps bracketed by HIP events on the stream the kernels
          run on (replays of captured graphs, launches back to back).
gpu_samples: the same K steps cut into at least six samples at graph-replay
          boundaries, each event-timed: median, minimum and maximum per step.
warm-up: W steps launched one by one, then the whole K-step plan of graph
          replays once, untimed, so that the GPU's clocks have settled under
          sustained load before the timed pass (after a short warm-up the first
          milliseconds of a run read several percent slow).
roofline.achieved = algorithmic bytes per launch of the dominant kernel /
          its average launch duration over the K steps.
cpu_baseline: the CPU oracle (plain C, double precision) on the same step,
          once on all the host cores the process may use (the step's rows
          split into one contiguous part per thread; the oracle releases the
          interpreter lock while it runs) and once on one thread; median of 5
          repetitions each; `value` is the all-cores leg.
--numerics eager times the eager-chain rounding points instead of the
          contract (the preset's cost).
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
GPU_SAMPLES = 6                # event-timed samples of the K steps
CPU_REPS = 5                   # repetitions of each CPU leg (median)
CPU_MAX_THREADS = 16           # the host share of one GPU

NUMERICS = "contract"          # set from --numerics before any workload is built
SLOTS = "random"               # set from --slots (cache workload)
STREAMS = 1                    # set from --streams (imrope)


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="joint",
                    choices=["joint", "joint-neox", "imrope", "vit", "vit-fused", "rows1", "rows32", "rows4096",
                             "addrms4096", "addrms4096-fp8", "addrms1", "cache", "tiny", "copy"])
    ap.add_argument("--numerics", default="contract", choices=["contract", "eager"])
    ap.add_argument("--slots", default="random", choices=["random", "blocks"],
                    help="cache workload's slot map: random slots (each token's K/V rows land alone), or "
                         "blocks (16 consecutive tokens fill one block, blocks in random order)")
    ap.add_argument("--streams", type=int, default=1,
                    help="imrope: issue the chunk launches of a step round-robin on this many streams "
                         "(default priority) that fork from and join the main stream, so one chunk's ramp "
                         "can overlap the previous chunk's tail; the line then reports the step time, and "
                         "the roofline's per-launch time is not a kernel duration")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0: enough to exceed the cache)")
    ap.add_argument("--cpu-seconds", type=float, default=60.0,
                    help="budget of the CPU oracle legs (0: skip): each leg repeats the step 5 times, or "
                         "3 times once its share of the budget is spent")
    ap.add_argument("--variant", default=None,
                    help="comma-separated kernel variant overrides (qkr_set_variant_override)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured HIP graph")
    return ap.parse_args()


def shard_ranges(total, n):
    """n contiguous [a, b) parts of range(total), sizes differing by at most one."""
    n = max(1, min(n, total))
    cuts = [total * i // n for i in range(n + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(n)]


class Workload:
    """name, config, bytes per step, dominant-kernel bytes per launch,
    launches of it per step, make_set() -> state, step(state) launches the
    path; cpu_parts(n) -> (n callables that together run the oracle on one
    step's input, share of the step they cover), each on its own rows."""


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
        qkr.joint_qk_norm_rope(g["text"], g["image"], case.eps, rope, out=outs, numerics=NUMERICS)

    qkv_bytes = joint * 3 * H * D * 2
    nbytes = 2 * qkv_bytes + case.positions.nbytes + 4 * D * 2 + case.inv_freq.nbytes

    def cpu_parts(n):
        import oracle

        orope = oracle.Rope("axes", D, pairing, inv_freq=case.inv_freq, sections=case.sections,
                            positions=case.positions)

        def stream(s, h0, h1):
            return {"q": W.as_f32(s.view(0, H, D)[:, :, h0:h1]), "k": W.as_f32(s.view(1, H, D)[:, :, h0:h1]),
                    "v": W.as_f32(s.view(2, H, D)[:, :, h0:h1]), "q_weight": W.as_f32(s.q_weight),
                    "k_weight": W.as_f32(s.k_weight)}

        def part(h0, h1):
            tx, im = stream(case.text, h0, h1), stream(case.image, h0, h1)
            return lambda: oracle.joint_qk_norm_rope(tx, im, case.eps, orope, "bf16", numerics=NUMERICS)
        return [part(a, b) for a, b in shard_ranges(H, n)], 1.0

    w = Workload()
    w.name = f"joint text/image QK RMSNorm + cat + 3-axis RoPE ({pairing})"
    w.config = {"workload": w.name, "text_tokens": st, "image_tokens": si, "heads": H, "head_dim": D,
                "axes_pairs": list(case.sections[:3]), "theta": 1e4, "eps": case.eps, "batch": 1}
    w.step_bytes = nbytes
    w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = "the full joint step (512 text + 4096 image tokens, Q/K/V), split over heads"
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

    side = []

    def step(state):
        q, k, qo, ko = state
        if STREAMS <= 1:
            for r in ropes:
                b = r.token_base
                qkr.qk_norm_rope(q[b:b + chunk], k[b:b + chunk], qw, kw, case.eps, r, q_out=qo[b:b + chunk],
                                 k_out=ko[b:b + chunk], numerics=NUMERICS)
            return
        # The chunks are independent: fork side streams from the current one,
        # launch chunk i on stream i mod STREAMS, join them back.
        main = torch.cuda.current_stream()
        while len(side) < STREAMS - 1:
            side.append(torch.cuda.Stream())
        streams = [main] + side[:STREAMS - 1]
        for st in streams[1:]:
            st.wait_stream(main)
        for i, r in enumerate(ropes):
            b = r.token_base
            with torch.cuda.stream(streams[i % STREAMS]):
                qkr.qk_norm_rope(q[b:b + chunk], k[b:b + chunk], qw, kw, case.eps, r, q_out=qo[b:b + chunk],
                                 k_out=ko[b:b + chunk], numerics=NUMERICS)
        for st in streams[1:]:
            main.wait_stream(st)

    rows = case.q.shape[1] + case.k.shape[1]
    chunk_bytes = 2 * chunk * rows * 128 * 2 + 4 * chunk * 4 + 2 * 128 * 2 + case.inv_freq.nbytes

    def cpu_parts(n):
        import oracle
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)

        def part(t0, t1):
            orope = oracle.Rope("imrope", 128, "neox", inv_freq=case.inv_freq, sections=case.sections,
                                positions=case.positions, token_base=t0)
            q, k = qf[t0:t1], kf[t0:t1]

            def run():
                oracle.qk_norm_rope(q, wq, case.eps, orope, numerics=NUMERICS)
                oracle.qk_norm_rope(k, wk, case.eps, orope, numerics=NUMERICS)
            return run
        return [part(a, b) for a, b in shard_ranges(T, n)], 1.0

    w = Workload()
    w.name = "IMROPE after per-head QK RMSNorm, 2048-token chunks"
    w.config = {"workload": w.name, "tokens": T, "chunk": chunk, "q_heads": case.q.shape[1],
                "k_heads": case.k.shape[1], "head_dim": 128, "sections": list(case.sections), "theta": 1e6}
    w.step_bytes = chunk_bytes * (T // chunk)
    w.launch_bytes = chunk_bytes
    w.launches = T // chunk
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = "all 8192 tokens, Q and K, split over tokens"
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
        qkr.qk_norm_rope(q, k, qw, kw, case.eps, rope, q_out=qo, k_out=ko, numerics=NUMERICS)

    heads = case.q.shape[1]
    planes = 2 * n * half * 4
    apply_bytes = 4 * n * heads * 2 * half * 2 + planes + 2 * 2 * half * 2

    def cpu_parts(nparts):
        import threading

        import oracle
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)
        planes = {}

        def part(i, t0, t1):
            q, k = qf[t0:t1], kf[t0:t1]

            def run():
                # the planes are the setup's output: part 0 computes them for
                # the whole step, the other parts apply them once they exist
                if i == 0:
                    planes["cs"] = oracle.vit_cos_sin(case.inv_t, case.inv_h, case.inv_w, case.grid_thw,
                                                      case.merge)
                    planes["ready"].set()
                else:
                    planes["ready"].wait()
                c, s = planes["cs"]
                orope = oracle.Rope("planes", 2 * half, "neox", sections=secs, cos_planes=c, sin_planes=s,
                                    token_base=t0)
                oracle.qk_norm_rope(q, wq, case.eps, orope, numerics=NUMERICS)
                oracle.qk_norm_rope(k, wk, case.eps, orope, numerics=NUMERICS)
            return run

        def reset():
            planes["ready"] = threading.Event()
        reset()
        w.cpu_reset = reset
        return [part(i, a, b) for i, (a, b) in enumerate(shard_ranges(n, nparts))], 1.0

    w = Workload()
    w.name = "ViT mrope cos/sin setup + apply after per-head QK RMSNorm"
    w.config = {"workload": w.name, "grid_thw": case.grid_thw, "spatial_merge": case.merge, "tokens": n,
                "heads": heads, "head_dim": 2 * half, "halves": list(secs[:3])}
    w.step_bytes = planes + apply_bytes
    w.launch_bytes = apply_bytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = "setup + apply over all 7952 tokens, the apply split over tokens"
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
        qkr.vit_qk_norm_rope(q, k, qw, kw, case.eps, *inv, case.grid_thw, case.merge, q_out=qo, k_out=ko,
                             numerics=NUMERICS)

    heads = case.q.shape[1]
    nbytes = 4 * n * heads * 2 * half * 2 + 2 * 2 * half * 2 + 4 * half

    def cpu_parts(nparts):
        import oracle
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)

        def part(h0, h1):
            q, k = np.ascontiguousarray(qf[:, h0:h1]), np.ascontiguousarray(kf[:, h0:h1])

            def run():
                oracle.vit_qk_norm_rope(q, wq, case.eps, case.inv_t, case.inv_h, case.inv_w, case.grid_thw,
                                        case.merge, numerics=NUMERICS)
                oracle.vit_qk_norm_rope(k, wk, case.eps, case.inv_t, case.inv_h, case.inv_w, case.grid_thw,
                                        case.merge, numerics=NUMERICS)
            return run
        return [part(a, b) for a, b in shard_ranges(heads, nparts)], 1.0

    w = Workload()
    w.name = "ViT QK RMSNorm + mrope with positions from the grids (setup folded in)"
    w.config = {"workload": w.name, "grid_thw": case.grid_thw, "spatial_merge": case.merge, "tokens": n,
                "heads": heads, "head_dim": 2 * half, "halves": [case.inv_t.size, case.inv_h.size, case.inv_w.size]}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = "all 7952 tokens, Q and K, split over heads"
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
        qkr.rms_norm(x, wgt, case.eps, out=y, numerics=NUMERICS)

    width = case.x.shape[1]
    nbytes = 2 * t * width * 2 + width * 2

    def cpu_parts(n):
        import oracle
        xf, wf = W.as_f32(case.x), W.as_f32(case.weight)

        def part(r0, r1):
            x = xf[r0:r1]
            return lambda: oracle.rms_norm(x, wf, case.eps, "bf16", numerics=NUMERICS)
        return [part(a, b) for a, b in shard_ranges(t, n)], 1.0

    w = Workload()
    w.name = f"plain row RMSNorm bf16 [{t}, {width}]"
    w.config = {"workload": w.name, "rows": t, "width": width, "eps": case.eps}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = f"the full [{t}, {width}] input, split over rows"
    return w


def build_cache():
    """IMROPE QK norm + RoPE of 8192 tokens (16 Q, 8 K/V heads x 128, bf16) with
    K and V written into a paged cache (2048 blocks x 16 slots), one launch.
    Slot map (--slots): random, an injective map of single slots (each
    token's 2 KB K and V rows land alone: the worst case for the writes), or
    blocks, the way a paged cache fills: 16 consecutive tokens take the 16
    slots of one block, the blocks drawn in random order."""
    import torch

    import transformer_qk_rmsnorm_amd as qkr
    import workloads as W

    case = W.imrope()
    dev = torch.device("cuda")
    T, H, KV, D = case.q.shape[0], case.q.shape[1], case.k.shape[1], 128
    blocks, bs = 2048, 16
    v_host = W.to_dtype(W.normal((T, KV, D), 0.0, 1.0, 61), "bf16")
    if SLOTS == "blocks":
        order = np.random.default_rng(61).permutation(blocks)[:T // bs].astype(np.int64)
        t_idx = np.arange(T, dtype=np.int64)
        slots_host = torch.from_numpy(order[t_idx // bs] * bs + t_idx % bs)
    else:
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
        qkr.qk_norm_rope_cache(q, k, v, qw, kw, kc, vc, slots, case.eps, rope, q_out=qo, numerics=NUMERICS)

    nbytes = 2 * T * (H + 2 * KV) * D * 2 + T * 8 + case.positions.nbytes + 2 * D * 2 + case.inv_freq.nbytes

    def cpu_parts(n):
        import oracle
        q, k, v = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(v_host)
        wq, wk = W.as_f32(case.q_weight), W.as_f32(case.k_weight)
        sl = slots_host.numpy()
        orope = oracle.Rope("imrope", D, "neox", inv_freq=case.inv_freq, positions=case.positions,
                            sections=case.sections)
        n = max(1, min(n, H))

        def part(qh, kh):
            # Q heads [qh) and K/V heads [kh) of every token; the part's cache
            # holds its own K/V heads of every slot
            qs = np.ascontiguousarray(q[:, qh[0]:qh[1]])
            ks, vs = np.ascontiguousarray(k[:, kh[0]:kh[1]]), np.ascontiguousarray(v[:, kh[0]:kh[1]])
            cache = np.zeros((blocks * bs, kh[1] - kh[0], D), np.float32)
            return lambda: oracle.qk_norm_rope_cache(qs, ks, vs, wq, wk, case.eps, orope, sl, cache, cache,
                                                     numerics=NUMERICS)
        qparts = [(H * i // n, H * (i + 1) // n) for i in range(n)]
        kparts = [(KV * i // n, KV * (i + 1) // n) for i in range(n)]
        return [part(a, b) for a, b in zip(qparts, kparts)], 1.0

    w = Workload()
    w.name = "IMROPE QK RMSNorm + RoPE with K/V written into a paged cache by slot mapping"
    w.config = {"workload": w.name, "tokens": T, "q_heads": H, "kv_heads": KV, "head_dim": D,
                "sections": list(case.sections), "cache_blocks": blocks, "block_size": bs, "slot_map": SLOTS}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = "all 8192 tokens, split over heads"
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
                         scale=scale, out=y, numerics=NUMERICS)

    width = case.x.shape[1]
    nbytes = t * width * (2 + 2 + 2 + (1 if fp8 else 2)) + width * 2 + (4 if fp8 else 0)

    def cpu_parts(n):
        import oracle
        xf, rf, wf = W.as_f32(case.x), W.as_f32(res), W.as_f32(case.weight)

        def part(r0, r1):
            x, r = xf[r0:r1], rf[r0:r1]
            return lambda: oracle.add_rms_norm(x, wf, case.eps, r, "bf16", "fp8_e4m3" if fp8 else "bf16", 0.02,
                                               numerics=NUMERICS)
        return [part(a, b) for a, b in shard_ranges(t, n)], 1.0

    w = Workload()
    w.name = f"residual add + RMSNorm bf16 [{t}, {width}] -> {'FP8 E4M3 (static scale)' if fp8 else 'bf16'}"
    w.config = {"workload": w.name, "rows": t, "width": width, "eps": case.eps, "out": "fp8_e4m3" if fp8 else "bf16"}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "bf16"
    w.sample = f"the full [{t}, {width}] input, split over rows"
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
        qkr.qk_norm_rope(q, k, ws[0], ws[1], case.eps, rope, q_out=qo, k_out=ko, numerics=NUMERICS)

    nbytes = 2 * 2 * case.q.numel() * 4 + 2 * 64 * 4 + 4 * 4 + 32 * 4

    def cpu_parts(n):
        import oracle
        orope = oracle.Rope("1d", 64, "neox", inv_freq=case.inv_freq, positions=case.positions)
        qf, kf, wq, wk = W.as_f32(case.q), W.as_f32(case.k), W.as_f32(case.q_weight), W.as_f32(case.k_weight)

        def run():
            oracle.qk_norm_rope(qf, wq, case.eps, orope, "f32", numerics=NUMERICS)
            oracle.qk_norm_rope(kf, wk, case.eps, orope, "f32", numerics=NUMERICS)
        return [run], 1.0

    w = Workload()
    w.name = "tiny fp32 QK RMSNorm + NeoX RoPE [4, 2, 64]"
    w.config = {"workload": w.name, "tokens": 4, "heads": 2, "head_dim": 64}
    w.step_bytes = w.launch_bytes = nbytes
    w.launches = 1
    w.make_set, w.step, w.cpu_parts = make_set, step, cpu_parts
    w.dtype = "f32"
    w.sample = "the full [4, 2, 64] input (too small to split)"
    return w


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
    w.cpu_parts = None
    w.dtype = "f32"
    w.sample = "none"
    return w


KERNEL_SOURCES = ["transformer_qk_rmsnorm_amd/csrc/" + f for f in
                  ("qkr_kernels.hip", "qkr_rope_part.hip", "qkr_token_part.hip", "qkr_rope_kernel.hpp",
                   "qkr_device.hpp", "qkr_internal.hpp", "qkr_fastdiv.hpp")]


def code_hash(texts):
    """Hash of C++ sources with comments removed and whitespace runs collapsed:
    the counters depend on the code, so a comment or layout edit keeps them
    valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for text in texts:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = re.sub(r"\s+", " ", text).strip()
        h.update(text.encode("utf-8") + b"\0")
    return h.hexdigest()


def kernel_source_hash():
    texts = []
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            texts.append(f.read())
    return code_hash(texts)


def measured_traffic(workload, variant):
    """HBM bytes per launch from the committed counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by
    what the counter reads for a plain copy of known size), or None when no
    summary exists, the kernels changed since the counters were taken, or
    the call now runs another kernel variant."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("kernel_source_sha256") != kernel_source_hash() or kv.get("variant") != variant:
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["write_scale"])
        return round(fetch + write)
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads():
    """Threads the all-cores leg uses: the cores this process may run on,
    at most the host share of one GPU (OMP_NUM_THREADS where it is set)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, CPU_MAX_THREADS))


def _time_leg(w, nthreads, budget):
    """Median, minimum and maximum seconds per step over CPU_REPS repetitions
    of one step split into nthreads parts run on as many threads."""
    import concurrent.futures
    parts, share = w.cpu_parts(nthreads)
    reset = getattr(w, "cpu_reset", None)

    def one():
        if reset is not None:
            reset()
        t0 = time.perf_counter()
        if len(parts) == 1:
            parts[0]()
        else:
            with concurrent.futures.ThreadPoolExecutor(max_workers=len(parts)) as ex:
                for f in [ex.submit(p) for p in parts]:
                    f.result()
        return time.perf_counter() - t0

    one()                                   # warm: page in, first touch
    times = []
    t_start = time.perf_counter()
    for _ in range(CPU_REPS):
        times.append(one())
        if time.perf_counter() - t_start > budget and len(times) >= 3:
            break
    times.sort()
    return {"threads": len(parts), "reps": len(times), "s_median": times[len(times) // 2] / share,
            "s_min": times[0] / share, "s_max": times[-1] / share}


def cpu_baseline(w, seconds):
    """The oracle on the host cores: an all-cores leg and a one-thread leg."""
    nthreads = host_threads()
    legs = {}
    for name, n, budget in (("all_cores", nthreads, seconds * 0.3), ("one_thread", 1, seconds * 0.7)):
        leg = _time_leg(w, n, budget)
        legs[name] = {"threads": leg["threads"], "reps": leg["reps"],
                      "us_per_step_median": round(leg["s_median"] * 1e6, 1),
                      "us_per_step_min": round(leg["s_min"] * 1e6, 1),
                      "us_per_step_max": round(leg["s_max"] * 1e6, 1),
                      "GB/s": round(w.step_bytes / leg["s_median"] / 1e9, 4)}
    main_leg = legs["all_cores"]
    return {"value": main_leg["GB/s"], "unit": "GB/s", "cores": main_leg["threads"], "kind": "oracle",
            "sample": f"median of {main_leg['reps']} repetitions of {w.sample} (plain C oracle, double "
                      f"precision, one part per thread), numerics {NUMERICS}",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "legs": legs}


def main():
    global NUMERICS, STREAMS, SLOTS
    args = _parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: every row of the path is per-row "
                                   "independent and shards without communication; run with --gpus 1"}))
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one process, one GPU; WORLD_SIZE > 1 is not supported", file=sys.stderr)
        sys.exit(2)
    NUMERICS = args.numerics
    STREAMS = max(1, args.streams)
    SLOTS = args.slots

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

    K = args.steps
    if args.eager:
        plan = [1] * K
    else:
        # Exactly K steps cycling over the buffer sets, captured in graphs of
        # at most 1024 kernel launches and at most K / GPU_SAMPLES steps, so
        # the timed region holds at least GPU_SAMPLES replays; replaying a
        # graph runs its launches back to back with no host work in between.
        # Each replay boundary costs several microseconds of idle GPU, so the
        # graphs stay long; a single graph of 4096 launches measured slower
        # per launch (IMROPE chunk 6.39 us against 5.93-5.97 us with 200 to
        # 2000 launches split over graphs of up to 1024).
        chunk = max(1, min(-(-K // GPU_SAMPLES), 1024 // w.launches))
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
        # The plan once untimed: the clocks settle under the same load.
        for n in plan:
            graphs[n].replay()
        torch.cuda.synchronize()
    # Sample boundaries at replay (or eager step) boundaries: GPU_SAMPLES
    # groups of consecutive replays, as even as the plan allows.
    nsamp = min(GPU_SAMPLES, len(plan))
    cuts = [len(plan) * i // nsamp for i in range(nsamp + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nsamp + 1)]
    torch.cuda.synchronize()
    events[0].record(stream)
    step_i = 0
    for s in range(nsamp):
        for j in range(cuts[s], cuts[s + 1]):
            if args.eager:
                w.step(sets[step_i % nsets])
                step_i += 1
            else:
                graphs[plan[j]].replay()
        events[s + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = events[0].elapsed_time(events[-1])
    sample_us = sorted(events[s].elapsed_time(events[s + 1]) * 1e3 / sum(plan[cuts[s]:cuts[s + 1]])
                       for s in range(nsamp))
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
                       numerics=NUMERICS, launch="eager" if args.eager else "hipGraph replay",
                       **({"streams": STREAMS} if STREAMS > 1 else {})),
        "gpu_samples": {"n": nsamp, "us_per_step_median": round(sample_us[len(sample_us) // 2], 3),
                        "us_per_step_min": round(sample_us[0], 3), "us_per_step_max": round(sample_us[-1], 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (measured_traffic(args.workload + ("-blocks" if SLOTS == "blocks" and args.workload == "cache"
                                                                    else ""), variant)
                                 if NUMERICS == "contract" else None),
                     "bytes_per_launch": w.launch_bytes, "kernel": variant},
    }
    if args.cpu_seconds > 0 and w.cpu_parts is not None:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
