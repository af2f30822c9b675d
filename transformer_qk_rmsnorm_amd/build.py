"""Build libqkrope.so (gfx950) in-tree with hipcc.

    python -m transformer_qk_rmsnorm_amd.build [-v]

Every translation unit is compiled as HIP for gfx950 only.  Packed fp32
VALU instructions are disabled (-packed-fp32-ops); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqkrope.so")
BUILD_DIR = os.path.join(PKG, "_build")

# (source, extra flags, object name): the QK RMSNorm + RoPE kernels are
# instantiated once per lanes-per-row value and numerics, in parallel
# compilations.
LANES_PER_ROW = (1, 2, 4, 8, 16, 32)
TOKEN_LANES = (3, 5, 6, 7)   # lanes per row of the token-tile kernels
UNITS = ([("qkr_kernels.hip", [], "qkr_kernels"), ("qkr_api.cpp", [], "qkr_api"), ("qkr_plan.cpp", [], "qkr_plan")] +
         [("qkr_rope_part.hip", [f"-DQKR_LPR={n}", f"-DQKR_EAGER={e}"], f"qkr_rope_lpr{n}_eager{e}")
          for n in LANES_PER_ROW for e in (0, 1)] +
         [("qkr_token_part.hip", [f"-DQKR_TOKEN_L={n}", f"-DQKR_EAGER={e}"], f"qkr_token_l{n}_eager{e}")
          for n in TOKEN_LANES for e in (0, 1)])
# Kernels must not use private (scratch) memory: a stray dynamic index into a
# by-value kernel argument or a local array silently costs a per-lane copy in
# scratch.  The compiler's resource remarks are checked on every build.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
ARCH = "gfx950"

FLAGS = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _scratch_users(lines):
    """Kernels whose resource remark reports a non-zero scratch size."""
    users, name = [], None
    for ln in lines:
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in ln:
            size = int(ln.split("ScratchSize [bytes/lane]:")[1].split()[0])
            if size and name:
                users.append((name, size))
    return users


# The largest LDS a kernel is meant to use per workgroup: the QK tile
# kernel's staging slice (4 waves x 128 vectors x 16 bytes), and the token-tile
# kernel's slice (4 waves x 320 row vectors x 16 bytes where the rows arrive
# by LDS DMA, so that eight workgroups fit the 160 KB of a compute unit; 4 x
# (320 + 32 weight vectors) x 16 bytes where they go through registers).
# More means the compiler has moved a private array into LDS (indexed by the
# work-item id, which also costs a read of the dispatch packet in every
# wave).
LDS_LIMIT = 8192
LDS_LIMIT_TOKEN = 22528


def _lds_overruns(lines):
    """Kernels whose resource remark reports more LDS than their limit."""
    over, name = [], None
    for ln in lines:
        if "Function Name:" in ln:
            name = ln.split("Function Name:")[1].split()[0]
        elif "LDS Size [bytes/block]:" in ln:
            size = int(ln.split("LDS Size [bytes/block]:")[1].split()[0])
            limit = LDS_LIMIT_TOKEN if name and "norm_rope_token_kernel" in name else LDS_LIMIT
            if size > limit and name:
                over.append((name, size))
    return over


def _compile(unit, verbose: bool) -> str:
    src, extra, name = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = ["hipcc", *FLAGS, *extra, *RESOURCE_REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = (r.stdout + r.stderr).splitlines()
    msgs = [ln for ln in lines if noise not in ln and "remark:" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name}:\n" + "\n".join(msgs))
    users = _scratch_users(lines)
    if users:
        raise RuntimeError(f"{name}: kernels using scratch memory: {users[:5]}")
    over = _lds_overruns(lines)
    if over:
        raise RuntimeError(f"{name}: kernels using more LDS than their slice: {over[:5]}")
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    workers = max(1, min(len(UNITS), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
