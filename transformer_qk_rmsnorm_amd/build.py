"""Build libqkrope.so (gfx950) in-tree with hipcc.

    python -m transformer_qk_rmsnorm_amd.build [-v]

Both translation units are compiled as HIP for gfx950 only.  Packed fp32
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

SOURCES = ["qkr_kernels.hip", "qkr_api.cpp"]
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


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, *RESOURCE_REMARKS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    lines = (r.stdout + r.stderr).splitlines()
    msgs = [ln for ln in lines if noise not in ln and "remark:" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    users = _scratch_users(lines)
    if users:
        raise RuntimeError(f"{src}: kernels using scratch memory: {users[:5]}")
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
