"""The kernels' division by invariant integers (csrc/qkr_fastdiv.hpp) equals
integer division: exhaustive small cases plus edge and random 32-bit values,
compiled for the host with g++ (CPU only)."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_qk_rmsnorm_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <random>
#include "qkr_fastdiv.hpp"
int main() {
    std::mt19937_64 rng(12345);
    long checked = 0;
    auto check = [&](uint32_t n, uint32_t d, const qkr::FastDiv& f) {
        ++checked;
        if (qkr::fast_div(n, f) != n / d) { std::printf("FAIL n=%u d=%u got=%u\n", n, d, qkr::fast_div(n, f)); return false; }
        return true;
    };
    for (uint32_t d = 1; d <= 4096; ++d) {
        qkr::FastDiv f = qkr::make_fastdiv(d);
        for (uint32_t n = 0; n < 20000; ++n) if (!check(n, d, f)) return 1;
        const uint32_t edges[] = {0xFFFFFFFFu, 0xFFFFFFFEu, 0x80000000u, 0x7FFFFFFFu, d * 1000u - 1, d * 1000u};
        for (uint32_t n : edges) if (!check(n, d, f)) return 1;
        for (int k = 0; k < 2000; ++k) if (!check((uint32_t)rng(), d, f)) return 1;
    }
    for (int k = 0; k < 20000; ++k) {
        uint32_t d = (uint32_t)(rng() % 0x7FFFFFFFu) + 1;
        qkr::FastDiv f = qkr::make_fastdiv(d);
        for (int i = 0; i < 200; ++i) if (!check((uint32_t)rng(), d, f)) return 1;
        if (!check(0xFFFFFFFFu, d, f) || !check(d, d, f) || !check(d - 1, d, f)) return 1;
    }
    std::printf("ok %ld\n", checked);
    return 0;
}
"""


def test_fast_div_matches_integer_division():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "t.cpp")
        exe = os.path.join(tmp, "t")
        open(src, "w").write(PROGRAM)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
