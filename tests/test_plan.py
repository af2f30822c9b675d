"""The variant planners (csrc/qkr_plan.cpp, pure host code) compiled for the
host with a small driver (CPU only): the kernel variant each timed workload
shape gets, including the seven-wave cap of the tile kernel, and forced
choices that cannot run refused with a reason rather than replaced."""
import json
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_qk_rmsnorm_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cstdlib>
#include "qkr_internal.hpp"
using namespace qkr;
// argv: rope dtype head_dim hq hk hv half planes token_ok np lpr stage token nt
//    or rms nvec rows kind nt mode
int main(int argc, char** argv) {
    auto I = [&](int i) { return atoi(argv[i]); };
    if (argv[1][0] == 'r' && argv[1][1] == 'o') {
        const int32_t heads[3] = {I(4), I(5), I(6)};
        RopePlan p{};
        const char* why = plan_norm_rope(I(2), I(3), heads, I(7), I(8) != 0, I(9) != 0, I(10), I(11), I(12),
                                         I(13), I(14), &p);
        if (why) { printf("{\"refused\": \"%s\"}\n", why); return 0; }
        printf("{\"lpr\": %d, \"np\": %d, \"stage\": %d, \"nt\": %d, \"token\": %d, \"waves_cap\": %d}\n",
               p.lpr, p.np, (int)p.stage, (int)p.nt, p.token, p.waves_cap);
    } else {
        RmsPlan p{};
        const char* why = plan_rms_norm(I(2), atoll(argv[3]), I(4), I(5), I(6), &p);
        if (why) { printf("{\"refused\": \"%s\"}\n", why); return 0; }
        printf("{\"kind\": %d, \"vpl\": %d, \"nt\": %d, \"mode\": %d}\n", p.kind, p.vpl, (int)p.nt, p.mode);
    }
    return 0;
}
"""

F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def planner():
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "driver.cpp")
        exe = os.path.join(tmp, "driver")
        with open(src, "w") as f:
            f.write(DRIVER)
        # Host code only: hipcc for the HIP headers the internal interface
        # includes, no device code in either file.
        subprocess.run(["hipcc", "-O1", "-std=c++17", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                        src, os.path.join(CSRC, "qkr_plan.cpp"), "-o", exe],
                       check=True, capture_output=True, text=True)

        def run(*args):
            r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=60)
            assert r.returncode == 0, r.stderr
            return json.loads(r.stdout)
        yield run


def rope(run, dtype, head_dim, heads, half, planes=False, token_ok=True, np=0, lpr=0, stage=-1, token=-1, nt=1):
    return run("rope", dtype, head_dim, *heads, half, int(planes), int(token_ok), np, lpr, stage, token, nt)


def test_joint_shape_two_passes_capped_at_seven_waves(planner):
    # 24 heads x 128 per tensor, V copied: two passes of 8 rows, 4 KB per wave.
    p = rope(planner, BF16, 128, (24, 24, 24), 64, token_ok=False)
    assert p == {"lpr": 8, "np": 2, "stage": 0, "nt": 1, "token": 0, "waves_cap": 7}


def test_imrope_shape(planner):
    p = rope(planner, BF16, 128, (16, 8, 0), 64)
    assert (p["lpr"], p["np"], p["stage"], p["token"], p["waves_cap"]) == (8, 2, 0, 0, 7)


def test_cache_write_shape_one_pass_uncapped(planner):
    # 16 Q + 8 K + 8 V heads: two passes would leave a third idle; 2 KB per wave.
    p = rope(planner, BF16, 128, (16, 8, 8), 64, token_ok=False)
    assert (p["np"], p["waves_cap"]) == (1, 0)


def test_vit_fused_shape_takes_token_tiles(planner):
    p = rope(planner, BF16, 80, (16, 16, 0), 40)
    assert (p["token"], p["lpr"], p["waves_cap"]) == (5, 5, 0)


def test_vit_planes_shape_stays_on_staged_tiles(planner):
    # 160-byte rows: 8 rows x 2 passes = 2.5 KB per wave, below the cap's 4 KB.
    p = rope(planner, BF16, 80, (16, 16, 0), 40, planes=True)
    assert p == {"lpr": 8, "np": 2, "stage": 1, "nt": 1, "token": 0, "waves_cap": 0}


def test_tiny_fp32_shape(planner):
    p = rope(planner, F32, 64, (2, 2, 0), 32)
    assert (p["lpr"], p["np"], p["token"], p["waves_cap"]) == (8, 1, 0, 0)


def test_norm_only_half_zero(planner):
    p = rope(planner, BF16, 128, (24, 24, 0), 0)
    assert (p["lpr"], p["np"], p["waves_cap"]) == (8, 2, 7)


@pytest.mark.parametrize("kwargs, reason", [
    (dict(lpr=4), "rope:lpr"),                    # each lane would hold four vectors of a 128-wide row
    (dict(np=5), "rope:np"),
    (dict(lpr=32, stage=1), "rope:stage1"),
    (dict(token=1, np=2), "rope:token"),
])
def test_forced_choices_that_cannot_run_are_refused(planner, kwargs, reason):
    p = rope(planner, BF16, 128, (16, 8, 0), 64, **kwargs)
    assert p.get("refused", "").startswith(reason), p


def test_forced_token_tiles_for_a_power_of_two_row_are_refused(planner):
    p = rope(planner, BF16, 128, (16, 8, 0), 64, token=1)
    assert "refused" in p and "token tiles serve" in p["refused"], p


@pytest.mark.parametrize("rows, kind", [(1, 2), (32, 2), (1024, 2), (2048, 0), (4096, 0), (4097, 2), (8192, 2)])
def test_row_norm_variant_by_row_count(planner, rows, kind):
    p = planner("rms", 640, rows, -1, 1, 0)   # rows of 5120 bf16: 640 vectors
    assert p["kind"] == kind, p
    assert p["vpl"] == (10 if kind == 0 else 3)


def test_row_norm_forced_split_with_residual_is_refused(planner):
    p = planner("rms", 640, 4, 1, 1, 1)
    assert p.get("refused", "").startswith("rms:split"), p


def test_row_norm_short_rows_keep_a_wave(planner):
    p = planner("rms", 8, 1, -1, 1, 0)         # rows of 64 bf16: fewer than 64 vectors
    assert (p["kind"], p["vpl"]) == (0, 1)
