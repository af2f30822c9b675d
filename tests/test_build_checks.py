"""The build's resource checks read the compiler's kernel-resource remarks:
a kernel with private (scratch) memory, or with more LDS than the staging
slice, fails the build."""
from transformer_qk_rmsnorm_amd import build

REMARKS = """x.hip:1:1: remark: Function Name: _Z4goodv [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     LDS Size [bytes/block]: 8192 [-Rpass-analysis=kernel-resource-usage]
x.hip:2:1: remark: Function Name: _Z5spillv [-Rpass-analysis=kernel-resource-usage]
x.hip:2:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
x.hip:2:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:3:1: remark: Function Name: _Z8promotedv [-Rpass-analysis=kernel-resource-usage]
x.hip:3:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:3:1: remark:     LDS Size [bytes/block]: 16384 [-Rpass-analysis=kernel-resource-usage]
""".splitlines()


def test_scratch_users_are_found():
    assert build._scratch_users(REMARKS) == [("_Z5spillv", 16)]


def test_lds_beyond_the_staging_slice_is_found():
    assert build._lds_overruns(REMARKS) == [("_Z8promotedv", 16384)]


def test_counter_summaries_are_keyed_to_code_not_comments():
    """The HBM-traffic summaries carry a hash of the kernel sources; a
    comment or layout edit keeps it, a code edit changes it."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    code = "int f(int a)\n{\n    return a + 1;   // one\n}\n"
    same = "/* header */\nint f(int a) {\n  // the sum\n  return a + 1;\n}"
    other = "int f(int a)\n{\n    return a + 2;\n}\n"
    assert bench.code_hash([code]) == bench.code_hash([same])
    assert bench.code_hash([code]) != bench.code_hash([other])
    assert bench.code_hash([code, ""]) != bench.code_hash(["", code])
    # every committed summary names a hash of that form and the figures it needs
    prof = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    for name in os.listdir(prof):
        if name.startswith("traffic_"):
            kv = dict(l.split(":", 1) for l in open(os.path.join(prof, name)) if ":" in l and not l.startswith("#"))
            assert len(kv["kernel_source_sha256"].strip()) == 64, name
            for key in ("fetch_kib_per_dispatch", "write_kib_per_dispatch", "fetch_scale", "write_scale"):
                float(kv[key])
