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
