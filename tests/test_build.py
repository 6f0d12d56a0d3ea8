"""The build's resource guard: a kernel that spills registers or keeps an
array in scratch memory fails the build (host-only)."""
from dense_gemm_preshuffle_amd import build as B

SAMPLE = """\
./k.hpp:171:1: remark: Function Name: _Z4fastv [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark: Function Name: _Z5arrayv [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     VGPRs: 70 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     ScratchSize [bytes/lane]: 1552 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark: Function Name: _Z5spillv [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     VGPRs Spill: 20 [-Rpass-analysis=kernel-resource-usage]
./k.hpp:171:1: remark:     ScratchSize [bytes/lane]: 68 [-Rpass-analysis=kernel-resource-usage]
"""


def test_resource_remarks_parsed():
    res = B.kernel_resources(SAMPLE)
    assert set(res) == {"_Z4fastv", "_Z5arrayv", "_Z5spillv"}
    assert res["_Z4fastv"]["VGPRs"] == "128"


def test_scratch_and_spills_flagged():
    bad = dict(B.spilling(B.kernel_resources(SAMPLE)))
    assert set(bad) == {"_Z5arrayv", "_Z5spillv"}
    assert bad["_Z5arrayv"] == [0, 0, 1552] and bad["_Z5spillv"] == [20, 0, 68]
