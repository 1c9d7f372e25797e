"""Host-side checks of the library build script (no compiler run)."""
from fine_grained_block_amd import build


def test_scratch_users_parses_resource_remarks():
    remarks = "\n".join([
        "gemm.hip:1:1: remark: Function Name: _ZN3fgb4k_aEv [-Rpass-analysis=kernel-resource-usage]",
        "gemm.hip:1:1: remark:     VGPRs: 216 [-Rpass-analysis=kernel-resource-usage]",
        "gemm.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "gemm.hip:1:1: remark: Function Name: _ZN3fgb4k_bEv [-Rpass-analysis=kernel-resource-usage]",
        "gemm.hip:1:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]",
        "gemm.hip:1:1: remark:     ScratchSize [bytes/lane]: 28 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build._scratch_users(remarks) == [("_ZN3fgb4k_bEv", 28)]
    assert build._scratch_users("") == []
