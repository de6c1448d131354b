"""The build refuses kernels whose waits count vector-memory operations in
flight when they spill registers to scratch (scratch traffic counts in the
same counter). CPU only: the guard parses the compiler's resource remarks."""
from io_aware_flashattention_amd import build as B

REMARKS = """\
x.hip:1:1: remark: Function Name: _ZN2fa6detail13fwd_pp_kernelILi128ELb1EDF16bLi3EEEvNS_9FwdParamsE [-Rpass]
x.hip:1:1: remark:     VGPRs: 256 [-Rpass]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: {pp} [-Rpass]
x.hip:1:1: remark: Function Name: _ZN2fa6detail15fwd_bf16_kernelILi64ELb1EDF16bLi4ELi1ELi3EEEvNS_9FwdParamsE [-Rpass]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass]
x.hip:1:1: remark: Function Name: _ZN2fa6detail19decode_split_kernelILi128EDF16bLb0EEEvNS_12DecodeParamsE [-Rpass]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: {dec} [-Rpass]
"""


def test_guard_names_counted_wait_kernels_that_spill():
    assert B.scratch_users(REMARKS.format(pp=0, dec=0)) == []       # the d=64 kernel's waits are all vmcnt(0)
    assert B.scratch_users(REMARKS.format(pp=16, dec=0)) == [
        "_ZN2fa6detail13fwd_pp_kernelILi128ELb1EDF16bLi3EEEvNS_9FwdParamsE"]
    assert len(B.scratch_users(REMARKS.format(pp=4, dec=4))) == 2
