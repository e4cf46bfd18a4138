"""The build refuses ring kernels that spill (their inline-asm loads must not be copied early)."""

import pytest

from tiled_online_softmax_flash_amd import _build

SPILLED = """\
x.h:85:1: remark: Function Name: _ZN2fa17fwd16_ring_kernelINS_10TraitsBF16ELi128EEEvNS_9FwdParamsE [-Rpass-analysis=kernel-resource-usage]
x.h:85:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.h:85:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]
x.h:85:1: remark:     SGPRs Spill: 40 [-Rpass-analysis=kernel-resource-usage]
x.h:85:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]
"""

CLEAN = SPILLED.replace("ScratchSize [bytes/lane]: 8", "ScratchSize [bytes/lane]: 0").replace(
    "VGPRs Spill: 2", "VGPRs Spill: 0")


def test_spilled_ring_kernel_is_refused():
    with pytest.raises(RuntimeError, match="must not"):
        _build._check_no_spills("fa_fwd_bf16_ring.hip", SPILLED)


def test_clean_ring_kernel_passes_and_sgpr_spills_are_allowed():
    _build._check_no_spills("fa_fwd_bf16_ring.hip", CLEAN)


def test_other_kernels_are_not_checked():
    _build._check_no_spills("fa_fwd_bf16.hip", SPILLED.replace("ring_kernel", "plain_kernel"))
