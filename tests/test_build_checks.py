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


def test_index_selection_scoring_has_no_fused_multiply_add(tmp_path):
    """The index selection reproduces float32 products and sums rounded one by one; the scoring
    kernels, as built, must hold no fused or packed multiply-add.  (The only v_fmamk_f32 allowed
    is the compiler's 64-bit integer division, which multiplies by the constants +-2^32.)"""
    import os
    import re
    import subprocess

    src = os.path.join(_build.CSRC, "dsa_select.hip")
    asm = tmp_path / "dsa.s"
    cmd = [_build.hipcc(), *_build.HIPCC_FLAGS, "-ffp-contract=off", "--offload-device-only", "-S",
           src, "-o", str(asm)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = asm.read_text()
    kernels = re.split(r"\n(?=_ZN3dsa16dsa_score_kernel\w*:)", text)[1:]
    assert len(kernels) == 9   # 3 dtypes x 3 head-dim bounds
    for body in kernels:
        name = body.split(":", 1)[0]
        body = body.split(".Lfunc_end", 1)[0]
        for line in body.splitlines():
            op = line.strip().split(" ", 1)[0]
            if re.match(r"v_(pk_)?(fma|fmac|mac|mad)\w*_f32|v_pk_(mul|add)_f32|v_dot", op):
                if op == "v_fmamk_f32" and ("0x4f800000" in line or "0xcf800000" in line):
                    continue
                raise AssertionError(f"{name}: {line.strip()}")
        assert "v_mul_f32" in body and "v_add_f32" in body
