"""Code-generation checks of the blockwise kernels (no GPU needed; hipcc cross-compiles gfx950).

* The partial of a K block is the unscaled fp8 MFMA: the kernels call the scaled builtin with
  both scale operands 0, which the compiler emits as v_mfma_f32_16x16x128_f8f6f4 (one instruction
  word instead of two, and no scale applied). The check fails if a compiler emits the scaled form.
* No VGPRs spill to scratch in the whole-item kernels (a spill reload's vmcnt wait would also wait
  for the copies in flight).
"""

import os
import re
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _asm(tmp_path_factory, src):
    from mx_grouped_gemm_amd.build import FLAGS, VGPR_FORM

    out = tmp_path_factory.mktemp("isa") / (src + ".s")
    flags = [f for f in FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, *VGPR_FORM, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return {s: _asm(tmp_path_factory, s) for s in ("bs_fp8_grouped.hip", "bs_fp8_small_m.hip")}


def test_unscaled_fp8_mfma(asm):
    for src, text in asm.items():
        assert "v_mfma_f32_16x16x128_f8f6f4" in text, src
        assert "v_mfma_scale" not in text, src


def test_whole_item_kernels_do_not_spill(asm):
    text = asm["bs_fp8_grouped.hip"]
    names = re.findall(r"\.name:\s+(\S+)", text)
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)
    assert len(names) == len(spills)
    forms = 0
    for n, v in zip(names, spills):
        # bw_fp8_grouped_kernel<OUT, false, false>: every launch of whole items of at least four
        # rounds. The form with the last round's ranges (<OUT, false, true>, shorter launches) may
        # keep a few values in scratch across a unit's start.
        if "Lb0ELb0E" in n:
            forms += 1
            assert int(v) == 0, n
        elif "Lb0ELb1E" in n:
            assert int(v) <= 4, n
    assert forms == 3
