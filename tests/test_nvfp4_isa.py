"""Code-generation checks of the nvfp4 kernel (no GPU needed; hipcc cross-compiles gfx950).

The kernel writes its MFMA as an instruction of its own, so the compiler neither unrolls around
it by necessity nor inserts that instruction's wait states. Both properties depend on the
compiler's scheduling, so they are checked on the assembly of every output-type variant:

* the 64-step K loop is fully unrolled: 512 MFMAs per kernel;
* every MFMA reads its A/B sources at least 2 wait states after the last VALU write of them
  (s_nop n counts n + 1);
* no VALU instruction writes an AGPR between the first and the last MFMA (the accumulators
  stay in place).
"""

import os
import re
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SRC = os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc", "nv_fp4.hip")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    from mx_grouped_gemm_amd.build import FLAGS

    out = tmp_path_factory.mktemp("isa") / "nv_fp4.s"
    flags = [f for f in FLAGS if f not in ("-fPIC",)]
    cmd = [HIPCC, *flags, "-Werror=pass-failed", "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text().splitlines()
    found = {}
    name = None
    for line in text:
        m = re.match(r"^(_Z\S*nv_fp4_kernel\S*):", line)
        if m:
            name = m.group(1)
            found[name] = []
            continue
        if name:
            s = line.strip()
            if s.startswith("s_endpgm"):
                name = None
            elif s and not s.startswith((";", ".")) and not s.endswith(":"):
                found[name].append(s.replace(",", " ").split())
    assert len(found) == 3, sorted(found)
    return found


def test_k_loop_fully_unrolled(kernels):
    for name, ins in kernels.items():
        assert sum(1 for p in ins if p[0].startswith("v_mfma")) == 512, name


def test_mfma_sources_wait_after_valu_writes(kernels):
    for name, ins in kernels.items():
        for n, p in enumerate(ins):
            if not p[0].startswith("v_mfma"):
                continue
            srcs = _regs(p[2]) | _regs(p[3])
            ws = 0
            for q in reversed(ins[max(0, n - 16):n]):
                if q[0] == "s_nop":
                    ws += int(q[1], 0) + 1
                    continue
                if q[0].startswith("v_") and not q[0].startswith("v_mfma") and len(q) > 1:
                    if _regs(q[1]) & srcs:
                        assert ws >= 2, f"{name}: {' '.join(p)} reads a VALU result after {ws} wait states"
                        break
                ws += 1


def test_no_agpr_writes_inside_the_k_loop(kernels):
    for name, ins in kernels.items():
        idx = [n for n, p in enumerate(ins) if p[0].startswith("v_mfma")]
        for p in ins[idx[0]:idx[-1]]:
            assert not p[0].startswith(("v_accvgpr_write", "v_accvgpr_mov")), f"{name}: {' '.join(p)}"
