"""The HIP kernels as compiled for gfx950 (device code only, on the CPU): no
kernel spills vector registers or uses scratch memory, and none asks for more
LDS than a CU has (160 KiB).  (A scalar register the compiler spills goes to a
vector register's lane, not to memory; the scratch size check covers both.)"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_bottleneck_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


@pytest.mark.parametrize("src", ["lr_kernels.hip", "lr_fused.hip", "lr_api.cpp"])
def test_no_spills_no_scratch(src, tmp_path):
    from rank_bottleneck_amd import build
    out = tmp_path / (src + ".s")
    cmd = [HIPCC] + build.flags() + ["--cuda-device-only", "-S", "-o", str(out)]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    subprocess.run(cmd + [os.path.join(CSRC, src)], check=True, capture_output=True)
    text = out.read_text()
    kernels = text.split("  - .agpr_count:")[1:]
    if src != "lr_api.cpp":
        assert kernels, "no kernel metadata found"
    for k in kernels:
        name = re.search(r"\.name:\s+(\S+)", k).group(1)
        spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", k).group(1))
        priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", k).group(1))
        lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", k).group(1))
        assert spill == 0, (name, spill)
        assert priv == 0, (name, priv)
        assert lds <= 160 * 1024, (name, lds)
