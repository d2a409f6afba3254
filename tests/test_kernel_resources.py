"""Every kernel instantiation compiles for gfx950 without register spills
and without any other scratch memory (a spill, or a local array the compiler
cannot keep in registers, turns into memory traffic inside the hot loops),
and within the LDS of one workgroup.  Compiles each kernel source to
assembly with the library's own flags; no GPU needed."""

import os
import re
import subprocess
import tempfile

import pytest

from gqa_attention_sinks_amd import build

KERNEL_SOURCES = sorted(build.KERNEL_SOURCES)


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_spills_and_lds_fits(src):
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, src + ".s")
        cmd = [build.hipcc(), *build.FLAGS, *build.KERNEL_FLAGS, "--cuda-device-only", "-S",
               os.path.join(build.CSRC, src), "-o", out]
        p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert p.returncode == 0, p.stdout[-2000:]
        text = open(out).read()
    meta = text[text.index("amdhsa.kernels:"):]
    kernels = meta.split("  - .agpr_count")[1:]
    assert kernels, "no kernels found"
    for block in kernels:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        vspill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", block).group(1))
        sspill = int(re.search(r"\.sgpr_spill_count:\s+(\d+)", block).group(1))
        lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1))
        scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
        assert vspill == 0 and sspill == 0, f"{name}: {vspill} VGPR / {sspill} SGPR spills"
        assert scratch == 0, f"{name}: {scratch} bytes of scratch per lane"
        assert lds <= 160 * 1024, f"{name}: {lds} bytes of LDS"
