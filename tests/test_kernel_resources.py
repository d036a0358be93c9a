"""No kernel spills to scratch memory (CPU; needs hipcc).

A kernel that indexes a register array with a runtime index, or runs out of
registers, gets per-lane private (scratch) memory.  On MI355X that cost the
document-map kernels about a microsecond per launch (their mask tail loop
once kept the loaded values in 92 bytes of scratch per lane).  This test
compiles every source of the library for gfx950 and checks, in the code
object metadata, that no kernel has a private segment or a dynamic stack.
"""
import os
import re
import shutil
import subprocess

import pytest

from varlen_attention_metadata_amd import _build

SOURCES = sorted(os.path.basename(p) for p in _build.sources())


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("source", SOURCES)
def test_no_kernel_uses_scratch(tmp_path, source):
    out = str(tmp_path / (source + ".s"))
    cmd = [_build._hipcc(), *_build.HIP_FLAGS, "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, source), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = open(out).read()
    kernels = re.findall(r"^\s+\.name:\s+(\S+)$", text, flags=re.M)
    private = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)
    dynamic = re.findall(r"\.uses_dynamic_stack:\s+(\w+)", text)
    assert len(private) == len(dynamic) >= 1 or not kernels
    for name, size, dyn in zip(kernels, private, dynamic):
        assert int(size) == 0, f"{source}: {name} uses {size} bytes of scratch per lane"
        assert dyn == "false", f"{source}: {name} uses a dynamic stack"
