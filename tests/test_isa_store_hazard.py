"""The wide streaming stores keep their hazard padding (CPU; needs hipcc).

The library writes non-temporal agent-scope stores as inline assembly, which
the compiler's hazard recognizer does not look into.  On gfx940 and later a
store of more than 8 bytes needs two wait states before a VALU instruction
writes its data registers; one was not enough (a squeeze build with a
register move scheduled right after the token-mask store wrote wrong mask
bytes).  This test compiles the kernels that use the 16-byte form for gfx950
and checks that every such store in the generated code is followed by at
least two wait states (``s_nop 1`` or more) before the next instruction.
"""
import os
import re
import shutil
import subprocess

import pytest

from varlen_attention_metadata_amd import _build


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("source", ["k_copy.hip", "k_thd.hip"])
def test_wide_streaming_stores_carry_two_wait_states(tmp_path, source):
    """The collapse copy (alone, and fused into the table kernel) uses the
    inline 16-byte form."""
    out = str(tmp_path / (source + ".s"))
    cmd = [_build._hipcc(), *_build.HIP_FLAGS, "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, source), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lines = [l.strip() for l in open(out) if l.strip()]
    stores = [i for i, l in enumerate(lines)
              if re.match(r"global_store_dwordx[34]\b", l) and "sc1 nt" in l]
    assert stores, "no wide streaming store found"
    for i in stores:
        nxt = lines[i + 1]
        m = re.match(r"s_nop\s+(\d+)", nxt)
        assert m and int(m.group(1)) >= 1, f"{source}: '{lines[i]}' followed by '{nxt}'"


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_squeeze_uses_the_compiler_stores(tmp_path):
    """The squeeze's stores are the compiler's non-temporal stores (the inline
    form gained less than 1 % there), so its hazards are the compiler's."""
    out = str(tmp_path / "k_pack.hip.s")
    cmd = [_build._hipcc(), *_build.HIP_FLAGS, "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, "k_pack.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = open(out).read()
    assert not re.search(r"global_store_dword\S*.*sc1 nt", text)
    assert re.search(r"global_store_dwordx2 .* nt", text)
