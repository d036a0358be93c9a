"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Every source of the library is compiled host-only (no device code) with
``-fsanitize=address,undefined`` and no recovery, and linked against
``abi_sanitize_stubs.c``, which stands in for the HIP runtime: a launch
checks its shape against HIP's limits and returns success.  So the C ABI's
argument validation, workspace sizing, grid and copy planning and launch
set-up all run on the CPU, and signed overflow in the size arithmetic, an
out-of-bounds access or a leak aborts the run.  ``abi_sanitize_driver.c``
replays every case of ``test_abi_host.py`` and then a seeded fuzz of every
entry point (sizes around the int32 and int64 limits, strides and
overlapping copies, chunk counts around their edges, null and misaligned
pointers), checking each workspace query against its call.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from varlen_attention_metadata_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_driver(tmp):
    hipcc = _build._hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        cmd = [hipcc, "--cuda-host-only", "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC",
               "-I", _build.INCLUDE, "-I", _build.CSRC, "-c", src, "-o", obj]
        for flag in SAN:             # host code only: each sanitizer flag after -Xarch_host
            cmd[1:1] = ["-Xarch_host", flag]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        return obj

    with ThreadPoolExecutor(max_workers=4) as pool:
        objs = list(pool.map(compile_one, _build.sources()))
    # host-only objects refer to device-code blobs that are not built: give
    # each a dummy definition
    nm = subprocess.run(["nm", "-u", *objs], check=True, capture_output=True, text=True).stdout
    blobs = sorted(set(re.findall(r"\b(__hip_fatbin_\w+)", nm)))
    blob_c = os.path.join(tmp, "fatbin_blobs.c")
    with open(blob_c, "w") as f:
        f.writelines(f"const char {b}[64];\n" for b in blobs)
    exe = os.path.join(tmp, "abi_sanitize_driver")
    c_objs = []
    for src in (os.path.join(HERE, "abi_sanitize_stubs.c"), os.path.join(HERE, "abi_sanitize_driver.c"),
                blob_c):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        subprocess.run([CLANG, "-std=c99", "-O1", "-g", *SAN, "-I", _build.INCLUDE, "-c", src,
                        "-o", obj], check=True, capture_output=True, text=True)
        c_objs.append(obj)
    subprocess.run([CLANG + "++", *SAN, *objs, *c_objs, "-o", exe, "-lpthread"], check=True,
                   capture_output=True, text=True)
    return exe


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(CLANG) or (shutil.which("hipcc") is None and
                                     not os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("ROCm's clang and hipcc are needed")
    return _build_driver(str(tmp_path_factory.mktemp("abi_san")))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_abi_host_code_clean_under_sanitizers(driver, seed):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    run = subprocess.run([driver, "100000", str(seed)], env=env, capture_output=True, text=True,
                         timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, run.stderr[-4000:]
    words = run.stdout.split()
    assert words[:2] == ["ok", "100000"], run.stdout
    counts = dict(zip(words[2::2], map(int, words[3::2])))
    # the fuzz reached every outcome, launches included
    assert counts["checks"] >= 130 and counts["launched"] > 5000, counts
    assert min(counts["arg"], counts["overflow"], counts["workspace"]) > 100, counts
