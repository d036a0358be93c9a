"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

``oracle_sanitize_driver.c`` calls every oracle function on many small
random inputs, valid and invalid, with buffers of exactly the contracted
sizes.  Built with gcc ``-fsanitize=address,undefined`` and no recovery,
any out-of-bounds access, leak or undefined behaviour in the oracle aborts
the run.  The driver also counts the calls that passed validation, so the
test knows the full computations ran too, not only the error exits.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_oracle_clean_under_sanitizers(tmp_path, seed):
    exe = str(tmp_path / "oracle_sanitize_driver")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(HERE, "oracle_sanitize_driver.c"),
                    os.path.join(ROOT, "oracle", "psq_oracle.c"), "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    run = subprocess.run([exe, "20000", str(seed)], env=env, capture_output=True, text=True,
                         timeout=300)
    assert run.returncode == 0, run.stderr[-4000:]
    words = run.stdout.split()
    counts = dict(zip(words[2::2], map(int, words[3::2])))
    assert words[:2] == ["ok", "20000"]
    assert min(counts.values()) > 100, counts
