"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
only): tests/oracle_sanitize.c runs every oracle function on random shapes
with exactly sized heap buffers; any out-of-bounds access or undefined
arithmetic aborts the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
         os.path.join(HERE, "oracle_sanitize.c"), "-lm"],
        capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower():
        pytest.skip("gcc has no sanitizer runtime here")
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stderr[-2000:]
