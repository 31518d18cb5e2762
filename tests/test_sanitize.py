"""The CPU oracle and the pins built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc), driven through every entry point on small
and edge-case inputs by tests/sanitize/driver.c: any out-of-bounds access,
leak, overflow or other undefined behaviour fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_and_pins_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitized")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "driver.c"), os.path.join(ROOT, "oracle", "r9k_oracle.c"),
            os.path.join(ROOT, "tests", "pins", "pins.c")]
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-pthread",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-o", exe, *srcs, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "ok" in r.stdout
