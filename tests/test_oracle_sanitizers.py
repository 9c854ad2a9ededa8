"""The C oracle under sanitizers (CPU only): tests/oracle_sanitizer_driver.c compiles
oracle/ssm_oracle.c into a program that runs its forward (threaded and one-thread) and backward
on small random problems with exactly sized buffers.  Built once with AddressSanitizer and
UndefinedBehaviorSanitizer, once with ThreadSanitizer; either reports out-of-bounds accesses,
undefined operations or data races of the oracle's worker threads as a failure."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "oracle_sanitizer_driver.c")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the driver")


def _build_and_run(tmp_path, flags):
    exe = str(tmp_path / "driver")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math"] + flags +
                          ["-o", exe, DRIVER, "-lm", "-lpthread"])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-2000:] + res.stderr[-4000:]


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"])


def test_oracle_under_thread_sanitizer(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=thread"])
