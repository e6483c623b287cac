"""The CPU oracle and the input generator under AddressSanitizer and
UndefinedBehaviorSanitizer: a C driver calls every exported function on
small inputs held in exact-size buffers; any out-of-bounds access, use after
free or undefined arithmetic aborts it. CPU only (gcc; no GPU code is built
with a sanitizer)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT


def test_oracle_and_generator_clean_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", exe,
           os.path.join(ROOT, "tests", "sanitize", "oracle_sanitize.c"),
           os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c"), "-lm"]
    subprocess.check_call(cmd)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all calls clean" in r.stdout
