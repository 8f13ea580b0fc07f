"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host only) and driven through every exported function on small ragged
shapes with exactly sized buffers (tests/sanitize_oracle.c): no out-of-bounds
access, no undefined arithmetic.  CPU only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "san_oracle")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-ffp-contract=off", os.path.join(ROOT, "oracle", "bitlinear_oracle.c"),
           os.path.join(HERE, "sanitize_oracle.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checksum" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
