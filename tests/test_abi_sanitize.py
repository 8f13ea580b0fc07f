"""The C-ABI layer (bl_api.hip: argument validation, workspace queries,
per-thread error strings) with its host code built under AddressSanitizer and
UndefinedBehaviorSanitizer, driven by the CPU contract tests
(tests/test_abi_cpu.py) in a child process.  The device code and the other
objects are the in-tree build's.  CPU only."""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "bit_ternary_weight_amd")
BUILD = os.path.join(PKG, "_build")


def _asan_runtime():
    c = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return c[-1] if c else None


@pytest.mark.skipif(not os.path.isdir(BUILD), reason="in-tree objects not built (run __graft_entry__.build())")
@pytest.mark.skipif(_asan_runtime() is None, reason="clang ASan runtime not found")
def test_abi_validation_under_host_sanitizers(tmp_path):
    sys.path.insert(0, PKG)
    try:
        import build as blbuild
    finally:
        sys.path.pop(0)
    cc = blbuild.hipcc()
    flags = [f for f in blbuild.HIPCC_FLAGS if f not in ("-shared", "-O3")]
    san = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    obj = str(tmp_path / "bl_api_san.o")
    subprocess.run([cc, *flags, *san, "-c", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
                    os.path.join(PKG, "csrc", "bl_api.hip"), "-o", obj], check=True, capture_output=True)
    objs = [o for o in sorted(glob.glob(os.path.join(BUILD, "*.o"))) if os.path.basename(o) != "bl_api.o"]
    lib = str(tmp_path / "libbitlinear_san.so")
    subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, obj, "-o", lib],
                   check=True, capture_output=True)
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, BL_LIBRARY=lib, LD_PRELOAD=(_asan_runtime() + (" " + pre if pre else "")),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")], capture_output=True, text=True, env=env,
                       cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
