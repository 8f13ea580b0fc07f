"""Build libbitlinear.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m bit_ternary_weight_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbitlinear.so")

SOURCES = ["bl_api.hip", "k_quant.hip", "k_ternarize.hip", "k_gemv.hip", "k_gemv_mt.hip", "k_gemm.hip", "k_attn.hip", "k_attn_prefill.hip", "k_ste.hip", "k_unpacked.hip", "k_chain.hip", "k_binary.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Exact fp32 arithmetic in the scale / rescale paths.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # Keep the compiler from forming packed fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source to an object (in parallel; each kernel is launched
    from the file that defines it), then link the shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = []
    cmds = []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *compile_flags, "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
