"""Build libsinkattn.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m gqa_attention_sinks_amd.build`` or ``build()``.  Objects
go to ``gqa_attention_sinks_amd/_build/``; the library is written next to
this file.  Every call recompiles.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsinkattn.so")
SOURCES = ["api.hip", "append.hip", "decode.hip", "decode_balanced.hip", "moe.hip", "prefill.hip", "verify.hip"]

ARCH = "gfx950"
# Packed fp32 VALU forms are switched off for all device code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax reads and rescales them with VALU ops
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Kernel files only: the kernels never feed a NaN to min/max (masked scores are
# -inf and rows past the last key are zero-filled), so max chains compile to
# v_max3 without NaN canonicalisation.  The host validation in api.hip keeps
# full NaN semantics (it must reject a NaN softmax scale).
KERNEL_SOURCES = {"append.hip", "decode.hip", "decode_balanced.hip", "moe.hip", "prefill.hip", "verify.hip"}
KERNEL_FLAGS = ["-fno-honor-nans"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link ``out``; ``extra_flags`` (e.g. -D tuning
    switches) go to every compile."""
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        flags = FLAGS + (KERNEL_FLAGS if src in KERNEL_SOURCES else [])
        out = _run([cc, *flags, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
