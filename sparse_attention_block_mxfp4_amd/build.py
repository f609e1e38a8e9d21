"""Build ``libmi_idx.so`` in-tree with hipcc for gfx950.

Every HIP source under ``csrc/`` goes into one shared library next to this
file.  All device code is compiled with packed-fp32 instructions disabled.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["api.hip", "insert.hip", "decode.hip", "prefill.hip"]
LIB = os.path.join(HERE, "libmi_idx.so")


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libmi_idx.so)")
    return exe


def build(verbose=False, extra=()):
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # device code: no NaN operands reach max/compare (keys test NaN on
           # the bits), MFMA results stay in VGPRs
           "-Xarch_device", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-I", os.path.join(ROOT, "include"), *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
