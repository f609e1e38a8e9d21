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
SOURCES = ["api.hip", "insert.hip", "decode.hip", "prefill.hip", "select.hip", "general.hip"]
LIB = os.path.join(HERE, "libmi_idx.so")
# HBM read-ceiling probes (a measurement aid of the benchmark, not the indexer)
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(HERE, "libmi_idx_probe.so")


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libmi_idx.so)")
    return exe


# Per-source code-generation flags.  The prefill scorer is scheduled for
# instruction-level parallelism (measured ~1.6 % faster on the mixed step; the
# decode scorer is slightly slower with it and keeps the default scheduler).
PER_SOURCE = {"prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results stay in VGPRs.  NaN is honoured: page maxima
            # propagate it (IEEE maximum), which -fno-honor-nans would let the
            # compiler turn back into the NaN-dropping max.
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")


def _build_lib(sources, lib, verbose, extra):
    from concurrent.futures import ThreadPoolExecutor
    tmp = lib + ".tmp"
    objs = [os.path.join(HERE, "_build_" + name.replace(".hip", ".o")) for name in sources]
    try:
        cmds = [[hipcc(), *_flags(), *PER_SOURCE.get(name, []), *extra, "-c",
                 os.path.join(HERE, "csrc", name), "-o", obj] for name, obj in zip(sources, objs)]
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(tmp, lib)
    return lib


# Host-code sanitizer build (CPU checks of the argument validation and the
# prefill planning): AddressSanitizer + UndefinedBehaviorSanitizer on the
# host pass only; device code is compiled as usual.
SANITIZE_FLAGS = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-omit-frame-pointer " \
                 "-Xarch_host -g".split()
SANITIZE_DIR = os.path.join(HERE, "_sanitize")


def asan_runtime():
    """The ASan runtime of hipcc's clang, to preload into the test process."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return found[-1]


def sanitize_check(verbose=False):
    """Build libmi_idx.so with sanitized host code into _sanitize/ and run the
    CPU ABI tests (argument errors, prefill planning) against it with the
    ASan runtime preloaded; returns pytest's exit status."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    lib = os.path.join(SANITIZE_DIR, "libmi_idx.so")
    _build_lib(SOURCES, lib, verbose, SANITIZE_FLAGS)
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), MI_IDX_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi.py")]
    print(" ".join(f"{k}={env[k]}" for k in ("LD_PRELOAD", "MI_IDX_LIB", "ASAN_OPTIONS",
                                              "UBSAN_OPTIONS")), " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


def build(verbose=False, extra=()):
    """Compile every source (one object each, with its own flags) and link
    them into libmi_idx.so, and the probes into libmi_idx_probe.so; a library
    is replaced only when all its sources compile."""
    _build_lib(SOURCES, LIB, verbose, extra)
    _build_lib(PROBE_SOURCES, PROBE_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    if "--sanitize-check" in sys.argv:
        sys.exit(sanitize_check(verbose=True))
    print(build(verbose=True))
