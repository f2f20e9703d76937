"""Build the HIP attention library ``libfa.so`` for gfx950, in-tree.

Usage: ``python -m exact_attention_110_amd.build`` (or ``build()`` from Python).
Each translation unit is compiled with hipcc in parallel and linked into
``exact_attention_110_amd/libfa.so``. Every call recompiles.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "fp8.hip"]
# Kernel translation units never produce or test for NaN on purpose, so the
# compiler may drop the NaN quieting it otherwise inserts around every float
# max; the argument checks in api.hip keep full IEEE semantics.
#
# The attention kernels run one or two waves per SIMD, so their speed rests on
# how well one wave's instruction stream overlaps matrix-core work with the
# softmax arithmetic and the LDS reads; LLVM's iterative ILP scheduling
# strategy orders the tile loops better than its default occupancy-driven one
# (2-4% on the long causal bf16 workload, forward and both backward kernels).
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
PER_FILE = {"fwd.hip": ["-fno-honor-nans", *_ILP], "bwd.hip": ["-fno-honor-nans", *_ILP],
            "fp8.hip": ["-fno-honor-nans"]}

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # float atomics as hardware add instructions
    "-munsafe-fp-atomics",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the library needs ROCm's hipcc to build")


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *PER_FILE.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, extra=()):
    """Compile every source and link libfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build of the C ABI's argument checking: api.hip with
# AddressSanitizer and UndefinedBehaviorSanitizer on its host code only (the
# device code is built as usual), linked with the kernel objects of the
# regular build into _build/libfa_sanitized.so. Loading it needs the ASan
# runtime preloaded (``asan_runtime()``); tests/test_abi_sanitized.py runs the
# C-ABI tests against it on the CPU.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(BUILD, "libfa_sanitized.so")


def asan_runtime():
    """Path of the AddressSanitizer runtime that belongs to hipcc's clang."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_sanitized():
    """Compile api.hip with host sanitizers and link it with the regular
    build's kernel objects (built first when missing); returns the path."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "api.hip":
            obj = os.path.join(BUILD, "api_sanitized.o")
            cmd = [_hipcc(), *FLAGS, *SANITIZE, "-c", os.path.join(CSRC, "api.hip"), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for the sanitized api.hip:\n{r.stderr}")
        else:
            obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                obj, _ = _compile(src, [])
        objs.append(obj)
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE, "-o", SANITIZED_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
