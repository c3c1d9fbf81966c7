"""Build libcar.so (the HIP kernels and the C-ABI shim) for gfx950, in-tree.

    python causal_attention_rope_amd/build.py [--sanitize]

(Run as a script: importing the package loads libcar.so, which the build
creates.)

Compiles every source under ``csrc/`` with hipcc for ``--offload-arch=gfx950``
into ``_build/`` and links ``libcar.so`` next to this file.  Always rebuilds.

``--sanitize`` builds ``libcar_san.so`` instead: the same sources with the
host code under AddressSanitizer and UndefinedBehaviorSanitizer (device code
unsanitized and unoptimised: this build is for the host-side ABI checks on a
machine without a GPU and is never launched).  The package loads it when
CAR_LIBRARY names it, with the sanitizer runtime (``asan_runtime()``)
preloaded.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcar.so")

SOURCES = ["rope_cache.hip", "decode.hip", "decode_i8.hip", "prefill.hip", "car_api.cpp",
           "decode_noalloc.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    # packed fp32 VALU ops stay disabled (scalar fp32 arithmetic only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcar.so)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # keep compiler diagnostics visible, minus the known host-pass notice
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def check_defined(lib: str) -> None:
    """Fail if the library leaves any of its own symbols undefined (a kernel
    whose host launch stub was not emitted would only fail at load time)."""
    r = subprocess.run(["nm", "-C", "-u", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return  # nm unavailable: the load test in tests/ still catches it
    missing = [ln.strip() for ln in r.stdout.splitlines() if "car::" in ln]
    if missing:
        raise RuntimeError("libcar.so has undefined symbols:\n" + "\n".join(missing))


SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(HERE, "libcar_san.so")
# host code: ASan + UBSan (every -fsanitize= for the host pass only); the
# device code is optimized as usual (its inline assembly needs the operands
# that optimization keeps in scalar registers)
SAN_FLAGS = [
    f"--offload-arch={ARCH}", "-O1", "-Xarch_device", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_LINK = ["-fsanitize=address,undefined", "-shared-libsan"]


def clangxx() -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cand = os.path.join(rocm, "llvm", "bin", "clang++")
    if not os.path.exists(cand):
        raise RuntimeError(f"{cand} not found (ROCm's clang links the sanitized build)")
    return cand


def asan_runtime() -> str:
    """Path of the shared ASan runtime the sanitized library links against."""
    r = subprocess.run([clangxx(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(SAN_BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc(), *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stderr}")
        return obj
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(one, SOURCES))
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib")
    tmp = SAN_LIB + ".tmp"
    link = [clangxx(), "-shared", "-fPIC", *SAN_LINK, *objs, "-L", rocm_lib,
            f"-Wl,-rpath,{rocm_lib}", "-lamdhip64", "-o", tmp]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(link)}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    check_defined(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if sys.argv[1:] == ["--sanitize"]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True, extra_flags=sys.argv[1:])
