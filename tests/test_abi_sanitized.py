"""The host-side ABI tests again, against the sanitized build.

``tests/test_abi_cpu.py`` runs in a child process that loads
``libcar_san.so`` (host code under AddressSanitizer and
UndefinedBehaviorSanitizer; see ``causal_attention_rope_amd/build.py
--sanitize``) with the ASan runtime preloaded.  Any sanitizer report ends the
child with an error, so a pass means every host check those tests drive ran
without a memory error or undefined behaviour.  No GPU is used.
"""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "causal_attention_rope_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_car_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stale(lib: str) -> bool:
    """Whether lib is missing or older than any source or header it is built from."""
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    dirs = [os.path.join(ROOT, "causal_attention_rope_amd", "csrc"), os.path.join(ROOT, "include")]
    return any(os.path.getmtime(os.path.join(d, f)) > t for d in dirs for f in os.listdir(d))


def test_abi_checks_are_clean_under_asan_and_ubsan():
    b = _build_module()
    if _stale(b.SAN_LIB):
        b.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": b.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "CAR_LIBRARY": b.SAN_LIB,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert "passed" in r.stdout
