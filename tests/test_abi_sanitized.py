"""The C-ABI checks of test_abi.py on a build of the same sources whose host
code carries AddressSanitizer and UndefinedBehaviorSanitizer (device code as
in libqlin.so), run in a child process with the sanitizer runtime preloaded.

Any out-of-bounds access, use after free or undefined behaviour (overflow,
misaligned access, invalid shift) in the argument checking, size arithmetic,
blob layout or launch planning that those calls reach ends the child with a
report and fails the test.  Leak detection is off: the library imports no
allocation function at all (checked below), and CPython's own objects alive
at exit would be reported as leaks.  No GPU is needed: every call returns
before a launch.
"""

import os
import subprocess
import sys

from decode_nvfp4_rtn_amd import build as qb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ALLOC = ("malloc", "calloc", "realloc", "free", "_Znwm", "_Znam", "_ZdlPv", "_ZdaPv",
         "hipMalloc", "hipMallocAsync", "hipFree", "hipFreeAsync", "hipHostMalloc",
         "hipMallocManaged", "hipExtMallocWithFlags")


def _undefined(lib):
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}


def test_library_imports_no_allocator():
    assert os.path.exists(qb.LIB), "build libqlin.so first (python -m decode_nvfp4_rtn_amd.build)"
    assert not (_undefined(qb.LIB) & set(ALLOC))


def test_abi_under_host_sanitizers():
    lib = qb.build_sanitized(verbose=False)
    exported = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in exported and "__ubsan_handle" in exported   # instrumented
    assert not (_undefined(lib) & set(ALLOC))
    rt = qb.sanitizer_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["QLIN_ABI_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "AddressSanitizer" not in r.stderr
