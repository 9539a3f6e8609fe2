"""Build libqlin.so (hand-written HIP for gfx950) in-tree.

    python -m decode_nvfp4_rtn_amd.build              # libqlin.so
    python -m decode_nvfp4_rtn_amd.build --sanitize   # host ASan/UBSan build

Each translation unit is compiled with hipcc for gfx950 only, then linked
into ``decode_nvfp4_rtn_amd/libqlin.so``.  Flags:
* ``-O3 -std=c++17 -fPIC``;
* packed-fp32 instructions disabled for the device (the compiler may not
  synthesise v_pk_{add,mul,fma}_f32);
* no fast-math anywhere: divisions stay correctly rounded and denormals are
  kept;
* ``-ffp-contract=off`` for the quantizers and for the per-wave W4A4 GEMM,
  whose fused variant runs the activation encoder, so no multiply is fused
  into an add and every binary32 step rounds once;
* the W4A4 block-cooperative GEMM is scheduled with the compiler's
  memory-clause strategy, which keeps its loads and LDS reads in tighter
  groups: 0.5-3.3 % faster over the Qwen3-8B-like and 27B-class prefill
  shapes (interleaved timing in one process, outputs bit-identical).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqlin.so")
ARCH = "gfx950"

SOURCES = {
    "api.cpp": [],
    "quantize.hip": ["-ffp-contract=off"],
    "weight_prep.hip": ["-ffp-contract=off"],
    "repack.hip": [],
    "gemm_w4a4.hip": ["-ffp-contract=off"],
    "gemm_w4a4_coop.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    "gemm_decode.hip": [],
    "gemm_sparse.hip": [],
}

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Host code with AddressSanitizer and UndefinedBehaviorSanitizer (each flag
# after -Xarch_host: the device code is built exactly as in libqlin.so).  The
# library expects the sanitizer runtime to be preloaded into the process
# (LD_PRELOAD of sanitizer_runtime()); tests/test_abi_sanitized.py runs the
# C-ABI tests on it.
SANITIZE = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
BUILD_SAN = os.path.join(HERE, "_build_asan")
LIB_SAN = os.path.join(BUILD_SAN, "libqlin_asan.so")


def sanitizer_runtime():
    """Path of the compiler's shared AddressSanitizer runtime (with UBSan)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    return r.stdout.strip()


def _compile(src, extra, out_dir=BUILD):
    obj = os.path.join(out_dir, src + ".o")
    cmd = [_hipcc(), *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True):
    """Compile every source and link libqlin.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(verbose=True):
    """The same sources with sanitized host code, linked into
    _build_asan/libqlin_asan.so (not loaded by the package); returns its path."""
    os.makedirs(BUILD_SAN, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], [*kv[1], *SANITIZE], BUILD_SAN),
                           SOURCES.items()))
    tmp = LIB_SAN + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_SAN)
    if verbose:
        print(f"built {LIB_SAN}")
    return LIB_SAN


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
    sys.exit(0)
