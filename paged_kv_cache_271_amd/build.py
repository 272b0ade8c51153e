"""Build libpagedkv.so for gfx950 with hipcc, in-tree.

Usage: python -m paged_kv_cache_271_amd.build  (or call build()).

build_host_sanitized() builds libpagedkv_host_san.so instead: the host
sources alone (allocator, slot mapping, reservations, prefix cache, launch
planning, argument checks) with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, every device launch replaced by a stub that
returns KV_E_HIP.  Load it with the ASan runtime preloaded
(sanitizer_env()) and PAGEDKV_LIB pointing at it.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libpagedkv.so")
SOURCES = ["pool.cpp", "prefix.cpp", "plan.cpp", "append.hip", "copy.hip", "decode.hip", "prefill.hip", "probe.hip", "noalloc.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-precision / and sqrt correctly rounded (the fp8 scale rule relies on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose=False, extra_flags=()):
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so: harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


HOST_SOURCES = ["pool.cpp", "prefix.cpp", "plan.cpp", "sanitize_stubs.cpp"]
SAN_LIB_PATH = os.path.join(LIB_DIR, "libpagedkv_host_san.so")


def build_host_sanitized():
    """g++ build of the host half with ASan + UBSan (no device code)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = SAN_LIB_PATH + ".tmp"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in HOST_SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, SAN_LIB_PATH)
    return SAN_LIB_PATH


def sanitizer_env(lib_path=SAN_LIB_PATH):
    """Environment for a Python process that loads the sanitizer build: the
    ASan runtime preloaded (Python itself is not instrumented), leak checks
    off (the interpreter keeps memory until exit), any report fatal."""
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    env = dict(os.environ)
    env["LD_PRELOAD"] = libasan
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PAGEDKV_LIB"] = lib_path
    return env


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
