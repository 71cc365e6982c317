"""Build libattn.so (the C-ABI attention library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libattn.so")
SOURCES = ["api.hip", "decode.hip", "fwd.hip", "bwd.hip", "probe.hip"]
# A plain C caller of the library (no Python in its process), run by the C-ABI GPU test.
CAPI_SRC = os.path.join(ROOT, "tests", "capi", "attn_capi_check.c")
CAPI_BIN = os.path.join(ROOT, "tests", "capi", "attn_capi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source for gfx950 and link libattn.so. Returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        jobs.append((obj, [cc, *COMMON, *DEVICE_FLAGS, *extra_flags, "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(min(len(jobs), 8)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB_PATH + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB_PATH)
    build_capi_check()
    return LIB_PATH


def build_capi_check() -> str:
    """Compile the C caller as C99 with the host C compiler against include/attn.h and the system HIP
    runtime; it finds libattn.so through a run path relative to itself."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C-ABI check program")
    tmp = CAPI_BIN + ".tmp"
    _run([cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", INCLUDE, CAPI_SRC, "-o", tmp, "-L", PKG, "-l:libattn.so", "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../attention_attn_decode_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, CAPI_BIN)
    return CAPI_BIN


if __name__ == "__main__":
    print(build(verbose=True))
