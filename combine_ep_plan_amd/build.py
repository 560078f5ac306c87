"""Build libep_mi355x.so (HIP kernels for gfx950 + the C ABI) in the package
directory with hipcc.  Usage: ``python -m combine_ep_plan_amd.build``.

``--host-sanitize`` builds libep_mi355x_hostsan.so instead: the kernels as
usual, the host runtime (ep_api.cpp, host code only) compiled by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer, for CPU-only checks of the
C ABI (load it with EP_MI355X_LIB and the sanitizer runtimes preloaded)."""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libep_mi355x.so")
OUT_HOSTSAN = os.path.join(PKG, "libep_mi355x_hostsan.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# Packed fp32 instructions are switched off for every device pass; hipcc's
# host pass does not know the feature and says so (harmless).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}"]
SOURCES = ["route.hip", "plan.hip", "dispatch.hip", "combine.hip", "dup_reduce.hip", "prefetch.hip",
           "gemm.hip", "scratch.hip", "ep_api.cpp"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build the library")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


# The host runtime has no device code, so the sanitized variant compiles it
# with the host compiler alone; no device pass is ever instrumented.
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def _compile_host_sanitized(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".hostsan.o")
    cmd = ["g++", "-O1", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}", *SAN_FLAGS,
           "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    device_srcs = [s for s in SOURCES if s.endswith(".hip")]
    host_srcs = [s for s in SOURCES if not s.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, device_srcs))
        objs += list(ex.map(_compile_host_sanitized if host_sanitize else _compile, host_srcs))
    out = OUT_HOSTSAN if host_sanitize else OUT
    tmp = out + ".tmp"
    if host_sanitize:   # the sanitizer runtimes come from the host compiler's link
        cmd = ["g++", "-shared", "-fPIC", *objs, *SAN_FLAGS, f"-L{ROCM}/lib",
               f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-o", tmp]
    else:
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, host_sanitize="--host-sanitize" in sys.argv[1:])
    sys.exit(0)
