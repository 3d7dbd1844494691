"""Build libwaveprune.so for gfx950 with hipcc (in-tree, no JIT cache).

python -m rope_positional_encoding_amd.build [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwaveprune.so")
CHECK = os.path.join(ROOT, "tests", "c_abi_check")
SOURCES = ["api.hip", "rope.hip", "prefill.hip", "prefill16.hip", "decode.hip", "backward.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 VALU forms are switched off for all device code.  IEEE mode is
# off (no signaling-NaN quieting before min/max, so row maxima become
# v_max3 chains); the kernels never produce or consume NaNs.
COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mno-amdgpu-ieee", "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source options.  The prefill kernel is scheduled with LLVM's max-ILP
# strategy (AMDGPU machine scheduler): same instructions, about 1% faster at
# 32K than the default occupancy-first strategy, no spills (the occupancy is
# fixed at two waves per SIMD by the register budget anyway).
SOURCE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the device feature: drop that one warning
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    # the tests' standalone C++ user of the C ABI (host code only, no torch)
    _run([HIPCC, *COMMON, os.path.join(ROOT, "tests", "c_abi_check.cpp"), "-o", CHECK, "-L", PKG,
          "-lwaveprune", "-Wl,-rpath,$ORIGIN/../rope_positional_encoding_amd"], verbose)
    build_host_check(verbose)
    return LIB


# The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
# linked with host stand-ins of the kernel launchers (tests/host_check/), for
# the CPU tests.  The sanitizers apply to host code only (-Xarch_host); the
# link is a host-only step.
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_CHECK = os.path.join(ROOT, "tests", "host_check", "host_check")


def build_host_check(verbose: bool = False) -> str:
    out = os.path.join(BUILD, "san")
    os.makedirs(out, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", *SAN_HOST,
             "-I", os.path.join(ROOT, "include")]
    srcs = [os.path.join(CSRC, "api.hip"), os.path.join(ROOT, "tests", "host_check", "launch_stubs.cpp"),
            os.path.join(ROOT, "tests", "host_check", "host_check.cpp")]
    objs = [os.path.join(out, os.path.basename(s).split(".")[0] + ".o") for s in srcs]
    for s, o in zip(srcs, objs):
        _run([HIPCC, *flags, "-c", s, "-o", o], verbose)
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    _run([clang, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", HOST_CHECK], verbose)
    return HOST_CHECK


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
