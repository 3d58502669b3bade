"""Build the gfx950 shared library libmoe_finalize.so in-tree with hipcc.

    python combine_moe_finalize_amd/build.py

Flags: fp-contract off (the finalize's fp32 operation order is part of its
contract: a separate multiply and add per gathered row, no fused
multiply-add), packed-fp32 instructions disabled, kernel-argument preload,
-O3, gfx950 only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

try:
    from ._paths import CSRC, INCLUDE, LIB_DIR, LIB_PATH, PROBE_LIB_PATH
except ImportError:            # run as a script
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from _paths import CSRC, INCLUDE, LIB_DIR, LIB_PATH, PROBE_LIB_PATH

SOURCES = ["moef_api.hip", "finalize_kernels.hip", "routing_kernels.hip", "act_quant_kernels.hip",
           "allreduce_kernels.hip"]
ARCH = "gfx950"
# Kernel arguments preloaded into SGPRs at wave start (gfx950 holds up to 14
# dwords there beside the kernel-argument pointer). A kernel with pointer and
# scalar parameters then starts without a dependent load of its arguments;
# the compiler adds a 256-byte prologue that loads them itself when the
# firmware does not preload. Parameters passed as a struct are not preloaded.
KERNARG_PRELOAD = 16


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return p


def compile_command(out: str) -> list:
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}",
            "-fPIC", "-shared", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", f"-amdgpu-kernarg-preload-count={KERNARG_PRELOAD}",
            "-Wall", "-Wno-unused-function",
            "-I", INCLUDE, "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES],
            "-o", out]


def build(verbose: bool = False) -> str:
    """Compile the library (always, even if one is present). Returns its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_probes() -> str:
    """Compile the streaming read / copy probe library the benchmark measures
    its same-session ceilings with (always, like the main library)."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = PROBE_LIB_PATH + ".tmp"
    cmd = [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
           "-I", CSRC, os.path.join(CSRC, "bandwidth_probes.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, PROBE_LIB_PATH)
    return PROBE_LIB_PATH


C_DRIVER_SRC = os.path.join(os.path.dirname(os.path.dirname(LIB_DIR)), "tests", "c",
                            "abi_driver.c")
C_DRIVER = os.path.splitext(C_DRIVER_SRC)[0]


def build_c_driver() -> str:
    """Compile the plain-C ABI driver used by the tests (gcc, links the library
    and the HIP runtime; the library is found through a relative rpath)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_DRIVER_SRC,
           "-L", LIB_DIR, "-lmoe_finalize", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../combine_moe_finalize_amd/_lib",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", C_DRIVER]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return C_DRIVER


HOST_CHECKS = os.path.join(os.path.dirname(C_DRIVER_SRC), "host_checks")


def build_host_checks() -> str:
    """Compile the C-ABI argument checks against host-only launch stubs with
    the address and undefined-behaviour sanitizers on the host side (no GPU
    code is built with them)."""
    cdir = os.path.dirname(C_DRIVER_SRC)
    sanitize = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    cmd = [hipcc(), "-O1", "-g", "-std=c++17", *sanitize,
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, "moef_api.hip"),
           os.path.join(cdir, "launch_stub.cpp"), os.path.join(cdir, "host_checks.cpp"),
           "-o", HOST_CHECKS]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr}")
    return HOST_CHECKS


HOST_STUB_LIB = os.path.join(os.path.dirname(C_DRIVER_SRC), "libmoef_host_stub.so")


def build_host_stub_lib() -> str:
    """The C-ABI entry points linked against the host-only launch stubs as a
    shared library (no GPU code runs; the stubs count launches), for tests
    that drive the argument checks from Python."""
    cdir = os.path.dirname(C_DRIVER_SRC)
    cmd = [hipcc(), "-O1", "-std=c++17", "-fPIC", "-shared", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, "moef_api.hip"), os.path.join(cdir, "launch_stub.cpp"),
           "-o", HOST_STUB_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr}")
    return HOST_STUB_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probes())
    print(build_c_driver())
    print(build_host_checks())
    print(build_host_stub_lib())
