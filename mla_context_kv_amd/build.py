"""Build libdcp.so (HIP kernels for gfx950 + the C ABI of include/dcp.h) in-tree.

Every .hip file under csrc/ is compiled to an object with hipcc for gfx950 and
linked into mla_context_kv_amd/libdcp.so.  The streaming-read probe under
probe/ (a measurement tool, not part of the attention path) is linked into its
own library, mla_context_kv_amd/libdcp_probe.so.  Packed-FP32 instructions are
disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROBE_SRC = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libdcp_probe.so")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdcp.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: ROCm is required to build libdcp")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """Compile every kernel source, link libdcp.so and libdcp_probe.so; returns libdcp's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PROBE_SRC, "*.hip")))
    if not srcs or not probe_srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    build_abi_client(verbose)
    build_sanitized(verbose)
    return LIB


ABI_CLIENT_SRC = os.path.join(ROOT, "tests", "abi_client.c")
ABI_CLIENT = os.path.join(ROOT, "tests", "abi_client")


def build_abi_client(verbose: bool = True) -> str:
    """Compile the plain C client of the C ABI (host code only: gcc against
    the HIP runtime and libdcp.so, found through its run path)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-O2", "-Wall", "-std=c11", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           f"-I{INCLUDE}", ABI_CLIENT_SRC, "-o", ABI_CLIENT,
           f"-L{rocm}/lib", "-lamdhip64", f"-L{PKG}", "-ldcp", f"-Wl,-rpath,{rocm}/lib",
           "-Wl,-rpath,$ORIGIN/../mla_context_kv_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling the C ABI client failed:\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {ABI_CLIENT}")
    return ABI_CLIENT


# The host-side argument checks of the C ABI, built with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (each sanitizer flag is
# given to the host compilation alone; the GPU code is built as usual) and
# linked with a C driver that calls every entry point with arguments the
# library must reject or answer on the host.  Runs on the CPU (tests/).
SAN_HOST_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_DRIVER_SRC = os.path.join(ROOT, "tests", "abi_errors.c")
SAN_DRIVER = os.path.join(ROOT, "tests", "abi_errors_san")


def llvm_tool(name: str) -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    exe = os.path.join(rocm, "lib", "llvm", "bin", name)
    if not os.path.exists(exe):
        raise RuntimeError(f"{exe} not found")
    return exe


def _compile_sanitized(src: str) -> str:
    obj = os.path.join(BUILD_DIR, "san_" + os.path.basename(src) + ".o")
    flags = [f for f in COMMON_FLAGS if f != "-O3"]
    cmd = [hipcc(), *flags, *SAN_HOST_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} with host sanitizers failed:\n{r.stdout}{r.stderr}")
    return obj


def build_sanitized(verbose: bool = True) -> str:
    """The ABI error-path driver against a copy of the library whose host code
    carries AddressSanitizer and UndefinedBehaviorSanitizer."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile_sanitized, srcs))
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    sanitize = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    drv = os.path.join(BUILD_DIR, "abi_errors.o")
    r = subprocess.run([llvm_tool("clang"), "-std=c11", "-O1", "-Wall", *sanitize, "-D__HIP_PLATFORM_AMD__",
                        f"-I{rocm}/include", f"-I{INCLUDE}", "-c", SAN_DRIVER_SRC, "-o", drv],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling the sanitized ABI driver failed:\n{r.stdout}{r.stderr}")
    r = subprocess.run([llvm_tool("clang++"), *sanitize, "-o", SAN_DRIVER, drv, *objs, f"-L{rocm}/lib",
                        "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking the sanitized ABI driver failed:\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"built {SAN_DRIVER}")
    return SAN_DRIVER


if __name__ == "__main__":
    build()
