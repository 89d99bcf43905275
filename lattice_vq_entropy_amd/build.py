"""Build libhq.so (HIP, gfx950) in-tree.

The library links the HIP runtime that PyTorch ships, so that a process that
also uses torch for device memory and streams has exactly one HIP runtime.
Device code is built with -ffp-contract=off (no FMA contraction: the fp32
decisions that pick lattice codes follow a fixed operation order) and without
packed fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhq.so")
# HQ_SANITIZE=1: a separate build, libhq_san.so, whose host code (plans,
# argument checks, layouts, header, CRC, calibration driver) carries
# AddressSanitizer and UndefinedBehaviorSanitizer checks; the device code is
# unchanged.  The sanitizer runtime is not linked in: preload clang's
# (libclang_rt.asan-x86_64.so under /opt/rocm/llvm/lib/clang/*/lib/linux).
SAN_LIB = os.path.join(HERE, "libhq_san.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all",
                  "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ["hq_kernels.hip", "hq_api.hip"]
HEADERS = ["hq_device.h", "hq_kernels.h", "hq_ws.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def torch_lib_dir() -> str:
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        raise RuntimeError("torch is required for its HIP runtime")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link libhq.so (libhq_san.so with
    sanitize: host code of hq_api.hip instrumented); always rebuilds."""
    objs = []
    bdir = os.path.join(HERE, "_build_san" if sanitize else "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        extra = SAN_HOST_FLAGS if (sanitize and src == "hq_api.hip") else []
        cmd = [HIPCC, *DEVICE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tlib = torch_lib_dir()
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    # (the sanitized library leaves the runtime's symbols to the preloaded runtime)
    strict = [] if sanitize else ["-Wl,--no-undefined", "-Wl,-z,defs"]
    cmd = ["/opt/rocm/llvm/bin/clang++", "-shared", "-fPIC", "-o", tmp, *objs,
           os.path.join(tlib, "libamdhip64.so"), f"-Wl,-rpath,{tlib}", *strict]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libhq.so failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv or os.environ.get("HQ_SANITIZE") == "1"))
