"""Compile the HIP libraries for gfx950 with hipcc.

* ``lib/libnvfp4.so``: the decode-projection library (every source in
  ``csrc/``), the C ABI of ``include/nvfp4.h``;
* ``lib/libnvfp4_probe.so``: the measurement and test probes of
  ``csrc/probe/`` (``include/nvfp4_probe.h``), which the projection library
  never calls.

Each source is compiled to an object under ``_build/``.  Flags:

* ``--offload-arch=gfx950`` only (no other targets, no CUDA);
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the compiler
  from emitting packed-FP32 VALU instructions;
* ``-mllvm -amdgpu-mfma-vgpr-form``: MFMA results in ordinary VGPRs, so the
  FP4-MFMA kernel scales them without copying each out of an AGPR first;
* ``-ffp-contract=off`` so no a*b+c is fused behind the code's back (the
  quantization recipe is a sequence of separately rounded float32 steps;
  the GEMV spells out every FMA it wants);
* IEEE float32 division and denormals are hipcc's defaults and are kept.
"""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIBDIR, "libnvfp4.so")
PROBE_LIB = os.path.join(LIBDIR, "libnvfp4_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
INCLUDE = os.path.join(ROOT, "include")

SOURCES = ["nvfp4_abi.cpp", "nvfp4_quant.hip", "nvfp4_gemv.hip", "nvfp4_sample.hip"]
PROBE_SOURCES = ["probe/nvfp4_probe.hip"]

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, src.replace("/", "_") + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-I", INCLUDE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def _link(objs: list, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link ``lib/libnvfp4.so`` and
    ``lib/libnvfp4_probe.so``; returns the projection library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


# Host-side checks: the library with its host code (the C ABI layer and the
# launchers) built with AddressSanitizer and UndefinedBehaviorSanitizer; the
# device code is the normal build.  Tests load it with the ASan runtime
# preloaded and drive the argument validation on the CPU.
SANITIZE_FLAGS = COMMON_FLAGS + [
    "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that matches hipcc."""
    import glob

    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no clang AddressSanitizer runtime under /opt/rocm/lib/llvm")
    return hits[-1]


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Compile the host side of every source with ASan + UBSan and link
    ``out_dir/libnvfp4_hostsan.so``; returns its path."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, src.replace("/", "_") + ".o")
        cmd = [hipcc(), *SANITIZE_FLAGS, "-I", INCLUDE, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized host build failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 4)) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libnvfp4_hostsan.so")
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", *objs, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host link failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
