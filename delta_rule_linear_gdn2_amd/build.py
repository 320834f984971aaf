"""Build the gfx950 HIP library ``libgdn2.so`` in-tree with hipcc.

Every source is compiled for gfx950 only, with code-object v5 (loadable by
the HIP 7.0 runtime that PyTorch bundles as well as the system ROCm 7.2
runtime) and with packed-FP32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn2.so")

SOURCES = [
    "gdn2_api.cpp",
    "recurrent_step.hip",
    "chunk_fwd_simple.hip",
    "chunk_fwd_mfma.hip",
    "chunk_bwd.hip",
    "chunk_bwd_mfma.hip",
    "mixer.hip",
    "scratch.hip",
    "segments.hip",
]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every source and link ``libgdn2.so``; returns the library path."""
    extra = list(extra or [])
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1, len(SOURCES))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the C ABI's
# argument checking (gdn2_api.cpp holds no device code; every sanitizer flag
# is host-only).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_RUNTIME = "libclang_rt.asan-x86_64.so"


def sanitizer_runtime_dir() -> str:
    """Directory of the clang sanitizer runtime the sanitized build links."""
    r = subprocess.run([HIPCC, "-print-resource-dir"], capture_output=True, text=True, check=True)
    return os.path.join(r.stdout.strip(), "lib", "linux")


def build_sanitized(out_dir: str) -> str:
    """``libgdn2_asan.so`` in out_dir: gdn2_api.cpp built with the host
    sanitizers, linked with the kernels' regular objects (built here if
    missing).  Load it with the clang sanitizer runtime preloaded."""
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "gdn2_api.cpp":
            obj = os.path.join(out_dir, "gdn2_api_asan.o")
            cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-Wall", *SAN_FLAGS,
                   f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"sanitized build of {src} failed:\n{' '.join(cmd)}\n{r.stderr}")
            objs.append(obj)
        else:
            obj = os.path.join(BUILD, os.path.basename(src) + ".o")
            if not os.path.exists(obj):
                os.makedirs(BUILD, exist_ok=True)
                obj = _compile(src, [])
            objs.append(obj)
    lib = os.path.join(out_dir, "libgdn2_asan.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libsan", "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(cmd)}\n{r.stderr}")
    return lib


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    print(build(sys.argv[1:]))
