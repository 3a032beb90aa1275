"""Build librehyat.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m hybrid_softmax_linear_amd.build        # or: from ... import build; build.build()
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librehyat.so")
ARCH = "gfx950"

SOURCES = ["attn_bf16.hip", "state_bf16.hip", "reduce.hip", "f32_path.hip", "bwd_bf16.hip", "api.cpp"]

# Packed fp32 VALU ops are switched off for all device code (ordinary fp32 math only).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librehyat)")


# Per-file extra flags. The attention kernel keeps its MFMA results in VGPRs (the softmax
# reads every S^T element with VALU; AGPR results would need a copy per element).
EXTRA = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + lang + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link librehyat.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking librehyat.so failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of ROCm's clang (to preload into a process that
    loads the sanitized library)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's shared AddressSanitizer runtime not found under /opt/rocm/llvm")
    return hits[-1]


def build_host_sanitized(out: str) -> str:
    """A copy of librehyat.so whose host code of the C ABI (api.cpp: argument checks,
    workspace layout, launch sequences) is built with AddressSanitizer and
    UndefinedBehaviorSanitizer; the kernels are the regular objects (device code is not
    sanitized). For host-side tests only: load it with the runtime from asan_runtime()
    preloaded. Returns the library path."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o"))
               for s in SOURCES if s != "api.cpp"):
        build(verbose=False)
    obj = os.path.join(BUILD, "api_hostsan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = ([hipcc(), "-x", "hip"] + FLAGS + san + ["-c", os.path.join(CSRC, "api.cpp"), "-o", obj])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling api.cpp with host sanitizers failed:\n{res.stderr}")
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.cpp"]
    cmd = ([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-o", out, obj] + objs)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking the sanitized library failed:\n{res.stderr}")
    return out


if __name__ == "__main__":
    build()
