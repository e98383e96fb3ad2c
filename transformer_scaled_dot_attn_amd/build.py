"""Build libattn.so (the gfx950 kernels and the C-ABI) in place with hipcc.

    python -m transformer_scaled_dot_attn_amd.build

Compiles every source under csrc/ for gfx950 and links the shared library
next to this file.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.cpp", "generic_f32.hip", "prefill_bf16.hip", "decode_bf16.hip",
           "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def compile_flags() -> list:
    # Packed FP32 instructions are disabled for the device code; the host pass
    # warns that it does not know the feature, which is harmless.
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libattn.so failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_sanitized(out_dir: str) -> str:
    """A copy of the library whose HOST code is built with AddressSanitizer
    and UndefinedBehaviorSanitizer (the device code is the ordinary build):
    for running the CPU tests of the argument checks, workspace sizing and
    kernel planning under the sanitizers.  Loading it needs the clang ASan
    runtime preloaded (asan_runtime()).  Returns the library's path."""
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer"]
    flags = compile_flags() + ["-Xarch_host", "-g"] + san

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        res = subprocess.run([hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compiling {src} with sanitizers failed:\n{res.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(5, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, "libattn_sanitized.so")
    clangxx = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin",
                           "clang++")
    if not os.path.exists(clangxx):
        clangxx = "/opt/rocm/llvm/bin/clang++"
    res = subprocess.run([clangxx, "-shared", "-fPIC", "-fsanitize=address,undefined", "-o", lib]
                         + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking the sanitized library failed:\n{res.stderr}")
    return lib


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized builds link against."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    build(verbose=True)
