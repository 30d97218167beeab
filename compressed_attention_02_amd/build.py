"""Build libv4attn.so in-tree with hipcc for gfx950.

Every .hip / .cpp file under csrc/ is compiled to an object in _build/ (in
parallel) and the objects are linked into compressed_attention_02_amd/libv4attn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libv4attn.so")

ARCH = "gfx950"
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", src, "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(SRC, f) for f in os.listdir(SRC) if f.endswith((".hip", ".cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


# Host-side sanitizers: api.cpp (argument checks, plans, workspace layout, the
# status and timing tables) built with AddressSanitizer and UndefinedBehaviorSanitizer
# on its host pass only (-Xarch_host: the device code is built as usual), linked
# with the kernels' objects of build() into a separate library.  A process that
# loads it needs the ASan runtime preloaded (asan_runtime()).
SAN_DIR = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libv4attn_sanitized.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all", "-g"]


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (it carries the UBSan handlers too)."""
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"ASan runtime not found ({path!r})")
    return path


def build_sanitized() -> str:
    srcs = [f for f in os.listdir(SRC) if f.endswith((".hip", ".cpp"))]
    newest = max(os.path.getmtime(os.path.join(d, f)) for d in (SRC, os.path.join(ROOT, "include"))
                 for f in os.listdir(d))
    objs_ok = all(os.path.exists(os.path.join(BUILD, f + ".o")) and
                  os.path.getmtime(os.path.join(BUILD, f + ".o")) >= newest for f in srcs)
    if not objs_ok:   # the kernels' objects come from the regular build
        build()
    os.makedirs(SAN_DIR, exist_ok=True)
    obj = os.path.join(SAN_DIR, "api.cpp.o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(SRC, "api.cpp"), "-o", obj] + FLAGS + SAN_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    objs = [obj] + sorted(os.path.join(BUILD, f + ".o") for f in os.listdir(SRC)
                          if f.endswith((".hip", ".cpp")) and f != "api.cpp")
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", SAN_LIB] + objs + [
        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
