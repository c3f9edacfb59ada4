"""Build libgdn.so (gfx950) in-tree with hipcc.

    python -m linear_attention_recurrence_chunked_amd.build

Compiles every source under ``csrc/`` for gfx950 only and links the shared library next to
this file.  It always rebuilds; the objects go to ``_build/`` (not tracked).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
COMMON = ["-O3", "-fPIC", "-std=c++17", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(PKG), "include")]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the device code is compiled as
# usual); the library then needs the clang sanitizer runtime preloaded in its process.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
LIB_SAN = os.path.join(PKG, "libgdn_san.so")
OUT_DIR_SAN = os.path.join(PKG, "_build_san")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(OUT_DIR_SAN if sanitize else OUT_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + (SANITIZE if sanitize else []) + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libgdn.so, or with sanitize libgdn_san.so (host code instrumented; for CPU tests
    of the host side, loaded when GDN_LIB names it)."""
    lib = LIB_SAN if sanitize else LIB
    os.makedirs(OUT_DIR_SAN if sanitize else OUT_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(8, len(srcs)))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, sanitize), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    san = (["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-shared-libsan"] if sanitize else [])
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + san + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
