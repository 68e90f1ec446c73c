"""Build libpagedkv.so (HIP for gfx950) in-tree.

    python -m paged_kv_cache_61_amd.build             # or: python paged_kv_cache_61_amd/build.py
    python -m paged_kv_cache_61_amd.build --sanitize  # lib/libpagedkv_san.so

Every source under csrc/ is compiled by hipcc for gfx950 only, with packed
FP32 instructions disabled, and linked into paged_kv_cache_61_amd/lib/.

``--sanitize`` builds a second library whose host code (argument checks, the
host metadata validator, the block manager) is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer; device code is built as
usual.  It links the shared ASan runtime, so a process that loads it needs
that runtime preloaded (``asan_runtime()``), and the binding loads it when
``PAGED_KV_LIBRARY`` names it.  It is meant for CPU-side test runs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
OBJDIR = os.path.join(os.path.dirname(HERE), "_build", "pagedkv")
LIB = os.path.join(LIBDIR, "libpagedkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wshadow", "-Wno-unused-function", "-Wno-unused-variable",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


LIB_SAN = os.path.join(LIBDIR, "libpagedkv_san.so")
# host-side instrumentation only: each sanitizer flag goes to the host pass
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """Path of the shared ASan runtime of hipcc's clang (to preload)."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("shared ASan runtime not found")
    return path


def _compile(src: str, sanitize: bool = False) -> str:
    objdir = OBJDIR + ("_san" if sanitize else "")
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(OBJDIR + ("_san" if sanitize else ""), exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp"
    link_san = ["-fsanitize=address,undefined", "-shared-libasan"] if sanitize else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_san, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
