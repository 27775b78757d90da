"""Builds libpagedattn.so (gfx950) in-tree with hipcc.

    python -m paged_kv_cache_248_amd.build            # build the library
    python -m paged_kv_cache_248_amd.build --clean    # remove objects and the library
    python -m paged_kv_cache_248_amd.build --sanitize # host ASan + UBSan build

The sanitized build (libpagedattn_san.so, objects in _build_san/) puts
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only — the
argument validation, launch set-up and the block manager; device code is
built as usual.  It is for CPU runs of the host-side tests:

    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 PA_LIBRARY=paged_kv_cache_248_amd/libpagedattn_san.so \
    python -m pytest tests/test_abi.py tests/test_block_manager.py -m "not gpu"
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")
SOURCES = ["abi.hip", "append.hip", "block_manager.cpp", "copy_blocks.hip", "decode.hip",
           "prefill.hip", "prefill_halftile.hip", "stream_read.hip", "unfused.hip"]
# the unfused prefill baseline calls hipBLASLt for its two matrix products
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
SAN_OBJ = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "libpagedattn_san.so")
# each sanitizer flag applies to the host pass only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: plain fp32 instructions only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OBJ if sanitize else OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *(SAN_FLAGS if sanitize else []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source (HIP kernels, host C++) and link the shared
    library; returns its path.  sanitize: the host-sanitized variant."""
    out = SAN_LIB if sanitize else LIB
    os.makedirs(SAN_OBJ if sanitize else OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = out + ".tmp"
    san_link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *san_link, *objs, *LIBS, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def clean() -> None:
    for d in (OBJ, SAN_OBJ):
        shutil.rmtree(d, ignore_errors=True)
    for f in (LIB, SAN_LIB):
        if os.path.exists(f):
            os.remove(f)


if __name__ == "__main__":
    if "--clean" in sys.argv:
        clean()
    else:
        build(verbose=True, sanitize="--sanitize" in sys.argv)
