"""Build libmoe_decode.so for gfx950 in-tree with hipcc.

    python quantized_moe_decode_amd/build.py

Each HIP source is compiled to an object under ``_build/`` (in parallel) and
linked into ``quantized_moe_decode_amd/lib/libmoe_decode.so``.  Packed FP32
instructions are disabled for the device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoe_decode.so")
SOURCES = ["route.hip", "expert_ffn.hip", "tail.hip", "layer.hip", "layer_a4.hip", "layer_a6.hip",
           "layer_a8.hip", "layer_a4p.hip", "layer_a6p.hip", "layer_a8p.hip", "probe.hip", "batch.hip", "grouped.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Host-only sanitizers (the device code is built as usual): AddressSanitizer and
# UndefinedBehaviorSanitizer on the host side of the library (argument
# validation, launch planning), for the CPU tests of the C ABI.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(LIBDIR, "libmoe_decode_hostsan.so")


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + (".san.o" if sanitize else ".o"))
    cmd = [hipcc(), *COMMON, *(SANITIZE_HOST if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build the library (sanitize=True: libmoe_decode_hostsan.so, host code
    under ASan and UBSan; load it with MOE_DECODE_LIB set to its path and
    clang's ASan runtime preloaded)."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC",
           *(["-fsanitize=address,undefined", "-shared-libsan"] if sanitize else []), "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize-host" in sys.argv)
    sys.exit(0)
