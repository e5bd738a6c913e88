"""Build libw12.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m lossless_bit_weight_encode_amd.build              # libw12.so
    python -m lossless_bit_weight_encode_amd.build --timeline   # libw12_timeline.so

The second is a measurement build: the same sources with W12_TIMELINE defined, so the
streaming GEMM also stamps a per-work-group timeline (include/w12_timeline.h).

Every HIP/C++ source under csrc/ is compiled for gfx950 and linked into
lossless_bit_weight_encode_amd/libw12.so.  Packed FP32 instructions are disabled for all
device code (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw12.so")
TIMELINE_LIB = os.path.join(PKG, "libw12_timeline.so")
ARCH = os.environ.get("W12_OFFLOAD_ARCH", "gfx950")

SOURCES = ["w12_encode.hip", "w12_decode.hip", "w12_gemm.hip", "w12_gemm_wide.hip", "w12_probe.hip", "w12_noalloc.hip", "w12_api.cpp", "w12_file.cpp"]

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found")
    return h


def _compile(src: str, build_dir: str = BUILD, defines: tuple = ()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *COMMON, *defines, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, timeline: bool = False) -> str:
    build_dir = BUILD + ("_timeline" if timeline else "")
    lib = TIMELINE_LIB if timeline else LIB
    defines = ("-DW12_TIMELINE",) if timeline else ()
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    try:
        build(timeline="--timeline" in sys.argv[1:])
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
