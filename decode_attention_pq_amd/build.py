"""Build libpqkv.so for gfx950 with hipcc (in-tree: decode_attention_pq_amd/libpqkv.so)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "pqkv")
LIB = os.path.join(HERE, "libpqkv.so")
# the decode kernel families come first: they take longest to compile
DECODE_FAMILIES = ["decode_m64d2.hip", "decode_m64d2_lut.hip", "decode_m32d4.hip", "decode_m32d4_lut.hip",
                   "decode_m32d2.hip", "decode_m32d2_lut.hip", "decode_m16d4.hip", "decode_m16d4_lut.hip"]
SOURCES = DECODE_FAMILIES + ["encode.hip", "encode_mfma.hip", "encode_pruned.hip", "decode.hip", "aux_kernels.hip", "append.hip", "kmeans.hip", "noalloc.hip", "fp16_decode.hip",
                            "api.cpp"]

ARCH = "gfx950"
# Packed fp32 VALU forms are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libpqkv.so.  Always recompiles."""
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
