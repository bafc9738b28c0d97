"""Build the gfx950 measurement probes under tests/probes/ (test infrastructure, not libpqkv).

lds_rates: LDS gather / atomic wave-instruction rates; stream_rate: the plain streaming
rate of the decode kernel's code-tile layout; libpqkv_timeline.so: libpqkv with the
64-subspace and the 32-subspace d_sub 4 decode kernels built with PQKV_TIMELINE (per-wave phase
and per-step stamps), linked from libpqkv's own objects (build libpqkv first).  Run by tests/test_gpu_probes.py.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROBES = ["lds_rates", "stream_rate"]


def build() -> list[str]:
    sys.path.insert(0, ROOT)
    from decode_attention_pq_amd import build as hipbuild

    outs = []
    for name in PROBES:
        exe = os.path.join(HERE, name)
        cmd = [hipbuild.hipcc(), "-O3", "-std=c++17", "-Wall", f"--offload-arch={hipbuild.ARCH}",
               *hipbuild.DEVICE_FLAGS, os.path.join(HERE, name + ".hip"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {name}:\n{r.stdout}\n{r.stderr}")
        outs.append(exe)
    outs.append(build_timeline_lib())
    return outs


def build_timeline_lib() -> str:
    """libpqkv_timeline.so: the 64-subspace (d_sub 2) and 32-subspace (d_sub 4) decode families
    recompiled with PQKV_TIMELINE, the rest of libpqkv's objects as built."""
    sys.path.insert(0, ROOT)
    from decode_attention_pq_amd import build as hipbuild

    obj_dir = os.path.join(ROOT, "_build", "probes")
    os.makedirs(obj_dir, exist_ok=True)
    stamped = ["decode_m64d2.hip", "decode_m32d4.hip"]
    tobjs = []
    for src in stamped:
        tobj = os.path.join(obj_dir, os.path.splitext(src)[0] + "_timeline.o")
        cmd = [hipbuild.hipcc(), *hipbuild.COMMON, *hipbuild.DEVICE_FLAGS, "-DPQKV_TIMELINE", "-c",
               os.path.join(hipbuild.CSRC, src), "-o", tobj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on the timeline build of {src}:\n{r.stdout}\n{r.stderr}")
        tobjs.append(tobj)
    objs = tobjs + [os.path.join(hipbuild.OBJ, os.path.splitext(s)[0] + ".o")
                    for s in hipbuild.SOURCES if s not in stamped]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"libpqkv objects missing (build libpqkv first): {missing[:3]}")
    lib = os.path.join(HERE, "libpqkv_timeline.so")
    r = subprocess.run([hipbuild.hipcc(), f"--offload-arch={hipbuild.ARCH}", "-shared", "-fPIC", "-o", lib, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed on the timeline library:\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build())
