"""Build the gfx950 measurement probes under tests/probes/ (test infrastructure, not libpqkv).

lds_rates: LDS gather / atomic wave-instruction rates; stream_rate: the plain streaming
rate of the decode kernel's code-tile layout.  Run by tests/test_gpu_probes.py.
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
    return outs


if __name__ == "__main__":
    print(build())
