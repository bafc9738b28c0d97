"""Per-phase timeline of one decode call at the 32K shape (test infrastructure).

Runs libpqkv_timeline.so -- libpqkv with the 64-subspace decode kernels built with
PQKV_TIMELINE -- through the Python binding.  The shape is batch 1, 32 query and kv
heads of 128, d_sub 2, 256 centroids, 32768 history and 128 recent tokens, with
random codes, q, recent rows and codebooks (decode time does not depend on code
values).  It runs 200 uninstrumented calls, then 50 with the stamps on, and reads the
stamps of the last one.  Lane 0 of every wave stamped s_memrealtime (100 MHz) at each
phase boundary.  The script prints, per boundary, the median and the maximum over
work-groups, for waves 0-3 and 4-7, in us from the earliest entry.  It also prints the
XCC_ID of every work-group against work-group id mod 8, the order the XCD-aware work
mapping assumes.

Usage: python tests/probes/decode_timeline.py   (exit status 0 on success)
"""
from __future__ import annotations

import ctypes
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import decode_attention_pq_amd as P  # noqa: E402

NAMES = ["entry", "codebook requests issued", "LUT part built", "phase 1 starts", "phase 1 ends",
         "maxima met", "phase 2 ends", "histogram complete", "epilogue done", "partial published",
         "counter returned", "merge done", "half of phase 1", "half of phase 2"]
ORDER = [0, 1, 2, 3, 12, 4, 5, 13, 6, 7, 8, 9, 10, 11]


def main() -> int:
    lib_path = os.path.join(HERE, "libpqkv_timeline.so")
    if not os.path.exists(lib_path):
        print("libpqkv_timeline.so not built (tests/probes/build_probes.py)")
        return 2
    P.LIB_PATH = lib_path  # the instrumented build, before the binding loads anything
    P._lib = None
    L = P.lib()
    L.pqkv_timeline_set.argtypes = [ctypes.c_void_p]
    L.pqkv_timeline_set.restype = ctypes.c_int

    dev = "cuda"
    B, H, d, dsub, K, T, R = 1, 32, 128, 2, 256, 32768, 128
    M = d // dsub
    t_cap = T
    dims = P.Dims(d, dsub, K, H, H)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    g = torch.Generator(device=dev).manual_seed(11)
    copies = []
    for _ in range(8):  # rotated inputs, so no call finds its data in the caches
        copies.append(dict(
            q=torch.randn((B, H, d), device=dev, generator=g).half(),
            ck=torch.randint(0, K, (B, H, t_cap * M), dtype=torch.uint8, device=dev, generator=g),
            cv=torch.randint(0, K, (B, H, t_cap * M), dtype=torch.uint8, device=dev, generator=g),
            rk=torch.randn((B, H, R, d), device=dev, generator=g).half(),
            rv=torch.randn((B, H, R, d), device=dev, generator=g).half(),
            cbk=torch.randn((H, K, M, dsub), device=dev, generator=g),
            cbv=torch.randn((H, K, M, dsub), device=dev, generator=g)))
    hl = torch.full((B,), T, dtype=torch.int32, device=dev)
    rl = torch.full((B,), R, dtype=torch.int32, device=dev)
    out = torch.empty((B, H, d), device=dev)
    lse = torch.empty((B, H), device=dev)
    ws = torch.zeros(P.decode_workspace_bytes(dims, B, T), dtype=torch.uint8, device=dev)
    max_wg = 4096
    buf = torch.zeros(max_wg * 8 * 16, dtype=torch.int64, device=dev)

    def call(i):
        c = copies[i % 8]
        P.decode_attention(dims, c["q"], c["cbk"], c["cbv"], c["ck"], c["cv"], t_cap, hl, T, c["rk"], c["rv"],
                           rl, scale, out, lse, ws)

    for i in range(200):
        call(i)
    torch.cuda.synchronize()
    if L.pqkv_timeline_set(ctypes.c_void_p(buf.data_ptr())) != 0:
        print("pqkv_timeline_set failed")
        return 1
    for i in range(50):
        call(i)
    torch.cuda.synchronize()
    L.pqkv_timeline_set(None)
    torch.cuda.synchronize()
    a = buf.cpu().numpy().reshape(max_wg, 8, 16)
    n = int((a[:, :, 0] > 0).any(axis=1).sum())
    a = a[:n]
    if n == 0 or not (a[:, :, 0] > 0).all():
        print(f"stamps missing: {n} work-groups")
        return 1
    # a boundary a wave did not reach in the last call (the merge, in the work-groups that
    # did not merge) holds a stamp of an earlier call: older than the wave's entry
    fresh = a[:, :, :14] >= a[:, :, :1]
    t0 = a[:, :, 0].min()
    us = (a[:, :, :14] - t0) * 0.01
    print(f"decode timeline, 32K shape: {n} work-groups of 8 waves; us from the earliest entry "
          "(s_memrealtime, 100 MHz), the last of 50 back-to-back calls")
    print(f"  {'boundary':26s} {'waves 0-3 median':>17s} {'max':>7s} {'waves 4-7 median':>17s} {'max':>7s}")
    med = {}
    for k in ORDER:
        ok = fresh[:, :, k]
        if not ok.any():
            continue
        lo, hi = us[:, :4, k][ok[:, :4]], us[:, 4:, k][ok[:, 4:]]
        med[k] = float(np.median(np.concatenate([lo, hi])))
        print(f"  {NAMES[k]:26s} {np.median(lo):17.2f} {lo.max():7.2f} {np.median(hi):17.2f} {hi.max():7.2f}")
    merged = fresh[:, :, 11]
    print(f"  work-groups that merged: {int(merged.any(axis=1).sum())}; "
          f"last merge done at {us[:, :, 11][merged].max():.2f} us")
    xcc = a[:, 0, 14] & 0xF
    match = int((xcc == np.arange(n) % 8).sum())
    print(f"  XCC_ID == work-group id mod 8: {match} of {n}")
    # every wave's boundaries come in program order
    seq = [0, 3, 4, 5, 6, 7, 8, 9]
    v = a[:, :, seq]
    if not (fresh[:, :, seq].all() and (np.diff(v, axis=2) >= 0).all()):
        print("stamps out of order")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
