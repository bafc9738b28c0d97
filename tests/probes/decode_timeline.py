"""Per-phase and per-step timeline of one decode call (test infrastructure).

Runs libpqkv_timeline.so -- libpqkv with the 64-subspace (d_sub 2) and the 32-subspace
(d_sub 4) decode kernels built with PQKV_TIMELINE -- through the Python binding.  Shapes
(--shape):
  32k     batch 1, 32 query and kv heads of 128, d_sub 2, 256 centroids, 32768 history and
          128 recent tokens (the 32K-context workload);
  gqa     batch 1, 32 query heads over 8 kv heads, d_sub 4, 131072 history and 256 recent;
  ragged  batch 4 with histories of 14698, 3634, 31436 and 30564 tokens and 128 recent each,
          32 heads, d_sub 2 (one layer of the 32-layer ragged workload).
Codes, q, recent rows and codebooks are random (decode time does not depend on code values).
The script runs 200 uninstrumented calls, then 50 with the stamps on, and reads the stamps of
the last one.  Lane 0 of every wave stamped s_memrealtime (100 MHz) at each phase boundary
and when each step's code tile was in its registers.  It prints, per boundary, the median and
the maximum over work-groups for waves 0-3 and 4-7 (one table per wave of work-groups when
the grid is larger than the 256 CUs), in us from the earliest entry; the per-step medians of
the first wave of work-groups; and the XCC_ID of every work-group against work-group id mod
8, the order the XCD-aware work mapping assumes.

Usage: python tests/probes/decode_timeline.py [--shape 32k|gqa|ragged]   (exit status 0 on success)
"""
from __future__ import annotations

import argparse
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
SLOTS = 48  # stamps per wave
SHAPES = {
    # name: (batch, Hq, Hkv, head_dim, d_sub, history lengths, recent, setter)
    "32k": (1, 32, 32, 128, 2, [32768], 128, "pqkv_timeline_set_m64d2"),
    "gqa": (1, 32, 8, 128, 4, [131072], 256, "pqkv_timeline_set_m32d4"),
    "ragged": (4, 32, 32, 128, 2, [14698, 3634, 31436, 30564], 128, "pqkv_timeline_set_m64d2"),
}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--shape", choices=sorted(SHAPES), default="32k")
    args = ap.parse_args()
    B, Hq, Hkv, d, dsub, hist, R, setter = SHAPES[args.shape]
    lib_path = os.path.join(HERE, "libpqkv_timeline.so")
    if not os.path.exists(lib_path):
        print("libpqkv_timeline.so not built (tests/probes/build_probes.py)")
        return 2
    P.LIB_PATH = lib_path  # the instrumented build, before the binding loads anything
    P._lib = None
    L = P.lib()
    set_tl = getattr(L, setter)
    set_tl.argtypes = [ctypes.c_void_p]
    set_tl.restype = ctypes.c_int

    dev = "cuda"
    K = 256
    M = d // dsub
    T = max(hist)
    t_cap = -(-T // 64) * 64
    dims = P.Dims(d, dsub, K, Hq, Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    g = torch.Generator(device=dev).manual_seed(11)
    copies = []
    for _ in range(8):  # rotated inputs, so no call finds its data in the caches
        copies.append(dict(
            q=torch.randn((B, Hq, d), device=dev, generator=g).half(),
            ck=torch.randint(0, K, (B, Hkv, t_cap * M), dtype=torch.uint8, device=dev, generator=g),
            cv=torch.randint(0, K, (B, Hkv, t_cap * M), dtype=torch.uint8, device=dev, generator=g),
            rk=torch.randn((B, Hkv, R, d), device=dev, generator=g).half(),
            rv=torch.randn((B, Hkv, R, d), device=dev, generator=g).half(),
            cbk=torch.randn((Hkv, K, M, dsub), device=dev, generator=g),
            cbv=torch.randn((Hkv, K, M, dsub), device=dev, generator=g)))
    hl = torch.tensor(hist, dtype=torch.int32, device=dev)
    rl = torch.full((B,), R, dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), device=dev)
    lse = torch.empty((B, Hq), device=dev)
    ws = torch.zeros(P.decode_workspace_bytes(dims, B, T), dtype=torch.uint8, device=dev)
    max_wg = 4096
    buf = torch.zeros(max_wg * 8 * SLOTS, dtype=torch.int64, device=dev)

    def call(i):
        c = copies[i % 8]
        P.decode_attention(dims, c["q"], c["cbk"], c["cbv"], c["ck"], c["cv"], t_cap, hl, T, c["rk"], c["rv"],
                           rl, scale, out, lse, ws)

    for i in range(200):
        call(i)
    torch.cuda.synchronize()
    if set_tl(ctypes.c_void_p(buf.data_ptr())) != 0:
        print("setting the timeline buffer failed")
        return 1
    for i in range(50):
        call(i)
    torch.cuda.synchronize()
    set_tl(None)
    torch.cuda.synchronize()
    a = buf.cpu().numpy().reshape(max_wg, 8, SLOTS)
    n = int((a[:, :, 0] > 0).any(axis=1).sum())
    a = a[:n]
    if n == 0 or not (a[:, :, 0] > 0).all():
        print(f"stamps missing: {n} work-groups")
        return 1
    # a boundary or step a wave did not reach in the last call (the merge, in the
    # work-groups that did not merge; a step past its history) holds an older stamp
    fresh = a >= a[:, :, :1]
    t0 = a[:, :, 0].min()
    us = (a - t0) * 0.01
    print(f"decode timeline, shape {args.shape}: {n} work-groups of 8 waves; us from the earliest entry "
          "(s_memrealtime, 100 MHz), the last of 50 back-to-back calls")
    # work-groups that entered after the first ones finished form a later wave: split the
    # entries at their widest gap when it exceeds 5 us
    ent = np.sort(us[:, 0, 0])
    gaps = np.diff(ent)
    first = np.ones(n, bool)
    if gaps.size and gaps.max() > 5.0:
        cut = ent[int(np.argmax(gaps))] + 0.5 * gaps.max()
        first = us[:, 0, 0] < cut
    groups = [("", np.ones(n, bool))] if first.all() else [("first wave of work-groups, ", first),
                                                           ("second wave, ", ~first)]
    for tag, sel in groups:
        print(f"  {tag}{int(sel.sum())} work-groups")
        print(f"  {'boundary':26s} {'waves 0-3 median':>17s} {'max':>7s} {'waves 4-7 median':>17s} {'max':>7s}")
        for k in ORDER:
            ok = fresh[sel][:, :, k]
            if not ok.any():
                continue
            u = us[sel][:, :, k]
            lo, hi = u[:, :4][ok[:, :4]], u[:, 4:][ok[:, 4:]]
            if lo.size == 0 or hi.size == 0:
                continue
            print(f"  {NAMES[k]:26s} {np.median(lo):17.2f} {lo.max():7.2f} {np.median(hi):17.2f} {hi.max():7.2f}")
    sel = groups[0][1]
    print("  per step, first wave of work-groups: the step's code tile in registers (median us, waves 0-3 / 4-7)")
    for st in range(SLOTS - 16):
        ok = fresh[sel][:, :, 16 + st]
        if not ok.any():
            continue
        u = us[sel][:, :, 16 + st]
        lo, hi = u[:, :4][ok[:, :4]], u[:, 4:][ok[:, 4:]]
        if lo.size == 0 or hi.size == 0:
            continue
        print(f"  step {st:2d}  {np.median(lo):7.2f} / {np.median(hi):7.2f}")
    merged = fresh[:, :, 11]
    print(f"  work-groups that merged: {int(merged.any(axis=1).sum())}; "
          f"last merge done at {us[:, :, 11][merged].max():.2f} us")
    xcc = a[:, 0, 14] & 0xF
    match = int((xcc == np.arange(n) % 8).sum())
    print(f"  XCC_ID == work-group id mod 8: {match} of {n}")
    # every wave's boundaries come in program order (every work-group reaches these)
    seq = [0, 3, 4, 5, 6, 7, 8]
    v = a[:, :, seq]
    if not (fresh[:, :, seq].all() and (np.diff(v, axis=2) >= 0).all()):
        print("stamps out of order")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
