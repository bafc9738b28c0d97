"""Benchmark: PQ decode attention KV tokens/s and % of HBM peak at 32K context, plus pq_encode tokens/s.

Workload (N=1): LLaMA-2-7B-shaped decode layer -- batch 1, 32 heads x 128, d_sub=2,
K=256 centroids, 32768 PQ history tokens + 128 fp16 recent tokens, K/V fp16 N(0,1)
with 4 outlier channels per head scaled x10 and 0.5% point outliers x20 (synthkv).

One step = one pqkv_decode_attention call: ad-LUT build, LUT-sum scoring of the
history, split softmax with the histogram value side, recent-window attention and
the log-sum-exp merge.  Inputs are resident in HBM; the timed loop rotates over
--copies independent copies of the code planes, codebooks, queries and recent
window so the working set (>= 1 GiB) does not sit in the 256 MiB last-level cache.

pq_encode is timed in the same run on the 32768-token history (K and V, all heads).

Prints ONE JSON line.  `--gpus N` with N > 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "PQ decode-attn KV tokens/s & % HBM peak at 32K ctx; pq_encode tokens/s"
HBM_PEAK_GBS = 8000.0
# fp32 vector peak of MI355X (published): 157.3 TFLOP/s = 256 CUs x 2.4 GHz x 256 flops per
# clock per CU, an FMA counting two flops.
FP32_VALU_PEAK_TFLOPS = 157.3
# The same peak in VALU lane-operations (one 32-bit VALU instruction on one lane, an FMA
# counted once): 78.65 T/s.  The encode scan is counted in these units.
VALU_LANE_OPS_PEAK_T = FP32_VALU_PEAK_TFLOPS / 2
# That peak counts packed fp32 instructions (two lane-operations each).  The kernels here are
# built without packed fp32, so the rate they can issue is half of it: a wave64 instruction every
# 4 clocks per SIMD, 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T lane-operations/s.
VALU_UNPACKED_ISSUE_T = VALU_LANE_OPS_PEAK_T / 2
# dense fp32 matrix-core peak of MI355X (published), for the d_sub 4 encode
FP32_MFMA_PEAK_TFLOPS = 157.3


class FenceFreeEvents:
    """hipEvents for timing only, created with hipEventDisableSystemFence.

    Recording a default event (torch.cuda.Event) ends in a system-scope fence that writes back
    and invalidates the caches, which slows the call recorded after it; with an event between
    every pair of calls that cost lands inside every interval.  These events skip the fence.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        import torch
        self._c = ctypes
        # the HIP runtime torch has loaded (dlopen of the same file returns that handle)
        self.hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.ev = [ctypes.c_void_p() for _ in range(n)]
        for e in self.ev:
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, i: int, stream: int):
        rc = self.hip.hipEventRecord(self.ev[i], self._c.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i: int, j: int) -> float:
        f = self._c.c_float()
        rc = self.hip.hipEventElapsedTime(self._c.byref(f), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the first few hundred calls after start run up to 10% slower (clocks, caches); untimed
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama2_7b_32k")
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--encode-reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline leg")
    ap.add_argument("--no-fp16", action="store_true", help="skip the dense fp16 decode baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU work for the baseline sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates the HBM byte counters)")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_pq_amd", "csrc", f) for f in ("decode_kernel.h", "decode_plan.h")]


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode dispatch from the committed rocprofv3 counter runs,
    or None if they were taken on another workload or another kernel source."""
    try:
        with open(os.path.join(ROOT, "profiles", f"pq_decode_kernel__{workload}.counters.json")) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("workload") != workload or c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_dispatch")


def algorithmic_bytes(w, r_len):
    """Bytes the method itself must move for one decode call: 2*M per history token and kv head for the
    codes, fp16 K and V per recent token, fp32 K and V codebooks per kv head, q in and out + lse out."""
    M = w.n_sub
    T = sum(w.hist_len)
    codes = 2 * M * T * w.n_kv_heads                       # K and V codes, 2*M per history token per kv head
    recent = 2 * 2 * w.head_dim * r_len * w.batch * w.n_kv_heads  # fp16 K and V
    books = 2 * w.n_kv_heads * w.n_centroids * w.head_dim * 4      # fp32 K and V codebooks
    q = 2 * w.head_dim * w.batch * w.n_q_heads
    out = (4 * w.head_dim + 4) * w.batch * w.n_q_heads
    return codes + recent + books + q + out


def encode_bytes(w, n_tokens):
    """fp16 K and V read, uint8 codes written, fp32 codebooks read, per encode of n_tokens per tensor."""
    return 2 * (n_tokens * w.n_kv_heads * (2 * w.head_dim + w.n_sub) + w.n_kv_heads * w.n_centroids * w.head_dim * 4)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no multi-GPU leg.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_pq_amd as P
    import synthkv

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    w = synthkv.WORKLOADS[args.workload]
    dev = "cuda"
    B, Hq, Hkv, d, M = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_sub
    T, R = w.max_hist, w.recent_len
    t_cap = w.t_cap
    dims = P.Dims(d, w.d_sub, w.n_centroids, Hq, Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)

    # ---- inputs
    t0 = time.time()
    enc_ms = {}

    def time_encode(x, cb, codes):
        P.encode(dims, x, cb, codes, t_cap)  # warm-up (and the codes used below)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.encode_reps):
            P.encode(dims, x, cb, codes, t_cap)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.encode_reps

    hist_len = torch.tensor(w.hist_len, dtype=torch.int32, device=dev)
    recent_len = torch.full((B,), R, dtype=torch.int32, device=dev)

    # offline codebook training (pqkv_fit_codebooks, timed on the key tensor): the
    # single-layer workloads decode with these fitted codebooks
    fit, fitted = None, {}
    if w.n_layers == 1:
        for tensor in ("k", "v"):
            cal = torch.from_numpy(synthkv.calibration_kv(w, 0, tensor)).to(dev)
            order = torch.from_numpy(synthkv.init_order(w, 0, tensor, cal.shape[0]).astype(np.int32)).to(dev)
            cb_fit = torch.empty((Hkv, w.n_centroids, M, w.d_sub), dtype=torch.float32, device=dev)
            P.fit_codebooks(dims, cal, order, w.kmeans_iters, cb_fit)
            torch.cuda.synchronize()
            if tensor == "k":
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                P.fit_codebooks(dims, cal, order, w.kmeans_iters, cb_fit)
                e1.record()
                torch.cuda.synchronize()
                fit = {"ms_per_tensor": round(e0.elapsed_time(e1), 3), "points": int(cal.shape[0]),
                       "problems": Hkv * M, "centroids": w.n_centroids, "iters": w.kmeans_iters, "arith": "f64"}
            fitted[tensor] = cb_fit
            del cal, order
        print(f"[bench] codebooks fitted ({fit['ms_per_tensor']} ms per tensor)", file=sys.stderr, flush=True)

    copies = []
    gpu_codes = {}  # sequence 0's history codes from the timed encode (the CPU leg compares them)
    if w.n_layers == 1:
        # the history's real codes, encoded with the fitted codebooks from its synthetic
        # values (and timed)
        cbk, cbv = fitted["k"], fitted["v"]
        planes = {}
        for tensor, cb in (("k", cbk), ("v", cbv)):
            x = torch.stack([torch.from_numpy(synthkv.history_kv(w, 0, tensor, b)) for b in range(B)]).to(dev)
            codes = torch.zeros((B, Hkv, t_cap * M), dtype=torch.uint8, device=dev)
            enc_ms[tensor] = time_encode(x, cb, codes)
            planes[tensor] = codes
            gpu_codes[tensor] = codes[0].cpu().numpy()
            del x
        enc_tokens = B * T * 2  # K and V of every history token
        q = torch.from_numpy(synthkv.queries(w)).to(dev)
        rk = torch.from_numpy(synthkv.recent_kv(w, 0, "k")).to(dev)
        rv = torch.from_numpy(synthkv.recent_kv(w, 0, "v")).to(dev)
        # every input of a call is rotated, codebooks included, so no call finds its
        # data in the caches the previous calls filled
        for i in range(args.copies):
            copies.append(dict(q=q.clone(), ck=planes["k"].clone(), cv=planes["v"].clone(), rk=rk.clone(),
                               rv=rv.clone(), cbk=cbk.clone(), cbv=cbv.clone()))
        del planes
        calls_per_step = 1
    else:
        # one decode step of every layer; each layer has its own codebooks, query, recent
        # window and codes.  The codes are uniform random bytes drawn on the device
        # (decode time does not depend on their values; the full history's synthetic
        # values would take hours to draw and encode on the host).  pq_encode is timed
        # on one layer's prefill draw.
        g = torch.Generator(device=dev).manual_seed(w.seed)
        for layer in range(w.n_layers):
            copies.append(dict(
                q=torch.from_numpy(synthkv.queries(w, layer)).to(dev),
                ck=torch.randint(0, w.n_centroids, (B, Hkv, t_cap * M), dtype=torch.uint8, device=dev, generator=g),
                cv=torch.randint(0, w.n_centroids, (B, Hkv, t_cap * M), dtype=torch.uint8, device=dev, generator=g),
                rk=torch.from_numpy(synthkv.recent_kv(w, layer, "k")).to(dev),
                rv=torch.from_numpy(synthkv.recent_kv(w, layer, "v")).to(dev),
                cbk=torch.from_numpy(synthkv.drawn_codebook(w, layer, "k")).to(dev),
                cbv=torch.from_numpy(synthkv.drawn_codebook(w, layer, "v")).to(dev)))
        npre = w.prefill_len
        pre_cap = max(64, -(-npre // 64) * 64)
        for tensor in ("k", "v"):
            x = torch.from_numpy(synthkv.kv_values(w, 0, tensor, "prefill", npre)).to(dev)[None]
            codes = torch.zeros((1, Hkv, pre_cap * M), dtype=torch.uint8, device=dev)
            cb = copies[0]["cbk" if tensor == "k" else "cbv"]
            P.encode(dims, x, cb, codes, pre_cap)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.encode_reps):
                P.encode(dims, x, cb, codes, pre_cap)
            e1.record()
            torch.cuda.synchronize()
            enc_ms[tensor] = e0.elapsed_time(e1) / args.encode_reps
            gpu_codes[tensor] = codes[0].cpu().numpy()
            del x, codes
        enc_tokens = npre * 2
        calls_per_step = w.n_layers
    print(f"[bench] inputs + encode ready in {time.time() - t0:.1f}s; encode K {enc_ms['k']:.3f} ms, "
          f"V {enc_ms['v']:.3f} ms", file=sys.stderr, flush=True)

    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_bytes = P.decode_workspace_bytes(dims, B, T)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    plan = P.decode_plan(dims, B, T)  # the preset the calls run (host only)

    def call(c):
        P.decode_attention(dims, c["q"], c["cbk"], c["cbv"], c["ck"], c["cv"], t_cap, hist_len, T, c["rk"],
                           c["rv"], recent_len, scale, out, lse, ws)

    def step(i):
        if calls_per_step == 1:
            call(copies[i % len(copies)])
        else:
            for c in copies:
                call(c)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(out).all() and torch.isfinite(lse).all(), "non-finite decode output"

    # per-call distribution: a second pass of back-to-back steps with one event between
    # consecutive steps, so each interval is one step and its launch gap (the mean
    # above has no events inside the timed region at all).  The events are timing-only
    # (no system fence on record), so they do not slow the calls they separate.
    nper = max(args.steps, 100)
    evs = FenceFreeEvents(nper + 1)
    sid = torch.cuda.current_stream().cuda_stream
    evs.record(0, sid)
    for i in range(nper):
        step(i)
        evs.record(i + 1, sid)
    torch.cuda.synchronize()
    per_call_us = sorted(evs.elapsed_ms(i, i + 1) * 1e3 / calls_per_step for i in range(nper))
    evs.close()
    pct = lambda p: round(per_call_us[min(len(per_call_us) - 1, int(p * len(per_call_us)))], 3)

    # the dense fp16 baseline (pqkv_fp16_decode_attention) at the same shape: history and recent
    # window as one fp16 cache, rotated over two copies (>= 1 GiB for the 32K and 128K shapes)
    fp16 = None
    if calls_per_step == 1 and not args.no_fp16:
        n_ctx = T + R
        f_cap = -(-n_ctx // 64) * 64
        fk = [torch.randn((B, Hkv, f_cap, d), device=dev, dtype=torch.float16) for _ in range(2)]
        fv = [torch.randn((B, Hkv, f_cap, d), device=dev, dtype=torch.float16) for _ in range(2)]
        flen = torch.full((B,), n_ctx, dtype=torch.int32, device=dev)
        fws = torch.zeros(P.fp16_decode_workspace_bytes(dims, B, n_ctx), dtype=torch.uint8, device=dev)
        fq = copies[0]["q"].to(torch.float16)

        def fcall(i):
            P.fp16_decode_attention(dims, fq, fk[i % 2], fv[i % 2], f_cap, flen, n_ctx, scale, out, lse, fws)

        for i in range(args.warmup):
            fcall(i)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for i in range(args.steps):
            fcall(i)
        f1.record()
        torch.cuda.synchronize()
        f_us = f0.elapsed_time(f1) * 1e3 / args.steps
        f_bytes = 2 * 2 * d * n_ctx * B * Hkv + 2 * d * B * Hq + (4 * d + 4) * B * Hq
        fp16 = {"kernel": "fp16_decode_kernel (pqkv_fp16_decode_attention)", "us_per_call": round(f_us, 3),
                "bytes_per_call": f_bytes, "gbs": round(f_bytes / (f_us * 1e-6) / 1e9, 1),
                "frac": round(f_bytes / (f_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "pq_speedup": round(f_us / (ms * 1e3), 3),
                "page_figure": "about 2x lower time per output token than an FP16 cache at 32K context "
                               "(end to end, whole model; hardware not stated): context only"}
        del fk, fv, fws

    # the product path on given inputs, for the CPU leg's parity check (outside the timed region)
    def gpu_decode_one(q, cb_k, cb_v, planes_k, planes_v, T0, rk0, rv0, R0):
        """One pqkv_decode_attention call of one sequence: numpy in (code planes in the
        cache layout, [1, Hkv, t_cap*M]), numpy out."""
        tc = planes_k.shape[-1] // M
        o = torch.empty((1, Hq, d), dtype=torch.float32, device=dev)
        l = torch.empty((1, Hq), dtype=torch.float32, device=dev)
        w0 = torch.zeros(max(256, P.decode_workspace_bytes(dims, 1, T0)), dtype=torch.uint8, device=dev)
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        P.decode_attention(dims, to(q), to(cb_k), to(cb_v), to(planes_k), to(planes_v), tc,
                           torch.tensor([T0], dtype=torch.int32, device=dev), T0, to(rk0), to(rv0),
                           torch.tensor([R0], dtype=torch.int32, device=dev), scale, o, l, w0)
        torch.cuda.synchronize()
        return o.cpu().numpy(), l.cpu().numpy()

    # the live-cache step: one new row per sequence, with and without a roll into the history
    append_us = None
    if calls_per_step == 1 and R > 1:
        c0 = copies[0]
        r_cap = R
        n_roll = R // 2
        nk = torch.zeros((B, Hkv, d), dtype=c0["rk"].dtype, device=dev)
        lens = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)]  # hist, recent (in / out pairs)
        rk_a, rv_a = c0["rk"].clone(), c0["rv"].clone()
        ck_a, cv_a = c0["ck"].clone(), c0["cv"].clone()

        def append(src, dst):
            P.append_kv(dims, nk, nk, rk_a, rv_a, lens[src], lens[src + 1], lens[dst], lens[dst + 1], n_roll,
                        c0["cbk"], c0["cbv"], ck_a, cv_a, t_cap, T - n_roll)

        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # untimed warm-up: the first launches of the roll and append kernels load their code
        for full in (True, False, False, False):
            lens[0].fill_(T - n_roll)
            lens[1].fill_(r_cap if full else r_cap - 21)
            append(0, 2)
        torch.cuda.synchronize()
        # 20 steps back to back, none of them rolls
        lens[0].fill_(T - n_roll)
        lens[1].fill_(r_cap - 21)
        torch.cuda.synchronize()
        a0.record()
        for i in range(20):
            append(2 * (i % 2), 2 * ((i + 1) % 2))
        a1.record()
        torch.cuda.synchronize()
        no_roll = round(a0.elapsed_time(a1) * 1e3 / 20, 2)
        # single steps that roll (median of 10)
        res = []
        for _ in range(10):
            lens[0].fill_(T - n_roll)
            lens[1].fill_(r_cap)
            torch.cuda.synchronize()
            a0.record()
            append(0, 2)
            a1.record()
            torch.cuda.synchronize()
            res.append(a0.elapsed_time(a1) * 1e3)
        roll = round(sorted(res)[len(res) // 2], 2)
        # the no-roll step is two tiny launches; back to back from Python it mostly measures the
        # host launch path
        append_us = {"no_roll_back_to_back": no_roll, "roll_single": roll, "n_roll": n_roll, "r_cap": r_cap}
        del rk_a, rv_a, ck_a, cv_a

    kv_tokens = w.n_layers * (sum(w.hist_len) + B * R)
    value = kv_tokens / (ms * 1e-3)
    abytes = algorithmic_bytes(w, R)
    call_ms = ms / calls_per_step
    achieved = abytes / (call_ms * 1e-3) / 1e9

    enc_total_ms = enc_ms["k"] + enc_ms["v"]
    enc_tok_s = enc_tokens / (enc_total_ms * 1e-3)
    # brute-force encode work: per (token, head, subspace, centroid) d_sub subtractions and d_sub FMAs
    enc_pairs = enc_tokens * Hkv * M * w.n_centroids  # (subvector, centroid) distance evaluations
    enc_flops = enc_pairs * (2 * w.d_sub)
    enc_tflops = enc_flops / (enc_total_ms * 1e-3) / 1e12
    # VALU instructions per pair.  The direct scan (encode_kernel), from its gfx950 asm: K a
    # multiple of 64: d_sub subtractions and d_sub FMAs, half a min (a three-operand min tree
    # per 16 centroids), a compare and two selects per 16 centroids, and the rescan of the
    # winning 16 centroids (16 distances, compares and selects plus 4 instructions per
    # subvector).  Other K: the distance, a compare and two selects per pair, and loop
    # bookkeeping (about 0.3 at d_sub 2, 0.6 at d_sub 4).  The bounded expanded-form scan
    # (encode_pruned_kernel, d_sub 2, K a multiple of 64): SQ_INSTS_VALU per pair on the 32K
    # workload, 4.01 (its asm: 3.33 in the first pass; the rescans of the candidate
    # sub-blocks, which depend on the data, and the per-subvector work make the rest).
    pruned = w.d_sub == 2 and w.n_centroids % 64 == 0 and w.head_dim in (64, 128)
    if pruned:
        enc_ops_per_pair = 4.01
    elif w.n_centroids % 64 == 0:
        enc_ops_per_pair = 2 * w.d_sub + 0.5 + 3 / 16 + (16 * (2 * w.d_sub + 2) + 4) / w.n_centroids
    else:
        enc_ops_per_pair = 2 * w.d_sub + 3 + (0.3 if w.d_sub == 2 else 0.6)
    enc_tops = enc_pairs * enc_ops_per_pair / (enc_total_ms * 1e-3) / 1e12
    enc_hbm = encode_bytes(w, enc_tokens // 2) / (enc_total_ms * 1e-3) / 1e9
    if w.d_sub == 4 and w.n_centroids == 256:
        # the matrix-core encode (encode_mfma_kernel): the 2 * d_sub flops of a pair are one
        # 16x16x4 fp32 product's share; the exact rescan of the candidates is extra
        encode = {"bound": "mfma", "kernel": "encode_mfma_kernel", "achieved": round(enc_tflops, 2),
                  "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(enc_tflops / FP32_MFMA_PEAK_TFLOPS, 4)}
    else:
        encode = {"bound": "alu", "kernel": "encode_pruned_kernel" if pruned else "encode_kernel",
                  "pairs_per_s": round(enc_pairs / (enc_total_ms * 1e-3), 1), "valu_ops_per_pair": enc_ops_per_pair,
                  "achieved": round(enc_tops, 2), "peak": round(VALU_LANE_OPS_PEAK_T, 2), "unit": "T VALU lane-ops/s",
                  "frac": round(enc_tops / VALU_LANE_OPS_PEAK_T, 4),
                  "unpacked_issue_peak": round(VALU_UNPACKED_ISSUE_T, 2),
                  "frac_of_unpacked_issue": round(enc_tops / VALU_UNPACKED_ISSUE_T, 4),
                  "flop_form_tflops": round(enc_tflops, 2),
                  "fp32_peak_tflops": FP32_VALU_PEAK_TFLOPS}

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "d_sub": w.d_sub, "centroids": w.n_centroids, "hist_tokens": T, "recent_tokens": R,
                   "layers": w.n_layers, "codes": "u8", "kv_dtype": w.dtype,
                   "rotating_copies": args.copies if calls_per_step == 1 else w.n_layers},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name),
                     "kernel": "pq_decode_kernel (one launch per pqkv_decode_attention call)",
                     "algorithmic_bytes_per_call": abytes, "us_per_call": round(call_ms * 1e3, 3),
                     "per_call_us": {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9)},
                     "frac_median": round(abytes / (pct(0.5) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "target_frac": 0.70, "meets_target": bool(achieved / HBM_PEAK_GBS >= 0.70),
                     "plan": {k: plan[k] for k in ("splits", "split_tokens", "build_rounds", "q_heads_per_group",
                                                   "work_groups", "device_plan")}},
        "encode": {"tokens_per_s": round(enc_tok_s, 1), "ms": round(enc_total_ms, 4),
                   "what": "K+V of the history" if calls_per_step == 1 else "K+V of one layer's prefill",
                   "tokens": enc_tokens, **encode, "hbm_gbs": round(enc_hbm, 1),
                   "hbm_frac": round(enc_hbm / HBM_PEAK_GBS, 4)},
    }
    if fit is not None:
        result["fit_codebooks"] = fit
    if fp16 is not None:
        result["fp16_baseline"] = fp16
    if append_us is not None:
        result["append_kv_us"] = append_us
    for c in copies:
        c.clear()
    torch.cuda.synchronize()
    # context for the roofline: what a plain device copy (torch's copy kernel, 1 GiB read and
    # 1 GiB written) reaches on this GPU, as (read + write bytes) / time, median of 5
    if not args.copy_probe:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            dst.copy_(src)
            c1.record()
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        copy_ms = sorted(times)[2]
        result["roofline"]["copy_gbs"] = round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1)
        del src, dst
    if args.copy_probe:  # a plain copy of known size, for the byte-counter calibration
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu:
        print("[bench] CPU oracle leg", file=sys.stderr, flush=True)
        gpu = {"decode": gpu_decode_one, "codes": gpu_codes, "encode_tokens_per_s": enc_tok_s,
               "decode_tokens_per_s": value,
               "codebooks": {t: c.cpu().numpy() for t, c in fitted.items()}}
        result["cpu_baseline"], result["parity"] = cpu_baseline(w, args.cpu_seconds, gpu)
    print(json.dumps(result), flush=True)


def _compare_codes(oracle, x, cb, got, ref, d1, d2):
    """GPU codes `got` against the oracle ([N, H, M]): against its fp32 decision, byte for
    byte everywhere; against its fp64 decision `ref`, byte-equal outside the ambiguity
    band, and inside it the GPU code must itself lie within the band."""
    f32_differ = int(np.sum(got != oracle.encode_f32(x, cb)))
    amb = oracle.ambiguous(d1, d2)
    outside = int(np.sum((got != ref) & ~amb))
    bad_in_band = 0
    if amb.any():
        dist = oracle.code_distance(x, cb, got)
        bad_in_band = int(np.sum(amb & ((dist - d1) >= oracle.AMBIGUITY_REL * np.maximum(1.0, d1))))
    return {"codes": int(ref.size), "differ_from_fp32_decision": f32_differ,
            "mismatch_outside_band": outside, "gpu_code_outside_band": bad_in_band,
            "in_relative_band": int(amb.sum()), "in_absolute_1e-5_band": int(np.sum((d2 - d1) < 1e-5))}


def cpu_baseline(w, target_s, gpu):
    """The CPU oracle on a bounded sample of the same workload, timed on this host's cores,
    and the parity of the GPU path against it on the same inputs.

    Encode leg: the oracle's fp64 brute-force encode of sequence 0's whole history, K and V
    (of a 4096-token slice of layer 0's prefill for the 32-layer workload), with the oracle's
    own codebooks (its fp64 Lloyd fit of the same calibration draw and initial order;
    drawn codebooks for the 32-layer workload).  Its codes are compared with the GPU's
    (`gpu["codes"]`, from the timed encode) and its codebooks with the GPU fit.
    Decode leg: fp64 dequantise-then-exact attention over the first kv heads of sequence 0
    (their query heads, at least one per host thread), scaled to all heads by the head count,
    then the same on one thread.  Parity: one GPU decode of sequence 0 on the oracle's own
    codebooks and codes (`gpu["decode"]`) against the oracle's result for every query head."""
    import oracle
    import synthkv

    d, M, K, Hkv = w.head_dim, w.n_sub, w.n_centroids, w.n_kv_heads
    g = w.n_q_heads // w.n_kv_heads
    R = w.recent_len
    scale = float(np.float32(1.0 / math.sqrt(d)))
    threads = oracle.max_threads()
    parity = {"tol": 2e-3}

    # ---- codebooks and the encode leg
    if w.n_layers == 1:
        T0 = int(w.hist_len[0])
        cbs = {t: oracle.fit_workload_codebooks(w, 0, t, synthkv) for t in ("k", "v")}
        gcb = gpu.get("codebooks") or {}
        parity["codebooks"] = {t: {"floats": int(cbs[t].size),
                                   "differ_from_gpu_fit": int(np.sum(cbs[t].view(np.uint32)
                                                                     != gcb[t].view(np.uint32)))}
                               for t in ("k", "v") if t in gcb}
        xs = {t: synthkv.history_kv(w, 0, t, 0) for t in ("k", "v")}
        positions = np.arange(T0)
        t_cap = w.t_cap
        what = f"sequence 0's {T0}-token history"
    else:
        T0 = int(w.hist_len[0])
        n = min(4096, w.prefill_len)
        cbs = {t: synthkv.drawn_codebook(w, 0, t) for t in ("k", "v")}
        xs = {t: synthkv.kv_values(w, 0, t, "prefill", w.prefill_len, chunks=range(synthkv.n_chunks(n)))[:n]
              for t in ("k", "v")}
        positions = np.arange(n)
        t_cap = max(64, -(-w.prefill_len // 64) * 64)
        what = f"the first {n} tokens of layer 0's prefill"
    t0 = time.time()
    enc = {t: oracle.encode(xs[t], cbs[t]) for t in ("k", "v")}
    enc_s = time.time() - t0
    n_enc = 2 * len(positions)
    off = oracle.code_offsets(M, t_cap)[positions]
    parity["encode"] = {}
    for t in ("k", "v"):
        got = gpu["codes"][t][:, off].transpose(1, 0, 2)  # [N, H, M]
        ref, d1, d2, _ = enc[t]
        parity["encode"][t] = _compare_codes(oracle, xs[t], cbs[t], got, ref, d1, d2)
    encode_leg = {"value": round(n_enc / enc_s, 1), "unit": "encoded tokens/s (K+V, all kv heads)",
                  "cores": threads, "kind": "oracle",
                  "sample": f"fp64 brute-force encode of {what}, K and V ({n_enc} token-tensors, "
                            f"{n_enc * Hkv * M * K:.3g} subvector-centroid pairs); {enc_s:.1f}s"}
    if gpu.get("encode_tokens_per_s"):
        encode_leg["gpu_over_cpu"] = round(gpu["encode_tokens_per_s"] / encode_leg["value"], 1)

    # ---- decode inputs of sequence 0: the oracle's own codes (random codes of the
    # right shape for the 32-layer workload, whose histories are not drawn)
    q = synthkv.queries(w)[:1]
    rk, rv = synthkv.recent_kv(w, 0, "k")[:1], synthkv.recent_kv(w, 0, "v")[:1]
    if w.n_layers == 1:
        ck = enc["k"][0].transpose(1, 0, 2)[None]  # [1, H, T, M]
        cv = enc["v"][0].transpose(1, 0, 2)[None]
    else:
        ck = synthkv.small_codes(7, (1, Hkv, T0, M), K)
        cv = synthkv.small_codes(8, (1, Hkv, T0, M), K)
    ref_out, ref_lse = oracle.decode_exact(q, cbs["k"], cbs["v"], ck, cv, [T0], rk, rv, [R], scale)
    tc = max(64, -(-T0 // 64) * 64)
    got, got_lse = gpu["decode"](q, cbs["k"], cbs["v"], oracle.tile_codes(ck, tc), oracle.tile_codes(cv, tc), T0,
                                 rk, rv, R)
    got, got_lse = got[0].astype(np.float64), got_lse[0].astype(np.float64)
    row = np.max(np.abs(got - ref_out[0]), axis=-1) / np.maximum(np.max(np.abs(ref_out[0]), axis=-1), 1e-6)
    lerr = np.abs(got_lse - ref_lse[0]) / np.maximum(1.0, np.abs(ref_lse[0]))
    parity["decode"] = {"what": f"GPU decode of sequence 0 ({T0}+{R} tokens, all {w.n_q_heads} query heads) on "
                                f"the oracle's codebooks and codes, against the oracle",
                        "max_row_rel_err": float(row.max()), "max_lse_rel_err": float(lerr.max())}
    enc_ok = all(v["differ_from_fp32_decision"] == 0 and v["mismatch_outside_band"] == 0
                 and v["gpu_code_outside_band"] == 0 for v in parity["encode"].values())
    cb_ok = all(v["differ_from_gpu_fit"] == 0 for v in parity.get("codebooks", {}).values())
    parity["ok"] = bool(row.max() <= 2e-3 and lerr.max() <= 2e-3 and enc_ok and cb_ok)

    # ---- decode leg timing: the first kv heads' query heads, one per host thread
    hk = min(Hkv, max(4, -(-threads // g)))
    hq = hk * g
    args = (q[:, :hq], cbs["k"][:hk], cbs["v"][:hk], ck[:, :hk], cv[:, :hk], [T0], rk[:, :hk], rv[:, :hk], [R],
            scale)
    t0, reps = time.time(), 0
    while True:
        oracle.decode_exact(*args)
        reps += 1
        if time.time() - t0 >= target_s:
            break
    el = time.time() - t0
    per_call = el / reps * (w.n_q_heads / hq) * w.batch * w.n_layers
    tokens = w.n_layers * (sum(w.hist_len) + w.batch * R)
    baseline = {"value": round(tokens / per_call, 1), "unit": "KV tokens/s", "cores": min(threads, hq),
                "kind": "oracle",
                "sample": f"{reps} x fp64 dequantise-then-exact attention over {hq} of {w.n_q_heads} query heads "
                          f"of sequence 0 ({T0}+{R} tokens), scaled to every head, sequence and layer of the "
                          f"step; {el:.1f}s"}
    if gpu.get("decode_tokens_per_s"):
        baseline["gpu_over_cpu"] = round(gpu["decode_tokens_per_s"] / baseline["value"], 1)
    oracle.set_threads(1)
    try:
        a1 = (q[:, :g], cbs["k"][:1], cbs["v"][:1], ck[:, :1], cv[:, :1], [T0], rk[:, :1], rv[:, :1], [R], scale)
        t1, reps1 = time.time(), 0
        while True:
            oracle.decode_exact(*a1)
            reps1 += 1
            if time.time() - t1 >= target_s / 3:
                break
        el1 = time.time() - t1
    finally:
        oracle.set_threads(threads)
    per_call1 = el1 / reps1 * (w.n_q_heads / g) * w.batch * w.n_layers
    baseline["one_thread"] = {"value": round(tokens / per_call1, 1), "cores": 1,
                              "sample": f"{reps1} x the same over {g} of {w.n_q_heads} query heads; {el1:.1f}s"}
    baseline["encode"] = encode_leg
    return baseline, parity


if __name__ == "__main__":
    main()
