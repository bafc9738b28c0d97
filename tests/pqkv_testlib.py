"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, prepare oracle-side inputs, and apply the comparison rules.

Comparison rules (the tolerances the tests assert):
  * codes: byte-equal wherever the oracle's runner-up distance is more than
    1e-5 * max(1, best) away from the best; inside that band the GPU code must
    itself be within the band of the best distance (both are correct answers).
  * attention output: per (sequence, query head) row,
        max_e |out - ref| / max(max_e |ref|, 1e-6) <= 2e-3;
  * lse: |lse - ref| <= 2e-3 * max(1, |ref|), -inf matching -inf exactly;
  * LUT: |lut - ref| <= 1e-6 * sum_j |q_j C_j| + 1e-30 per entry.
The 2e-3 bound is the accuracy target of fp16 inputs with fp32 accumulation.
"""
from __future__ import annotations

import math

import numpy as np

import oracle

OUT_RTOL = 2e-3
LSE_RTOL = 2e-3


def to_dev(a, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def dims_for(head_dim, d_sub, K, Hq, Hkv):
    import decode_attention_pq_amd as P

    return P.Dims(head_dim, d_sub, K, Hq, Hkv)


def run_gpu_decode(dims, q, cb_k, cb_v, planes_k, planes_v, t_cap, hist_len, recent_k, recent_v, recent_len,
                   scale, max_hist=None, out_fill=np.nan, lut="none", workspace=None):
    """Everything numpy in, numpy out; planes_* already in the cache layout.

    lut: "none" (the kernel builds the ad-LUT), "gpu" (pqkv_build_lut's table from q and
    cb_k is passed in, and cb_k is not), or a numpy table [B, Hq, M, K] to pass in.
    workspace: a device tensor to use (and keep), else a fresh zeroed one."""
    import torch

    import decode_attention_pq_amd as P

    B, Hq, d = q.shape
    max_hist = int(max(hist_len)) if max_hist is None else int(max_hist)
    qd = to_dev(q)
    cbk, cbv = to_dev(cb_k), to_dev(cb_v)
    ck, cv = to_dev(planes_k), to_dev(planes_v)
    hl = to_dev(np.asarray(hist_len, np.int32))
    if recent_k is not None and recent_k.shape[2] > 0:
        rk, rv = to_dev(recent_k), to_dev(recent_v)
        rl = to_dev(np.asarray(recent_len, np.int32))
    else:
        rk = rv = rl = None
    table = None
    if isinstance(lut, str) and lut == "gpu":
        table = torch.full((B, Hq, dims.head_dim // dims.d_sub, dims.n_centroids), np.nan, dtype=torch.float32,
                           device="cuda")
        P.build_lut(dims, qd, cbk, table)
        cbk = None
    elif not isinstance(lut, str):
        table = to_dev(np.asarray(lut, np.float32))
        cbk = None
    out = torch.full((B, Hq, d), out_fill, dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), out_fill, dtype=torch.float32, device="cuda")
    if workspace is None:
        nbytes = P.decode_workspace_bytes(dims, B, max_hist)
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    P.decode_attention(dims, qd, cbk, cbv, ck, cv, t_cap, hl, max_hist, rk, rv, rl, scale, out, lse, workspace,
                       lut=table)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def run_gpu_encode(dims, x, codebook, n_seqs_planes, t_cap, t_start=0, init_codes=None):
    """x: [n_seqs, N, H, d] numpy; returns the code planes [n_seqs, H, t_cap*M] numpy."""
    import torch

    import decode_attention_pq_amd as P

    xd = to_dev(x)
    cbd = to_dev(codebook)
    M = dims.head_dim // dims.d_sub
    if init_codes is None:
        codes = torch.zeros((n_seqs_planes, dims.n_kv_heads, t_cap * M), dtype=torch.uint8, device="cuda")
    else:
        codes = to_dev(init_codes)
    P.encode(dims, xd, cbd, codes, t_cap, t_start)
    torch.cuda.synchronize()
    return codes.cpu().numpy()


def check_codes(gpu_codes, x, codebook, ref_codes, d1, d2):
    """gpu_codes/ref_codes logical [N, H, M]; returns (n_ambiguous, n_total).

    Every code must be the oracle's fp32 decision (encode_f32), byte for byte, near
    ties included.  Against the fp64 decision (ref_codes, best and runner-up distances
    d1, d2): equal outside the 1e-5 band, and inside it the GPU code's fp64 distance
    within the band of the best."""
    c32 = oracle.encode_f32(x, codebook)
    diff = gpu_codes != c32
    if diff.any():
        idx = np.argwhere(diff)[:5]
        raise AssertionError(f"{int(diff.sum())} codes differ from the fp32 decision, first at {idx.tolist()}")
    amb = oracle.ambiguous(d1, d2)
    ok = ~amb
    mism = (gpu_codes != ref_codes) & ok
    if mism.any():
        idx = np.argwhere(mism)[:5]
        raise AssertionError(f"{int(mism.sum())} code mismatches outside the band, first at {idx.tolist()}")
    if amb.any():
        dist = oracle.code_distance(x, codebook, gpu_codes)
        band = oracle.AMBIGUITY_REL * np.maximum(1.0, d1)
        bad = amb & ((dist - d1) >= band)
        assert not bad.any(), f"{int(bad.sum())} ambiguous codes outside the band"
    return int(amb.sum()), int(amb.size)


def check_attention(out, lse, ref_out, ref_lse, rtol=OUT_RTOL, lse_rtol=LSE_RTOL):
    """Returns (max row-relative out error, max lse error) after asserting them."""
    out = np.asarray(out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    assert np.all(np.isfinite(out)), "non-finite output"
    den = np.maximum(np.abs(ref_out).max(axis=-1), 1e-6)
    err = np.abs(out - ref_out).max(axis=-1) / den
    worst = float(err.max()) if err.size else 0.0
    assert worst <= rtol, f"max row-relative output error {worst:.3e} > {rtol}"
    lse = np.asarray(lse, np.float64)
    ref_lse = np.asarray(ref_lse, np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse)), "-inf lse mismatch"
    fin = ~both_inf
    lerr = np.abs(lse[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
    lworst = float(lerr.max()) if lerr.size else 0.0
    assert lworst <= lse_rtol, f"max lse error {lworst:.3e} > {lse_rtol}"
    return worst, lworst


def softmax_scale(head_dim):
    """The softmax scale as both sides see it: 1/sqrt(d) rounded to fp32."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))
