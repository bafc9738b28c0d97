"""GPU parity of pqkv_append_kv (the live cache: recent-window roll-over into the
PQ history) against the oracle's step function over many decode steps.

Each case starts from a ragged state (some windows empty, some full, some
histories empty), runs tens of steps with seeded new rows, and then compares
the lengths (exact), the recent rows (bit-exact), the history codes (the encode
rule: exact outside the ambiguity band, the starting codes untouched, bytes past
the history never written) and finally decode attention over the resulting
cache against the dequantise-then-exact oracle.
"""
import math

import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, check_codes, dims_for, run_gpu_decode, softmax_scale, to_dev

pytestmark = pytest.mark.gpu

FILL = 0xAB  # code bytes the test never expects the kernel to write

CASES = [
    # d, d_sub, K, Hq, Hkv, dtype, r_cap, n_roll, steps, start history, start recent
    (128, 2, 256, 8, 4, np.float16, 48, 32, 90, (0, 70, 130), (0, 20, 48)),
    (64, 4, 16, 2, 2, np.float32, 16, 16, 40, (5, 0), (16, 3)),
    (128, 4, 200, 4, 1, np.float16, 8, 1, 30, (64,), (8,)),
    (64, 2, 256, 4, 2, np.float16, 1024, 512, 3, (10, 0), (1023, 1024)),
]


def _codebook(seed, H, K, M, dsub):
    return (synthkv.small_normal(seed, (H, K, M, dsub)) * 2.0).astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c[0]}s{c[1]}K{c[2]}r{c[6]}n{c[7]}")
def test_append_steps_match_oracle(case):
    import torch

    import decode_attention_pq_amd as P

    d, dsub, K, Hq, Hkv, dt, r_cap, n_roll, steps, T0, R0 = case
    B, M = len(T0), d // dsub
    dims = dims_for(d, dsub, K, Hq, Hkv)
    t_cap = 64 * math.ceil((max(T0) + steps + r_cap + 64) / 64)
    seed = 500 + d + K + r_cap
    cbk, cbv = _codebook(seed, Hkv, K, M, dsub), _codebook(seed + 1, Hkv, K, M, dsub)
    start_codes = {t: [synthkv.small_codes(seed + 2 + 2 * b + (t == "v"), (T0[b], Hkv, M), K) for b in range(B)]
                   for t in "kv"}
    start_rec = {t: [synthkv.small_normal(seed + 10 + 2 * b + (t == "v"), (R0[b], Hkv, d)).astype(dt)
                     for b in range(B)] for t in "kv"}
    new = {t: synthkv.small_normal(seed + 20 + (t == "v"), (steps, B, Hkv, d)).astype(dt) for t in "kv"}

    # device state: code planes pre-filled with FILL past each start history
    planes, recent = {}, {}
    for t in "kv":
        pl = np.full((B, Hkv, t_cap * M), FILL, np.uint8)
        off = oracle.code_offsets(M, t_cap)
        for b in range(B):
            for h in range(Hkv):
                pl[b, h, off[:T0[b]].reshape(-1)] = start_codes[t][b][:, h, :].reshape(-1)
        planes[t] = to_dev(pl)
        rb = np.zeros((B, Hkv, r_cap, d), dt)
        for b in range(B):
            rb[b, :, :R0[b]] = start_rec[t][b].transpose(1, 0, 2)
        recent[t] = to_dev(rb)
    lens = [[to_dev(np.asarray(T0, np.int32)), to_dev(np.asarray(R0, np.int32))],
            [torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda")]]
    cbk_d, cbv_d = to_dev(cbk), to_dev(cbv)
    max_hist = max(T0)
    for s in range(steps):
        src, dst = lens[s % 2], lens[(s + 1) % 2]
        P.append_kv(dims, to_dev(new["k"][s]), to_dev(new["v"][s]), recent["k"], recent["v"], src[0], src[1],
                    dst[0], dst[1], n_roll, cbk_d, cbv_d, planes["k"], planes["v"], t_cap, max_hist)
        max_hist += n_roll  # a bound on the history after this step
        max_hist = min(max_hist, t_cap - n_roll)
    torch.cuda.synchronize()
    T_gpu = lens[steps % 2][0].cpu().numpy()
    R_gpu = lens[steps % 2][1].cpu().numpy()

    # oracle
    state = {"codes_k": start_codes["k"], "codes_v": start_codes["v"],
             "amb_k": [np.zeros(c.shape, bool) for c in start_codes["k"]],
             "amb_v": [np.zeros(c.shape, bool) for c in start_codes["v"]],
             "recent_k": start_rec["k"], "recent_v": start_rec["v"]}
    for s in range(steps):
        state = oracle.append_kv_step(state, new["k"][s], new["v"][s], cbk, cbv, r_cap, n_roll)
    T_ref = np.array([c.shape[0] for c in state["codes_k"]])
    R_ref = np.array([r.shape[0] for r in state["recent_k"]])
    np.testing.assert_array_equal(T_gpu, T_ref)
    np.testing.assert_array_equal(R_gpu, R_ref)

    off = oracle.code_offsets(M, t_cap)
    gpu_codes = {}
    for t, cb in (("k", cbk), ("v", cbv)):
        pl = planes[t].cpu().numpy()
        rec = recent[t].cpu().numpy()
        gpu_codes[t] = []
        for b in range(B):
            np.testing.assert_array_equal(rec[b, :, :R_ref[b]], state["recent_" + t][b].transpose(1, 0, 2))
            got = oracle.untile_codes(pl[b], T_ref[b], M).transpose(1, 0, 2)  # [T, H, M]
            np.testing.assert_array_equal(got[:T0[b]], start_codes[t][b])
            rolled = T_ref[b] - T0[b]
            if rolled:
                tokens = np.concatenate([start_rec[t][b], new[t][:, b]], axis=0)[:rolled]
                ref, d1, d2, _ = oracle.encode(tokens, cb)
                check_codes(got[T0[b]:], tokens, cb, ref, d1, d2)
            untouched = np.ones(t_cap * M, bool)
            untouched[off[:T_ref[b]].reshape(-1)] = False
            assert np.all(pl[b][:, untouched] == FILL), "code bytes past the history were written"
            gpu_codes[t].append(got)

    # decode attention over the resulting cache
    q = synthkv.small_normal(seed + 30, (B, Hq, d)).astype(dt)
    scale = softmax_scale(d)
    Tm = int(T_ref.max())
    ck = np.zeros((B, Hkv, max(Tm, 1), M), np.uint8)
    cv = np.zeros_like(ck)
    for b in range(B):
        ck[b, :, :T_ref[b]] = gpu_codes["k"][b].transpose(1, 0, 2)
        cv[b, :, :T_ref[b]] = gpu_codes["v"][b].transpose(1, 0, 2)
    rk = recent["k"].cpu().numpy()
    rv = recent["v"].cpu().numpy()
    out, lse = run_gpu_decode(dims, q, cbk, cbv, planes["k"].cpu().numpy(), planes["v"].cpu().numpy(), t_cap,
                              T_ref, rk, rv, R_ref, scale, max_hist=max(Tm, 0))
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, T_ref, rk, rv, R_ref, scale)
    check_attention(out, lse, ref_out, ref_lse)


def test_append_leaves_bad_sequences_unchanged():
    """A sequence whose device lengths are out of bounds is not touched and its
    lengths are copied through; the others proceed."""
    import torch

    import decode_attention_pq_amd as P

    d, dsub, K, H, r_cap, n_roll, t_cap = 64, 2, 16, 2, 8, 4, 128
    M = d // dsub
    dims = dims_for(d, dsub, K, H, H)
    B = 3
    T0 = np.array([0, -5, 10], np.int32)   # sequence 1 has a negative history length
    R0 = np.array([8, 3, 99], np.int32)    # sequence 2's window is past r_cap
    cbk = _codebook(900, H, K, M, dsub)
    rk = to_dev(np.full((B, H, r_cap, d), 0.25, np.float16))
    rv = to_dev(np.full((B, H, r_cap, d), -0.5, np.float16))
    nk = to_dev(np.ones((B, H, d), np.float16))
    planes_k = torch.full((B, H, t_cap * M), FILL, dtype=torch.uint8, device="cuda")
    planes_v = planes_k.clone()
    hin, rin = to_dev(T0), to_dev(R0)
    hout = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    rout = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    P.append_kv(dims, nk, nk, rk, rv, hin, rin, hout, rout, n_roll, to_dev(cbk), to_dev(cbk), planes_k, planes_v,
                t_cap, 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(hout.cpu().numpy(), [n_roll, -5, 10])
    np.testing.assert_array_equal(rout.cpu().numpy(), [r_cap - n_roll + 1, 3, 99])
    rkh = rk.cpu().numpy()
    assert np.all(rkh[1] == np.float16(0.25)) and np.all(rkh[2] == np.float16(0.25))
    assert np.all(planes_k[1:].cpu().numpy() == FILL)
    assert np.all(rkh[0, :, r_cap - n_roll] == 1.0)  # the new row of the good sequence
