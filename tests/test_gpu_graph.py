"""Decode calls captured in a HIP graph.

A decode step allocates nothing, never synchronises with the host, records no
memset (the workspace's completion counters reset themselves) and reads the
sequence lengths from device memory, so a serving loop can capture it once and
replay it.  The graph below holds two decode calls (an 8-split long history
and a batch of single-split units); it is replayed several times with new
queries and lengths written into the captured buffers and eager work in
between, and every replay must equal an eager call on the same inputs bit for
bit, and the oracle within the attention tolerance.
"""
import math

import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, dims_for, softmax_scale, to_dev

pytestmark = pytest.mark.gpu


def _setup(B, Hq, Hkv, d, dsub, K, T, R, seed):
    M = d // dsub
    t_cap = -(-T // 64) * 64
    cbk = (synthkv.small_normal(seed + 1, (Hkv, K, M, dsub)) * 1.5).astype(np.float32)
    cbv = (synthkv.small_normal(seed + 2, (Hkv, K, M, dsub)) * 1.5).astype(np.float32)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (B, Hkv, R, d), np.float16)
    rv = synthkv.small_normal(seed + 6, (B, Hkv, R, d), np.float16)
    return dict(dims=dims_for(d, dsub, K, Hq, Hkv), B=B, Hq=Hq, d=d, T=T, R=R, t_cap=t_cap, np_cbk=cbk, np_cbv=cbv,
                np_ck=ck, np_cv=cv, np_rk=rk, np_rv=rv, cbk=to_dev(cbk), cbv=to_dev(cbv),
                ck=to_dev(oracle.tile_codes(ck, t_cap)), cv=to_dev(oracle.tile_codes(cv, t_cap)), rk=to_dev(rk),
                rv=to_dev(rv), scale=softmax_scale(d))


def test_decode_replays_in_a_graph():
    import torch

    import decode_attention_pq_amd as P

    cases = [_setup(1, 32, 32, 128, 2, 256, 32768, 16, 11), _setup(6, 8, 4, 128, 4, 256, 3000, 8, 12)]
    for c in cases:
        c["q"] = torch.zeros((c["B"], c["Hq"], c["d"]), dtype=torch.float16, device="cuda")
        c["hl"] = torch.zeros(c["B"], dtype=torch.int32, device="cuda")
        c["rl"] = torch.zeros(c["B"], dtype=torch.int32, device="cuda")
        c["out"] = torch.empty((c["B"], c["Hq"], c["d"]), dtype=torch.float32, device="cuda")
        c["lse"] = torch.empty((c["B"], c["Hq"]), dtype=torch.float32, device="cuda")
        c["ws"] = torch.zeros(P.decode_workspace_bytes(c["dims"], c["B"], c["T"]), dtype=torch.uint8, device="cuda")
        c["ws_eager"] = torch.zeros_like(c["ws"])

    def call(c, out, lse, ws):
        P.decode_attention(c["dims"], c["q"], c["cbk"], c["cbv"], c["ck"], c["cv"], c["t_cap"], c["hl"], c["T"],
                           c["rk"], c["rv"], c["rl"], c["scale"], out, lse, ws)

    def set_inputs(c, step):
        rng = np.random.default_rng(100 * step + c["B"])
        q = rng.standard_normal((c["B"], c["Hq"], c["d"])).astype(np.float16)
        hist = rng.integers(0, c["T"] + 1, c["B"]).astype(np.int32)
        hist[0] = c["T"] if step % 2 == 0 else hist[0]
        rec = rng.integers(0, c["R"] + 1, c["B"]).astype(np.int32)
        c["q"].copy_(torch.from_numpy(q))
        c["hl"].copy_(torch.from_numpy(hist))
        c["rl"].copy_(torch.from_numpy(rec))
        return q, hist, rec

    for c in cases:  # warm up outside the capture
        set_inputs(c, 0)
        call(c, c["out"], c["lse"], c["ws"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in cases:
            call(c, c["out"], c["lse"], c["ws"])
    for step in range(1, 5):
        inputs = [set_inputs(c, step) for c in cases]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        graph_res = [(c["out"].cpu().numpy().copy(), c["lse"].cpu().numpy().copy()) for c in cases]
        # eager work between replays: the same calls, on their own outputs and workspace
        for c, (go, gl), (q, hist, rec) in zip(cases, graph_res, inputs):
            eo, el = torch.empty_like(c["out"]), torch.empty_like(c["lse"])
            call(c, eo, el, c["ws_eager"])
            torch.cuda.synchronize()
            assert np.array_equal(go, eo.cpu().numpy()), f"replay {step}: output differs from the eager call"
            assert np.array_equal(gl, el.cpu().numpy(), equal_nan=True), f"replay {step}: lse differs"
            ref_out, ref_lse = oracle.decode_exact(q, c["np_cbk"], c["np_cbv"], c["np_ck"], c["np_cv"], hist,
                                                   c["np_rk"], c["np_rv"], rec, c["scale"])
            check_attention(go, gl, ref_out, ref_lse)
