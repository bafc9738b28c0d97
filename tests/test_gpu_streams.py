"""Calls on two streams at once.

The library keeps no mutable global state (the no-allocation entry point aside): every
decode call owns its workspace and outputs, every encode call its code planes.  Here two
independent decode problems (a 32K-token history with 8 splits, and a ragged batch of four
sequences on the device-side plan) and an encode run concurrently, each repeatedly on its own
stream (default priority), and every result must equal the same call run alone on one stream,
bit for bit.  The kernels are deterministic: integer histogram adds, and partials merged in
split order by whichever work-group finishes last.
"""
import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import dims_for, softmax_scale, to_dev

pytestmark = pytest.mark.gpu


def _decode_case(B, Hq, Hkv, d, dsub, K, hist, R, seed):
    import torch

    import decode_attention_pq_amd as P

    M = d // dsub
    T = max(hist)
    t_cap = -(-T // 64) * 64
    c = dict(dims=dims_for(d, dsub, K, Hq, Hkv), B=B, T=T, t_cap=t_cap, scale=softmax_scale(d))
    c["q"] = to_dev(synthkv.small_normal(seed, (B, Hq, d), np.float16))
    c["cbk"] = to_dev((synthkv.small_normal(seed + 1, (Hkv, K, M, dsub)) * 1.5).astype(np.float32))
    c["cbv"] = to_dev((synthkv.small_normal(seed + 2, (Hkv, K, M, dsub)) * 1.5).astype(np.float32))
    c["ck"] = to_dev(oracle.tile_codes(synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K), t_cap))
    c["cv"] = to_dev(oracle.tile_codes(synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K), t_cap))
    c["rk"] = to_dev(synthkv.small_normal(seed + 5, (B, Hkv, R, d), np.float16))
    c["rv"] = to_dev(synthkv.small_normal(seed + 6, (B, Hkv, R, d), np.float16))
    c["hl"] = torch.tensor(hist, dtype=torch.int32, device="cuda")
    c["rl"] = torch.full((B,), R, dtype=torch.int32, device="cuda")
    c["out"] = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    c["lse"] = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    c["ws"] = torch.zeros(P.decode_workspace_bytes(c["dims"], B, T), dtype=torch.uint8, device="cuda")
    return c


def _decode(c):
    import decode_attention_pq_amd as P

    P.decode_attention(c["dims"], c["q"], c["cbk"], c["cbv"], c["ck"], c["cv"], c["t_cap"], c["hl"], c["T"],
                       c["rk"], c["rv"], c["rl"], c["scale"], c["out"], c["lse"], c["ws"])


def test_decode_and_encode_on_two_streams():
    import torch

    import decode_attention_pq_amd as P

    a = _decode_case(1, 32, 32, 128, 2, 256, [32768], 64, 31)
    b = _decode_case(4, 16, 8, 128, 4, 256, [9000, 700, 15000, 4100], 32, 32)
    # an encode of 3 sequences x 3000 tokens x 4 heads, d_sub 2 (the bounded-scan kernel)
    d, dsub, K, H, N, ns = 128, 2, 256, 4, 3000, 3
    M = d // dsub
    t_cap = -(-N // 64) * 64
    rng = np.random.default_rng(33)
    x = rng.standard_normal((ns, N, H, d)).astype(np.float32)
    x[..., :3] *= 10.0
    x = to_dev(x.astype(np.float16))
    cb = to_dev((np.random.default_rng(34).standard_normal((H, K, M, dsub)) * 3).astype(np.float32))
    edims = dims_for(d, dsub, K, H, H)
    codes = torch.zeros((ns, H, t_cap * M), dtype=torch.uint8, device="cuda")

    # each call alone, on the current stream
    _decode(a)
    _decode(b)
    P.encode(edims, x, cb, codes, t_cap)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (a["out"], a["lse"], b["out"], b["lse"], codes)]

    # then concurrently: 20 decode calls of each problem and 5 encodes, on two streams
    for t in (a["out"], a["lse"], b["out"], b["lse"]):
        t.fill_(float("nan"))
    codes.fill_(0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        for _ in range(20):
            _decode(a)
    with torch.cuda.stream(s2):
        for i in range(20):
            _decode(b)
            if i % 4 == 0:
                P.encode(edims, x, cb, codes, t_cap)
    torch.cuda.synchronize()
    got = (a["out"], a["lse"], b["out"], b["lse"], codes)
    for name, r, g in zip(("out A", "lse A", "out B", "lse B", "codes"), ref, got):
        assert torch.equal(r, g), name
    # and the lone calls were right in the first place
    assert torch.isfinite(ref[0]).all() and torch.isfinite(ref[2]).all()
