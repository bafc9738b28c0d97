"""pqkv_decode_attention_noalloc (static device scratch instead of a workspace)
against pqkv_decode_attention on the same inputs: identical results, and within
the oracle's tolerance, over calls in a row whose sizes go down and up again
(the counters of the shared array must be zero at every call's start)."""
import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, dims_for, softmax_scale, to_dev

pytestmark = pytest.mark.gpu

CALLS = [
    # d, dsub, K, Hq, Hkv, hist, rec, r_cap
    (128, 2, 256, 32, 32, (8192,), (128,), 128),          # 2 splits of 4096 per head: partials and merge
    (128, 2, 256, 8, 8, (3000, 100), (5, 0), 16),         # a smaller call
    (128, 4, 256, 32, 8, (20000, 700, 0), (17, 3, 9), 64),  # larger again: GQA, more rows and splits
    (64, 2, 16, 4, 4, (512,), (16,), 16),                 # the smallest
]


def _inputs(i, case):
    d, dsub, K, Hq, Hkv, hist, rec, r_cap = case
    B, M = len(hist), d // dsub
    t_cap = max(64, -(-max(hist) // 64) * 64)
    s = 900 + 10 * i
    cb = lambda k: (np.random.default_rng(s + k).standard_normal((Hkv, K, M, dsub))).astype(np.float32)
    return dict(q=synthkv.small_normal(s, (B, Hq, d), np.float16), cbk=cb(1), cbv=cb(2),
                ck=synthkv.small_codes(s + 3, (B, Hkv, t_cap, M), K),
                cv=synthkv.small_codes(s + 4, (B, Hkv, t_cap, M), K),
                rk=synthkv.small_normal(s + 5, (B, Hkv, r_cap, d), np.float16),
                rv=synthkv.small_normal(s + 6, (B, Hkv, r_cap, d), np.float16), t_cap=t_cap)


def _run(P, dims, x, hist, rec, noalloc):
    import torch

    B, Hq, d = x["q"].shape
    t_cap = x["t_cap"]
    out = torch.full((B, Hq, d), np.nan, dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), np.nan, dtype=torch.float32, device="cuda")
    ws = None
    if not noalloc:
        ws = torch.zeros(P.decode_workspace_bytes(dims, B, max(hist)), dtype=torch.uint8, device="cuda")
    P.decode_attention(dims, to_dev(x["q"]), to_dev(x["cbk"]), to_dev(x["cbv"]),
                       to_dev(oracle.tile_codes(x["ck"], t_cap)), to_dev(oracle.tile_codes(x["cv"], t_cap)), t_cap,
                       to_dev(np.asarray(hist, np.int32)), max(hist), to_dev(x["rk"]), to_dev(x["rv"]),
                       to_dev(np.asarray(rec, np.int32)), softmax_scale(d), out, lse, ws, noalloc=noalloc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_noalloc_matches_workspace_entry_point():
    import decode_attention_pq_amd as P

    for rep in range(2):  # every size twice over: the array keeps the last call's contents
        for i, case in enumerate(CALLS):
            d, dsub, K, Hq, Hkv, hist, rec, r_cap = case
            print(f"[noalloc] pass {rep} call {i}: d {d} d_sub {dsub} K {K} heads {Hq}/{Hkv} hist {hist}",
                  flush=True)
            dims = dims_for(d, dsub, K, Hq, Hkv)
            x = _inputs(i, case)
            got, got_lse = _run(P, dims, x, hist, rec, noalloc=True)
            ref, ref_lse = _run(P, dims, x, hist, rec, noalloc=False)
            np.testing.assert_array_equal(got, ref)
            np.testing.assert_array_equal(got_lse, ref_lse)
            o_out, o_lse = oracle.decode_exact(x["q"], x["cbk"], x["cbv"], x["ck"], x["cv"], hist, x["rk"], x["rv"],
                                               rec, softmax_scale(d))
            check_attention(got, got_lse, o_out, o_lse)
