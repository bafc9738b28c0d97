"""GPU parity on small shapes: every entry point of libpqkv against the CPU oracle.

Sizes are small enough for the oracle to finish in seconds but span several
64-token tiles, several history splits and ragged tails, and cover the edge
cases: empty history, empty recent window, both empty, one token, GQA groups,
both subspace dimensions and head sizes, fp16 and fp32 inputs, duplicate
centroids and unaligned append positions.
"""
import itertools

import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import (check_attention, check_codes, dims_for, run_gpu_decode, run_gpu_encode,
                          softmax_scale, to_dev)

pytestmark = pytest.mark.gpu


def _outlier_values(seed, shape, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x[..., :3] *= 10.0
    x[rng.random(shape) < 0.01] *= 20.0
    return x.astype(dtype)


def _codebook(seed, H, K, M, dsub, scale=3.0):
    return (np.random.default_rng(seed).standard_normal((H, K, M, dsub)) * scale).astype(np.float32)


@pytest.mark.parametrize("d,dsub", [(128, 2), (128, 4), (64, 2), (64, 4)])
@pytest.mark.parametrize("K", [256, 37])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_encode_matches_oracle(d, dsub, K, dtype):
    H, N, n_seqs, t_cap, t_start = 3, 300, 2, 384, 17
    M = d // dsub
    x = _outlier_values(d * 7 + K, (n_seqs, N, H, d), dtype)
    cb = _codebook(K + dsub, H, K, M, dsub)
    dims = dims_for(d, dsub, K, H, H)
    fill = np.full((n_seqs, H, t_cap * M), 0xAB, np.uint8)
    planes = run_gpu_encode(dims, x, cb, n_seqs, t_cap, t_start, init_codes=fill)
    off = oracle.code_offsets(M, t_cap)
    written = np.zeros(t_cap * M, bool)
    written[off[t_start:t_start + N].ravel()] = True
    assert np.all(planes[..., ~written] == 0xAB), "bytes outside the encoded tokens changed"
    for s in range(n_seqs):
        ref, d1, d2, amb = oracle.encode(x[s], cb)
        got = oracle.untile_codes(planes[s], t_start + N, M)[:, t_start:].transpose(1, 0, 2)
        check_codes(got, x[s], cb, ref, d1, d2)


@pytest.mark.parametrize("d,dsub", [(128, 2), (128, 4), (64, 2), (64, 4)])
@pytest.mark.parametrize("K", [64, 192])
def test_encode_several_tokens_per_lane(d, dsub, K):
    # 2500 tokens: every lane scans 2 or 4 tokens (one to three of them live in the
    # last block), over 1 or 3 blocks of 64 centroids
    H, N, t_cap, t_start = 2, 2500, 2560, 40
    M = d // dsub
    x = _outlier_values(d * 3 + K + dsub, (1, N, H, d), np.float16)
    cb = _codebook(K * 5 + dsub, H, K, M, dsub)
    fill = np.full((1, H, t_cap * M), 0xAB, np.uint8)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x, cb, 1, t_cap, t_start, init_codes=fill)
    off = oracle.code_offsets(M, t_cap)
    written = np.zeros(t_cap * M, bool)
    written[off[t_start:t_start + N].ravel()] = True
    assert np.all(planes[..., ~written] == 0xAB), "bytes outside the encoded tokens changed"
    ref, d1, d2, amb = oracle.encode(x[0], cb)
    got = oracle.untile_codes(planes[0], t_start + N, M)[:, t_start:].transpose(1, 0, 2)
    check_codes(got, x[0], cb, ref, d1, d2)


@pytest.mark.parametrize("K,keep,dups", [(64, 7, (40, 63)), (256, 70, (130, 200, 255)), (256, 7, (64, 100)),
                                         (48, 5, (17, 47)), (128, 3, (5, 15)), (256, 17, (18, 31, 32, 47)),
                                         (256, 240, (241, 255))])
def test_encode_duplicate_centroids_lowest_index(K, keep, dups):
    # exact ties inside one sub-block of 16 centroids, across sub-blocks and across
    # blocks of 64: the lowest index wins
    d, dsub, H = 128, 2, 2
    M = d // dsub
    cb = _codebook(5, H, K, M, dsub)
    for c in dups:
        cb[:, c] = cb[:, keep]
    x = np.repeat(cb[:, keep][None], 70, axis=0).reshape(70, H, d).astype(np.float32)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x[None], cb, 1, 128)
    got = oracle.untile_codes(planes[0], 70, M)
    assert np.all(got == keep)


@pytest.mark.parametrize("keep,dups", [(70, (130, 200, 255)), (100, (3, 250)), (17, (16, 18, 19)),
                                       (240, (0, 241, 255)), (5, (6, 7, 21, 37))])
@pytest.mark.parametrize("d", [128, 64])
def test_encode_ties_at_dsub4(d, keep, dups):
    # d_sub 4 with 256 centroids (the matrix-core encode): exact copies of one centroid
    # in the same group of 4, in other groups of the same block, in other blocks, and
    # below its index -- the lowest index of the copies wins -- and near copies (a few
    # ulp away) whose codes must lie in the oracle's ambiguity band
    dsub, K, H = 4, 256, 2
    M = d // dsub
    cb = _codebook(11 + keep, H, K, M, dsub)
    for c in dups:
        cb[:, c] = cb[:, keep]
    x = np.repeat(cb[:, keep][None], 70, axis=0).reshape(70, H, d).astype(np.float32)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x[None], cb, 1, 128)
    got = oracle.untile_codes(planes[0], 70, M)
    assert np.all(got == min((keep,) + tuple(dups)))
    # near copies: each copy moved by a few ulp in one component
    cb2 = cb.copy()
    for n, c in enumerate(dups):
        cb2[:, c, :, n % dsub] = np.nextafter(np.nextafter(cb[:, c, :, n % dsub], np.inf), np.inf)
    x2 = x + np.float32(1e-3) * synthkv.small_normal(keep, x.shape)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x2[None], cb2, 1, 128)
    got = oracle.untile_codes(planes[0], 70, M).transpose(1, 0, 2)
    ref, d1, d2, _ = oracle.encode(x2, cb2)
    check_codes(got, x2, cb2, ref, d1, d2)


@pytest.mark.parametrize("keep,dups", [(70, (130, 200, 255)), (17, (16, 18, 19)), (240, (0, 241)),
                                       (5, (21,)), (100, (36, 164, 228))])
@pytest.mark.parametrize("d", [128, 64])
def test_encode_near_ties_at_dsub2(d, keep, dups):
    # d_sub 2 with 256 centroids (the bounded expanded-form scan): copies of one centroid
    # in its own and in other sub-blocks of 16, exact (the lowest index wins) and moved by
    # a few ulp (near ties the bound cannot separate: the second or third best sub-block
    # is rescanned, or the whole subspace); every code against the fp32 decision
    dsub, K, H = 2, 256, 2
    M = d // dsub
    cb = _codebook(31 + keep, H, K, M, dsub)
    for c in dups:
        cb[:, c] = cb[:, keep]
    x = np.repeat(cb[:, keep][None], 70, axis=0).reshape(70, H, d).astype(np.float32)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x[None], cb, 1, 128)
    got = oracle.untile_codes(planes[0], 70, M)
    assert np.all(got == min((keep,) + tuple(dups)))
    cb2 = cb.copy()
    for n, c in enumerate(dups):
        cb2[:, c, :, n % dsub] = np.nextafter(np.nextafter(cb[:, c, :, n % dsub], np.inf), np.inf)
    x2 = x + np.float32(1e-3) * synthkv.small_normal(keep + 1, x.shape)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x2[None], cb2, 1, 128)
    got = oracle.untile_codes(planes[0], 70, M).transpose(1, 0, 2)
    ref, d1, d2, _ = oracle.encode(x2, cb2)
    check_codes(got, x2, cb2, ref, d1, d2)


@pytest.mark.parametrize("K", [256, 40])
def test_encode_nan_and_inf_rows(K):
    # a NaN subvector has no nearest centroid under '<': code 0, as in the oracle; an
    # infinite one is at infinite distance from every centroid: code 0 as well
    d, dsub, H = 64, 4, 1
    M = d // dsub
    cb = _codebook(6, H, K, M, dsub)
    x = _outlier_values(7, (1, 64, H, d), np.float32)
    x[0, 3, 0, 8] = np.nan
    x[0, 9, 0, :] = np.inf
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x, cb, 1, 64)
    got = oracle.untile_codes(planes[0], 64, M)
    ref, _, _, _ = oracle.encode(x[0], cb)
    assert got[0, 3, 2] == 0 and np.all(got[0, 9] == 0)
    assert got[0, 3, 2] == ref[3, 0, 2] and np.array_equal(got[0, 9], ref[9, 0])
    np.testing.assert_array_equal(got.transpose(1, 0, 2), oracle.encode_f32(x[0], cb))


@pytest.mark.parametrize("d", [128, 64])
def test_encode_nonfinite_and_huge_centroids(d):
    # d_sub 4, 256 centroids: a NaN centroid (never the code), an infinite one, and one
    # whose |c|^2 overflows fp32, each in its own subspace; every code against the fp32
    # decision
    dsub, K, H = 4, 256, 2
    M = d // dsub
    cb = _codebook(21, H, K, M, dsub)
    cb[0, 7, 1, 2] = np.nan
    cb[1, 200, 3, 0] = np.inf
    cb[0, 31, 5, :] = 3.0e19
    x = _outlier_values(22, (1, 300, H, d), np.float32)
    x[0, 5, 0, 5 * dsub:6 * dsub] = 2.9e19  # nearest to the huge centroid, at a finite fp32 distance
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x, cb, 1, 320)
    got = oracle.untile_codes(planes[0], 300, M).transpose(1, 0, 2)
    np.testing.assert_array_equal(got, oracle.encode_f32(x[0], cb))
    assert np.all(got[:, 0, 1] != 7)


@pytest.mark.parametrize("dsub", [4, 2])
def test_encode_denormal_distances(dsub):
    # values near 1e-20: squared distances in the fp32 denormal range, where the code
    # depends on denormals being kept; every code against the fp32 decision
    d, K, H = 64, 256, 1
    M = d // dsub
    cb = (_codebook(23, H, K, M, dsub) * np.float32(1e-20)).astype(np.float32)
    x = (_outlier_values(24, (1, 500, H, d), np.float32) * np.float32(1e-20)).astype(np.float32)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x, cb, 1, 512)
    got = oracle.untile_codes(planes[0], 500, M).transpose(1, 0, 2)
    np.testing.assert_array_equal(got, oracle.encode_f32(x[0], cb))


def test_encode_deterministic():
    d, dsub, K, H = 128, 2, 256, 4
    x = _outlier_values(3, (1, 1000, H, d), np.float16)
    cb = _codebook(4, H, K, d // dsub, dsub)
    dims = dims_for(d, dsub, K, H, H)
    a = run_gpu_encode(dims, x, cb, 1, 1024)
    b = run_gpu_encode(dims, x, cb, 1, 1024)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("d,dsub,Hq,Hkv", [(128, 2, 4, 2), (128, 4, 8, 2), (64, 2, 3, 3), (64, 4, 8, 2)])
@pytest.mark.parametrize("qdtype", [np.float16, np.float32])
def test_build_lut_matches_oracle(d, dsub, Hq, Hkv, qdtype):
    import torch

    import decode_attention_pq_amd as P

    K, B = 200, 3
    M = d // dsub
    q = synthkv.small_normal(11, (B, Hq, d), qdtype)
    cb = _codebook(12, Hkv, K, M, dsub)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    lut = torch.full((B, Hq, M, K), np.nan, dtype=torch.float32, device="cuda")
    P.build_lut(dims, to_dev(q), to_dev(cb), lut)
    torch.cuda.synchronize()
    got = lut.cpu().numpy()
    ref = oracle.lut(q, cb, Hq // Hkv)
    g = Hq // Hkv
    qs = np.abs(q.astype(np.float64)).reshape(B, Hq, M, dsub)
    bound = np.einsum("bhmj,hcmj->bhmc", qs, np.abs(cb[np.arange(Hq) // g]).astype(np.float64))
    assert np.all(np.abs(got - ref) <= 1e-6 * bound + 1e-30)


DECODE_CASES = [
    # d, dsub, K, Hq, Hkv, hist_len, recent_len, r_cap, dtype
    (128, 2, 256, 4, 4, (700,), (5,), 8, np.float16),            # one split, ragged tail
    (128, 2, 256, 2, 1, (5000, 0), (3, 0), 4, np.float16),        # many splits; second row empty
    (128, 2, 256, 2, 2, (0, 1, 64, 65), (7, 0, 1, 0), 8, np.float16),  # empty history / one token / tile edges
    (128, 2, 37, 8, 2, (3000, 1025), (0, 12), 16, np.float16),    # GQA g=4 with M=64 (two groups), K=37
    (128, 4, 256, 8, 2, (4097, 2048), (16, 1), 16, np.float16),   # d_sub=4: two query heads per work-group
    (64, 2, 16, 4, 4, (512,), (16,), 16, np.float32),             # the tiny shape, fp32
    (64, 4, 64, 8, 2, (1500, 3), (2, 2), 4, np.float32),          # M=16: four query heads per work-group
    (128, 2, 256, 2, 2, (2000, 40), (0, 0), 0, np.float16),       # no recent window at all
    (128, 2, 256, 1, 1, (0,), (0,), 4, np.float16),               # nothing cached
    # ragged batches: sequences that use fewer splits than the longest (their other
    # work-groups exit early; the recent window goes to the splits in use), a window
    # larger than one split's share, and units that straddle XCDs
    (128, 2, 256, 2, 2, (100, 9000), (200, 3), 256, np.float16),
    (128, 2, 256, 3, 3, (4096, 0, 17, 12000, 4097, 8191), (1, 64, 0, 5, 64, 2), 64, np.float16),
    (128, 4, 256, 8, 2, (20000, 300, 0), (33, 0, 9), 64, np.float16),
    # the largest recent window: 1024 rows in the one split of a short or empty history, and
    # spread over the splits of a long one
    (128, 2, 256, 2, 2, (100, 0), (1024, 1024), 1024, np.float16),
    (64, 4, 256, 8, 2, (70000,), (1000,), 1024, np.float32),
    # enough (sequence, head) units to fill the CUs with one split each: 13 rounds per wave
    # in the 16-round build (three unused steps), ragged and empty rows among them
    (128, 2, 64, 32, 32, (6500, 100, 0, 6144, 6145, 3000, 6600, 5000), (3,) * 8, 8, np.float16),
    # 10 rounds per wave in the 12-round build (two unused steps)
    (128, 2, 256, 32, 32, (5000, 4999, 1, 2500, 5000, 4097, 64, 4096), (0, 1, 2, 3, 4, 5, 6, 7), 8, np.float16),
    # 2 rounds, the 2-round build's full length, ragged, with empty rows
    (128, 2, 256, 32, 32, (1000, 513, 0, 1024, 999, 64, 1, 700), (2, 0) * 4, 4, np.float16),
    # 4 rounds (the 4-round build) and 3 rounds in it, ragged, with empty rows
    (128, 2, 256, 32, 32, (2000, 1900, 0, 1, 2048, 1500, 64, 1999), (4, 0) * 4, 4, np.float16),
    (128, 2, 256, 32, 32, (1536, 1000, 1535, 0, 1200, 1, 513, 1536), (0, 3) * 4, 4, np.float16),
    # 12 rounds, the 12-round build's full length, and 9 rounds in it
    (128, 2, 256, 32, 32, (6144, 6100, 0, 12, 6144, 3001, 6143, 64), (2,) * 8, 4, np.float16),
    (128, 2, 96, 32, 32, (4500, 4400, 4097, 1, 0, 4500, 3000, 4499), (1, 0) * 4, 4, np.float16),
    # d_sub 4, two query heads per work-group, 10 rounds in the 16-round build
    (128, 4, 256, 32, 8, (20000, 19000, 300, 20000), (5, 0, 9, 2), 16, np.float16),
    # the device-side split plan at its largest batch (16 ragged sequences, empty ones and
    # tile edges among them), one sequence more (the host plan again), and 16 equal
    # lengths (the device plan keeps the host's)
    (128, 2, 256, 4, 4, (9000, 0, 1, 64, 65, 4096, 4097, 300, 8191, 8192, 2, 1000, 7000, 513, 0, 3333),
     (1, 2, 0, 8, 3, 0, 5, 8, 1, 0, 2, 7, 0, 4, 6, 8), 8, np.float16),
    (128, 2, 256, 4, 4, (9000, 0, 1, 64, 65, 4096, 4097, 300, 8191, 8192, 2, 1000, 7000, 513, 0, 3333, 5000),
     (1, 2, 0, 8, 3, 0, 5, 8, 1, 0, 2, 7, 0, 4, 6, 8, 3), 8, np.float16),
    (128, 4, 256, 8, 2, (3000,) * 16, (2,) * 16, 4, np.float16),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"case{i}" for i in range(len(DECODE_CASES))])
def test_decode_matches_oracle(case):
    d, dsub, K, Hq, Hkv, hist, rec, r_cap, dt = case
    B = len(hist)
    M = d // dsub
    t_cap = max(64, -(-max(hist) // 64) * 64)
    seed = sum(hist) + 31 * K + d
    q = synthkv.small_normal(seed, (B, Hq, d), dt)
    cbk = _codebook(seed + 1, Hkv, K, M, dsub, 1.0)
    cbv = _codebook(seed + 2, Hkv, K, M, dsub, 1.0)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (B, Hkv, r_cap, d), dt)
    rv = synthkv.small_normal(seed + 6, (B, Hkv, r_cap, d), dt)
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, hist, rk, rv, rec, scale)
    pk, pv = oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    out, lse = run_gpu_decode(dims, q, cbk, cbv, pk, pv, t_cap, hist, rk if r_cap else None,
                              rv if r_cap else None, rec, scale)
    check_attention(out, lse, ref_out, ref_lse)
    if max(hist) > 0:  # a looser host bound on the history length gives the same result
        out2, lse2 = run_gpu_decode(dims, q, cbk, cbv, pk, pv, t_cap, hist, rk if r_cap else None,
                                    rv if r_cap else None, rec, scale, max_hist=t_cap)
        check_attention(out2, lse2, ref_out, ref_lse)


LUT_CASES = [i for i, c in enumerate(DECODE_CASES) if c[2] % 4 == 0 and max(c[5]) > 0]


@pytest.mark.parametrize("i", LUT_CASES, ids=[f"case{i}" for i in LUT_CASES])
def test_decode_with_materialised_lut(i):
    """pqkv_build_lut's table passed to pqkv_decode_attention in place of the key
    codebook (the ad-LUT built first, then read for every token), against the
    oracle's exact attention."""
    d, dsub, K, Hq, Hkv, hist, rec, r_cap, dt = DECODE_CASES[i]
    B = len(hist)
    M = d // dsub
    t_cap = max(64, -(-max(hist) // 64) * 64)
    seed = sum(hist) + 31 * K + d + 7
    q = synthkv.small_normal(seed, (B, Hq, d), dt)
    cbk = _codebook(seed + 1, Hkv, K, M, dsub, 1.0)
    cbv = _codebook(seed + 2, Hkv, K, M, dsub, 1.0)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (B, Hkv, r_cap, d), dt)
    rv = synthkv.small_normal(seed + 6, (B, Hkv, r_cap, d), dt)
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, hist, rk, rv, rec, scale)
    pk, pv = oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    r = (rk, rv) if r_cap else (None, None)
    out, lse = run_gpu_decode(dims, q, cbk, cbv, pk, pv, t_cap, hist, r[0], r[1], rec, scale, lut="gpu")
    check_attention(out, lse, ref_out, ref_lse)
    # the oracle's own table (fp64, rounded to fp32) gives the same result
    out2, lse2 = run_gpu_decode(dims, q, cbk, cbv, pk, pv, t_cap, hist, r[0], r[1], rec, scale,
                                lut=oracle.lut(q, cbk, Hq // Hkv))
    check_attention(out2, lse2, ref_out, ref_lse)


def test_decode_recent_window_only_without_lengths():
    """No history (max_hist_len 0): hist_len, codes and codebooks may all be NULL."""
    import torch

    import decode_attention_pq_amd as P

    d, dsub, K, Hq, Hkv, B, r_cap = 128, 2, 256, 8, 4, 3, 16
    rec = [16, 0, 5]
    q = synthkv.small_normal(91, (B, Hq, d), np.float16)
    rk = synthkv.small_normal(92, (B, Hkv, r_cap, d), np.float16)
    rv = synthkv.small_normal(93, (B, Hkv, r_cap, d), np.float16)
    scale = softmax_scale(d)
    M = d // dsub
    empty = np.zeros((B, Hkv, 64, M), np.uint8)
    cb = np.zeros((Hkv, K, M, dsub), np.float32)
    ref_out, ref_lse = oracle.decode_exact(q, cb, cb, empty, empty, [0] * B, rk, rv, rec, scale)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    out = torch.full((B, Hq, d), np.nan, device="cuda")
    lse = torch.full((B, Hq), np.nan, device="cuda")
    ws = torch.zeros(P.decode_workspace_bytes(dims, B, 0), dtype=torch.uint8, device="cuda")
    P.decode_attention(dims, to_dev(q), None, None, None, None, 0, None, 0, to_dev(rk), to_dev(rv),
                       to_dev(np.asarray(rec, np.int32)), scale, out, lse, ws)
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)


def test_workspace_reuse_when_max_hist_len_changes():
    """One zeroed workspace across calls whose split plans differ (4096 tokens: 8
    splits per head; 4160: 5 splits; and back), each checked against the oracle: the
    completion counters sit at a fixed place, so no call reads another's partials as
    counters."""
    import torch

    import decode_attention_pq_amd as P

    d, dsub, K, H, B = 128, 2, 256, 32, 1
    M = d // dsub
    dims = dims_for(d, dsub, K, H, H)
    t_cap = 4224
    sizes = [P.decode_workspace_bytes(dims, B, T) for T in (4096, 4160)]
    assert sizes[0] != sizes[1], "the two lengths should take different split plans"
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device="cuda")
    scale = softmax_scale(d)
    for it, T in enumerate((4096, 4160, 4096, 4160)):
        q = synthkv.small_normal(700 + it, (B, H, d), np.float16)
        cbk = _codebook(710 + it, H, K, M, dsub, 1.0)
        cbv = _codebook(720 + it, H, K, M, dsub, 1.0)
        ck = synthkv.small_codes(730 + it, (B, H, t_cap, M), K)
        cv = synthkv.small_codes(740 + it, (B, H, t_cap, M), K)
        ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, [T], np.zeros((B, H, 0, d), np.float16),
                                               np.zeros((B, H, 0, d), np.float16), [0], scale)
        out, lse = run_gpu_decode(dims, q, cbk, cbv, oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap),
                                  t_cap, [T], None, None, [0], scale, max_hist=T, workspace=ws)
        check_attention(out, lse, ref_out, ref_lse)


def test_tiny_workload_end_to_end():
    """The Tiny workload: codebooks fit by 10 Lloyd iterations on its own history,
    GPU encode bit-exact with the oracle, GPU decode within tolerance."""
    w = synthkv.WORKLOADS["tiny"]
    M, d = w.n_sub, w.head_dim
    dims = dims_for(d, w.d_sub, w.n_centroids, w.n_q_heads, w.n_kv_heads)
    t_cap = w.t_cap
    cbs, codes = {}, {}
    for tensor in ("k", "v"):
        cb = oracle.fit_workload_codebooks(w, 0, tensor, synthkv)
        x = synthkv.history_kv(w, 0, tensor, 0)
        ref, d1, d2, _ = oracle.encode(x, cb)
        planes = run_gpu_encode(dims, x[None], cb, 1, t_cap)
        got = oracle.untile_codes(planes[0], w.hist_len[0], M).transpose(1, 0, 2)
        check_codes(got, x, cb, ref, d1, d2)
        cbs[tensor] = cb
        codes[tensor] = ref.transpose(1, 0, 2)[None]  # [1, H, T, M]
    q = synthkv.queries(w)
    rk, rv = synthkv.recent_kv(w, 0, "k"), synthkv.recent_kv(w, 0, "v")
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbs["k"], cbs["v"], codes["k"], codes["v"], w.hist_len, rk, rv,
                                           [w.recent_len], scale)
    out, lse = run_gpu_decode(dims, q, cbs["k"], cbs["v"], oracle.tile_codes(codes["k"], t_cap),
                              oracle.tile_codes(codes["v"], t_cap), t_cap, w.hist_len, rk, rv, [w.recent_len],
                              scale)
    check_attention(out, lse, ref_out, ref_lse)


def test_merge_matches_oracle():
    import torch

    import decode_attention_pq_amd as P

    rng = np.random.default_rng(21)
    n, d = 37, 128
    oa, ob = rng.standard_normal((n, d)).astype(np.float32), rng.standard_normal((n, d)).astype(np.float32)
    la, lb = (rng.standard_normal(n) * 5).astype(np.float32), (rng.standard_normal(n) * 5).astype(np.float32)
    la[3] = -np.inf
    lb[4] = -np.inf
    la[5] = lb[5] = -np.inf
    ref_o, ref_l = oracle.merge_states(oa, la, ob, lb)
    A, LA, Bt, LB = to_dev(oa), to_dev(la), to_dev(ob), to_dev(lb)
    out = torch.empty_like(A)
    lse = torch.empty_like(LA)
    P.merge(A, LA, Bt, LB, out, lse)
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, rtol=1e-5, lse_rtol=1e-6)
    P.merge(A, LA, Bt, LB, A, LA)  # in place over the first state
    torch.cuda.synchronize()
    check_attention(A.cpu().numpy(), LA.cpu().numpy(), ref_o, ref_l, rtol=1e-5, lse_rtol=1e-6)


def test_two_step_decode_merges_like_one():
    """Splitting the recent window off into a second state and merging with
    pqkv_merge reproduces the single call (blockwise history/new-token attention)."""
    import torch

    import decode_attention_pq_amd as P

    d, dsub, K, H = 128, 2, 256, 4
    M = d // dsub
    T, R, t_cap = 900, 12, 960
    q = synthkv.small_normal(1, (1, H, d), np.float16)
    cbk, cbv = _codebook(2, H, K, M, dsub, 1.0), _codebook(3, H, K, M, dsub, 1.0)
    ck, cv = synthkv.small_codes(4, (1, H, t_cap, M), K), synthkv.small_codes(5, (1, H, t_cap, M), K)
    rk, rv = synthkv.small_normal(6, (1, H, R, d), np.float16), synthkv.small_normal(7, (1, H, R, d), np.float16)
    scale = softmax_scale(d)
    dims = dims_for(d, dsub, K, H, H)
    pk, pv = oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap)
    o1, l1 = run_gpu_decode(dims, q, cbk, cbv, pk, pv, t_cap, [T], None, None, [0], scale)
    empty = np.zeros((1, H, t_cap * M), np.uint8)
    o2, l2 = run_gpu_decode(dims, q, cbk, cbv, empty, empty, t_cap, [0], rk, rv, [R], scale)
    out, lse = torch.empty(H, d, device="cuda"), torch.empty(H, device="cuda")
    P.merge(to_dev(o1[0]), to_dev(l1[0]), to_dev(o2[0]), to_dev(l2[0]), out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, [T], rk, rv, [R], scale)
    check_attention(out.cpu().numpy()[None], lse.cpu().numpy()[None], ref_out, ref_lse)


@pytest.mark.parametrize("hist", [8192, 4096])
def test_decode_many_small_weights_are_kept(hist):
    """One token outweighs each of the others by about 2^20.5, and the others together
    carry ~0.5% of the attention.  Their weights must survive the histogram's fixed
    point: dropping them moves the output by ~1%, five times the tolerance.  Splits of
    4096 and 8192 tokens (one split per sequence: 8 x 32 = 256 units fill the CUs)."""
    d, dsub, K, H, B = 128, 2, 16, 32, 8
    M = d // dsub
    t_cap = hist
    top = 2917  # the heavy token
    cbk = np.zeros((H, K, M, dsub), np.float32)
    cbk[:, 1, :, 0] = 1.0
    cbv = np.zeros((H, K, M, dsub), np.float32)
    cbv[:, 0] = 1.0
    cbv[:, 1] = -1.0
    ck = np.zeros((B, H, t_cap, M), np.uint8)
    ck[:, :, top] = 1
    cv = ck.copy()
    scale = softmax_scale(d)
    # score gap scale * M * q: 20.5 bits in the log2 domain
    q = np.zeros((B, H, d), np.float16)
    q[:, :, 0::2] = np.float16(20.5 * np.log(2.0) / (scale * M))
    rk = rv = np.zeros((B, H, 0, d), np.float16)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, [hist] * B, rk, rv, [0] * B, scale)
    assert np.all(np.abs(ref_out + 1.0) > 5e-3), "the small weights must matter"
    pk, pv = oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap)
    out, lse = run_gpu_decode(dims_for(d, dsub, K, H, H), q, cbk, cbv, pk, pv, t_cap, [hist] * B, None, None,
                              [0] * B, scale)
    check_attention(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("B,H,hist", [(8, 32, 8192), (8, 32, 4096), (1, 2, 70000)])
def test_decode_identical_tokens_fill_one_cell(B, H, hist):
    """Every history token has the same K and V codes: all weights are equal and each
    (centroid, subspace) histogram cell of a split takes every token of it -- the largest
    a cell can get.  The result is the selected value centroids exactly, lse = s + ln T."""
    d, dsub, K = 128, 2, 4
    M = d // dsub
    t_cap = -(-hist // 64) * 64
    cbk = _codebook(11, H, K, M, dsub, 1.0)
    cbv = _codebook(12, H, K, M, dsub, 1.0)
    ck = np.full((B, H, t_cap, M), 1, np.uint8)
    cv = np.full((B, H, t_cap, M), 2, np.uint8)
    q = synthkv.small_normal(13, (B, H, d), np.float16)
    rk = rv = np.zeros((B, H, 0, d), np.float16)
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, [hist] * B, rk, rv, [0] * B, scale)
    pk, pv = oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap)
    out, lse = run_gpu_decode(dims_for(d, dsub, K, H, H), q, cbk, cbv, pk, pv, t_cap, [hist] * B, None, None,
                              [0] * B, scale)
    check_attention(out, lse, ref_out, ref_lse)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-5 * np.abs(ref_out).max())


@pytest.mark.parametrize("dsub", [2, 4])
def test_decode_large_magnitudes(dsub):
    """Queries 40x and codebooks 30x the unit scale (outlier-sized values, scores in the
    thousands): the softmax is sharply peaked and fp32 LUT sums carry large terms."""
    d, K, Hq, Hkv, r_cap = 128, 256, 8, 4, 32
    hist, rec = (3000, 9000), (32, 5)
    B, M = len(hist), d // dsub
    t_cap = -(-max(hist) // 64) * 64
    seed = 4040 + dsub
    q = (synthkv.small_normal(seed, (B, Hq, d)) * 40).astype(np.float16)
    cbk = _codebook(seed + 1, Hkv, K, M, dsub, 30.0)
    cbv = _codebook(seed + 2, Hkv, K, M, dsub, 30.0)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = (synthkv.small_normal(seed + 5, (B, Hkv, r_cap, d)) * 40).astype(np.float16)
    rv = (synthkv.small_normal(seed + 6, (B, Hkv, r_cap, d)) * 40).astype(np.float16)
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, hist, rk, rv, rec, scale)
    out, lse = run_gpu_decode(dims_for(d, dsub, K, Hq, Hkv), q, cbk, cbv, oracle.tile_codes(ck, t_cap),
                              oracle.tile_codes(cv, t_cap), t_cap, hist, rk, rv, rec, scale)
    check_attention(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("dsub,K", [(2, 256), (4, 256), (2, 100)], ids=["bounded-scan", "matrix-core", "direct-scan"])
def test_encode_strided_input(dsub, K):
    """Every encode kernel reads x through its strides: a view that skips every other token
    and whose head rows are padded (as a slice of a wider projection output) gives the codes
    of the contiguous copy, byte for byte, and those are the fp32 decision."""
    import torch

    import decode_attention_pq_amd as P

    d, H, N, ns = 128, 3, 1500, 2
    M = d // dsub
    t_cap = -(-N // 64) * 64
    rng = np.random.default_rng(4100 + K + dsub)
    x = rng.standard_normal((ns, N, H, d)).astype(np.float32)
    x[..., :3] *= 10.0
    x[rng.random(x.shape) < 0.01] *= 20.0
    x = x.astype(np.float16)
    cb = (np.random.default_rng(4200 + K).standard_normal((H, K, M, dsub)) * 3).astype(np.float32)
    dims = dims_for(d, dsub, K, H, H)
    wide = np.zeros((ns, 2 * N, H, d + 8), np.float16)
    wide[:, ::2, :, :d] = x
    view = to_dev(wide)[:, ::2, :, :d]
    assert not view.is_contiguous() and view.stride(1) == 2 * H * (d + 8) and view.stride(2) == d + 8
    cbd = to_dev(cb)
    planes = []
    for xin in (view, to_dev(x)):
        codes = torch.zeros((ns, H, t_cap * M), dtype=torch.uint8, device="cuda")
        P.encode(dims, xin, cbd, codes, t_cap)
        torch.cuda.synchronize()
        planes.append(codes.cpu().numpy())
    assert np.array_equal(planes[0], planes[1])
    for s in range(ns):
        ref, d1, d2, _ = oracle.encode(x[s], cb)
        got = oracle.untile_codes(planes[0][s], N, M).transpose(1, 0, 2)
        check_codes(got, x[s], cb, ref, d1, d2)


@pytest.mark.parametrize("hist,t_cap", [((3000,), 32768), ((100, 0, 7000), 20480), ((9000, 9000), 65536)],
                         ids=["one-sequence", "ragged", "equal-lengths"])
def test_decode_with_capacity_as_max_hist(hist, t_cap):
    """A serving loop passes its cache capacity as max_hist_len: the plan is then sized for
    the capacity, most splits hold no tokens and leave at once (one sequence), or the
    device-side plan resizes them from the actual lengths (2..16 sequences); the result is
    the attention over the actual lengths."""
    d, dsub, K, Hq, Hkv, R = 128, 2, 256, 8, 4, 16
    B, M = len(hist), d // dsub
    seed = 900 + sum(hist) + t_cap
    q = synthkv.small_normal(seed, (B, Hq, d), np.float16)
    cbk = _codebook(seed + 1, Hkv, K, M, dsub, 1.0)
    cbv = _codebook(seed + 2, Hkv, K, M, dsub, 1.0)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (B, Hkv, R, d), np.float16)
    rv = synthkv.small_normal(seed + 6, (B, Hkv, R, d), np.float16)
    rec = tuple(R - i for i in range(B))
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, hist, rk, rv, rec, scale)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    out, lse = run_gpu_decode(dims, q, cbk, cbv, oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap), t_cap,
                              hist, rk, rv, rec, scale, max_hist=t_cap)
    check_attention(out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("qdt,rdt", [(np.float16, np.float32), (np.float32, np.float16)], ids=["q16-r32", "q32-r16"])
@pytest.mark.parametrize("dsub,Hq,Hkv", [(2, 4, 4), (4, 8, 4)], ids=["mha-dsub2", "gqa-dsub4"])
def test_decode_mixed_q_and_recent_dtypes(qdt, rdt, dsub, Hq, Hkv):
    """q and the recent window take their dtypes independently (every combination is its
    own kernel build)."""
    d, K, R = 128, 256, 40
    hist, rec = (5000, 700), (40, 13)
    B, M = len(hist), d // dsub
    t_cap = -(-max(hist) // 64) * 64
    seed = 7100 + dsub + Hq
    q = synthkv.small_normal(seed, (B, Hq, d), qdt)
    cbk = _codebook(seed + 1, Hkv, K, M, dsub, 1.0)
    cbv = _codebook(seed + 2, Hkv, K, M, dsub, 1.0)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (B, Hkv, R, d), rdt)
    rv = synthkv.small_normal(seed + 6, (B, Hkv, R, d), rdt)
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, hist, rk, rv, rec, scale)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    out, lse = run_gpu_decode(dims, q, cbk, cbv, oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap), t_cap,
                              hist, rk, rv, rec, scale)
    check_attention(out, lse, ref_out, ref_lse)
