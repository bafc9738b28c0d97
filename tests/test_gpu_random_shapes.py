"""Seeded sweeps of random decode and encode shapes against the oracle.

Four hundred and eighty decode shapes drawn from one seed cover the combinations the
hand-written cases do not list: head size, subspace size, centroid count (2..256), kv and
query heads (groups of 1, 2, 4 and 8), batch 1..5 with independent history
lengths (empty, sub-tile, multi-split), recent windows from none to 300 rows,
fp16 and fp32.  Every case runs the HIP decode through the C ABI and compares
it with the dequantise-then-exact oracle at the usual tolerance.  Two hundred and
forty encode shapes (head size, subspace size, centroid counts with and without whole
blocks of 64, 1..3 heads, 1..4999 tokens at a random start, one or two
sequences, fp16 and fp32, outlier-heavy values) are compared code by code.
"""
import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, check_codes, dims_for, run_gpu_decode, run_gpu_encode, softmax_scale

pytestmark = pytest.mark.gpu


def _shapes(n=480, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        dsub = int(rng.choice([2, 4]))
        K = int(rng.choice([2, 7, 16, 64, 100, 255, 256]))
        Hkv = int(rng.integers(1, 5))
        g = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 6))
        kind = rng.integers(0, 4, size=B)
        hist = tuple(int(v) for v in np.where(kind == 0, 0, np.where(kind == 1, rng.integers(1, 64, B),
                                                                      rng.integers(64, 6000, B))))
        r_cap = int(rng.choice([0, 1, 8, 64, 300]))
        rec = tuple(int(v) for v in rng.integers(0, r_cap + 1, B)) if r_cap else (0,) * B
        dt = np.float16 if rng.random() < 0.7 else np.float32
        out.append((d, dsub, K, Hkv * g, Hkv, hist, rec, r_cap, dt))
    return out


@pytest.mark.parametrize("case", _shapes(), ids=lambda c: f"d{c[0]}s{c[1]}K{c[2]}h{c[3]}/{c[4]}b{len(c[5])}r{c[7]}")
def test_random_shape_decode(case):
    d, dsub, K, Hq, Hkv, hist, rec, r_cap, dt = case
    B, M = len(hist), d // dsub
    t_cap = max(64, -(-max(hist) // 64) * 64)
    seed = 7000 + sum(hist) + K + d + Hq
    q = synthkv.small_normal(seed, (B, Hq, d), dt)
    cbk = (synthkv.small_normal(seed + 1, (Hkv, K, M, dsub)) * 1.5).astype(np.float32)
    cbv = (synthkv.small_normal(seed + 2, (Hkv, K, M, dsub)) * 1.5).astype(np.float32)
    ck = synthkv.small_codes(seed + 3, (B, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (B, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (B, Hkv, max(r_cap, 1), d), dt)[:, :, :r_cap]
    rv = synthkv.small_normal(seed + 6, (B, Hkv, max(r_cap, 1), d), dt)[:, :, :r_cap]
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, hist, rk, rv, rec, scale)
    dims = dims_for(d, dsub, K, Hq, Hkv)
    out, lse = run_gpu_decode(dims, q, cbk, cbv, oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap), t_cap,
                              hist, np.ascontiguousarray(rk) if r_cap else None,
                              np.ascontiguousarray(rv) if r_cap else None, rec, scale)
    check_attention(out, lse, ref_out, ref_lse)


def _encode_shapes(n=240, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dsub = int(rng.choice([2, 4]))
        K = int(rng.choice([16, 37, 64, 128, 192, 200, 256]))
        H = int(rng.integers(1, 4))
        N = int(rng.integers(1, 5000))
        ns = int(rng.integers(1, 3))
        t_start = int(rng.integers(0, 100))
        dt = np.float16 if rng.random() < 0.6 else np.float32
        out.append((d, dsub, K, H, N, ns, t_start, dt, 3000 + i))
    return out


def _mfma_encode_shapes(seed=91):
    """d_sub 4 with 256 centroids (the matrix-core encode): token counts at the edges of a
    16-token group and of a work-group's 4096 tokens, and random ones."""
    rng = np.random.default_rng(seed)
    out = []
    for i, N in enumerate((1, 15, 16, 17, 4095, 4096, 4097, int(rng.integers(5000, 20000)))):
        d = (64, 128)[i % 2]
        H = int(rng.integers(1, 9))
        ns = int(rng.integers(1, 4)) if N < 5000 else 1
        t_start = int(rng.integers(0, 100))
        dt = np.float16 if i % 3 else np.float32
        out.append((d, 4, 256, H, N, ns, t_start, dt, 5000 + i))
    return out


@pytest.mark.parametrize("case", _encode_shapes() + _mfma_encode_shapes(),
                         ids=lambda c: f"d{c[0]}s{c[1]}K{c[2]}h{c[3]}n{c[4]}x{c[5]}t{c[6]}")
def test_random_shape_encode(case):
    d, dsub, K, H, N, ns, t_start, dt, seed = case
    M = d // dsub
    t_cap = -(-(t_start + N) // 64) * 64
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((ns, N, H, d)).astype(np.float32)
    x[..., :3] *= 10.0
    x[rng.random(x.shape) < 0.01] *= 20.0
    x = x.astype(dt)
    cb = (np.random.default_rng(seed + 1).standard_normal((H, K, M, dsub)) * 3).astype(np.float32)
    planes = run_gpu_encode(dims_for(d, dsub, K, H, H), x, cb, ns, t_cap, t_start)
    for s in range(ns):
        ref, d1, d2, _ = oracle.encode(x[s], cb)
        got = oracle.untile_codes(planes[s], t_start + N, M)[:, t_start:].transpose(1, 0, 2)
        check_codes(got, x[s], cb, ref, d1, d2)
