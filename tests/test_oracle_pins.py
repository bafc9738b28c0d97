"""Pins of the CPU oracle to things other than itself.

Each test ties an oracle function to what the MILLION page (the DAC 2025
write-up) or plain mathematics fixes: closed forms, the
page's stated figures, textbook special cases, library routines (scipy,
scikit-learn, torch) and brute force on tiny inputs.  A plausible mistake in
the oracle (a dropped term, a wrong sign or index, a transposed operand) should
fail at least one of them.
"""
import itertools
from fractions import Fraction
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _nearest_bruteforce(X, C):
    """Pure-Python nearest centroid, lowest index on exact ties."""
    out = []
    for x in X:
        best, bd = 0, None
        for c, cc in enumerate(C):
            d = sum((float(a) - float(b)) ** 2 for a, b in zip(x, cc))
            if bd is None or d < bd:
                best, bd = c, d
        out.append(best)
    return np.array(out)


# ------------------------------------------------------------------ O1 k-means
def test_lloyd_invariants(oracle_mod):
    rng = np.random.default_rng(7)
    X = rng.standard_normal((600, 2))
    X[:50] *= 8.0
    order = rng.permutation(600)
    iters = 8
    C, assign, trace, kept = oracle.kmeans(X, 16, iters, order)
    assert kept == 16
    # SSE never increases, through assignment and update steps alike
    assert np.all(np.diff(trace) <= 1e-12 * trace[0])
    # every non-empty centroid is the mean of the members of the last assignment
    for c in range(16):
        mem = X[assign == c]
        if len(mem):
            np.testing.assert_allclose(C[c], mem.mean(axis=0), rtol=0, atol=1e-12)
    # the last assignment is the nearest one for the centroids before the last update
    C_prev, _, _, _ = oracle.kmeans(X, 16, iters - 1, order)
    np.testing.assert_array_equal(assign, _nearest_bruteforce(X, C_prev))
    # initialisation: the first 16 points of the order (all distinct here)
    C0, a0, _, _ = oracle.kmeans(X, 16, 0, order)
    np.testing.assert_array_equal(C0, X[order[:16]])
    np.testing.assert_array_equal(a0, _nearest_bruteforce(X, C0))


def test_kmeans_fig4_line8_bruteforce(oracle_mod):
    """Fig. 4 setting: 8 points, 2 bits.  Optimal 1-D k-means clusters are
    contiguous in sorted order, so enumerating the C(7,3)=35 cut sets gives the
    optimum.  Lloyd's best over every initial subset reaches it, the optimum's
    means are a Lloyd fixed point, and uniform 2-bit quantisation leaves code
    10 unused while the clustering uses all four codes."""
    g = _golden("fig4_line8.json")
    pts = np.array(g["points"], dtype=np.float64)
    K = g["n_clusters"]
    xs = np.sort(pts)
    best_sse, best_part = math.inf, None
    for cuts in itertools.combinations(range(1, len(xs)), K - 1):
        bounds = (0,) + cuts + (len(xs),)
        parts = [xs[bounds[i]:bounds[i + 1]] for i in range(K)]
        sse = sum(float(((p - p.mean()) ** 2).sum()) for p in parts)
        if sse < best_sse:
            best_sse, best_part = sse, parts
    assert abs(best_sse - g["optimal_sse_by_hand"]) < 1e-12
    assert [list(p) for p in best_part] == g["optimal_partition_by_hand"]
    X = pts[:, None]
    # Lloyd never beats the optimum; from some initial subset it reaches it
    lloyd_best = math.inf
    for init in itertools.combinations(range(8), K):
        order = np.array(list(init) + [i for i in range(8) if i not in init])
        C, assign, trace, _ = oracle.kmeans(X, K, 20, order)
        final = float(((X[:, 0] - C[assign, 0]) ** 2).sum())
        assert final >= best_sse - 1e-12
        lloyd_best = min(lloyd_best, final)
    assert abs(lloyd_best - best_sse) < 1e-12
    # the optimum's means are a fixed point of Lloyd
    means = np.array([[p.mean()] for p in best_part])
    C, assign, _ = oracle.lloyd(X, means, 3)
    np.testing.assert_array_equal(C, means)
    assert len(set(assign.tolist())) == 4
    # uniform 2-bit quantisation over [min, max] leaves level 2 (code 10) empty
    step = (pts.max() - pts.min()) / 4
    uni = np.minimum(((pts - pts.min()) / step).astype(int), 3)
    assert uni.tolist() == g["uniform_codes_by_hand"]
    assert 2 not in set(uni.tolist())


def test_kmeans_distinct_points_equal_k(oracle_mod):
    """When the data has exactly K distinct points, k-means keeps them all: SSE 0."""
    rng = np.random.default_rng(3)
    P = rng.standard_normal((12, 4))
    X = P[rng.integers(0, 12, size=300)]
    X[:12] = P  # every distinct point present
    C, assign, trace, kept = oracle.kmeans(X, 12, 10, rng.permutation(300))
    assert kept == 12
    # the mean of n equal values is that value up to the rounding of sum/n
    assert trace[-1] < 1e-24
    np.testing.assert_allclose(np.array(sorted(map(tuple, C))), np.array(sorted(map(tuple, P))),
                               rtol=1e-15, atol=1e-15)


def test_kmeans_fewer_distinct_than_k(oracle_mod):
    """Fewer distinct points than K: the remaining slots copy slot 0 and stay empty."""
    X = np.array([[1.0, 2.0]] * 5 + [[3.0, -1.0]] * 4)
    C, assign, trace, kept = oracle.kmeans(X, 4, 3, np.arange(9))
    assert kept == 2
    np.testing.assert_array_equal(C[2], C[0])
    np.testing.assert_array_equal(C[3], C[0])
    assert set(assign.tolist()) == {0, 1}
    assert trace[-1] == 0.0


def test_kmeans_matches_sklearn_lloyd(oracle_mod):
    """Library pin: scikit-learn's Lloyd from the same initial centroids."""
    from sklearn.cluster import KMeans

    rng = np.random.default_rng(11)
    centers = rng.standard_normal((8, 2)) * 6
    X = centers[rng.integers(0, 8, size=800)] + rng.standard_normal((800, 2))
    C0 = X[:8].copy()
    order = np.arange(800)
    for iters in (1, 3, 30):
        C, _, _, _ = oracle.kmeans(X, 8, iters, order)
        km = KMeans(n_clusters=8, init=C0, n_init=1, max_iter=iters, tol=0.0, algorithm="lloyd")
        km.fit(X)
        np.testing.assert_allclose(C, km.cluster_centers_, rtol=0, atol=1e-9)


def test_fit_codebooks_layout(oracle_mod):
    """fit_codebooks places subspace m of head h at cb[h, :, m, :] and equals
    per-subspace k-means on the same points and initial order."""
    rng = np.random.default_rng(5)
    N, H, d, dsub, K = 200, 3, 8, 2, 6
    x = rng.standard_normal((N, H, d)).astype(np.float32)
    M = d // dsub
    order = np.stack([np.stack([rng.permutation(N) for _ in range(M)]) for _ in range(H)])
    cb = oracle.fit_codebooks(x, dsub, K, 5, order)
    assert cb.shape == (H, K, M, dsub) and cb.dtype == np.float32
    for h in range(H):
        for m in range(M):
            C, _, _, _ = oracle.kmeans(x[:, h, m * dsub:(m + 1) * dsub].astype(np.float64), K, 5, order[h, m])
            np.testing.assert_array_equal(cb[h, :, m, :], C.astype(np.float32))


# ------------------------------------------------------------------ O2 encode
def test_encode_pure_python_tiny(oracle_mod):
    rng = np.random.default_rng(2)
    N, H, d, dsub, K = 9, 2, 6, 2, 5
    x = rng.standard_normal((N, H, d)).astype(np.float32)
    cb = rng.standard_normal((H, K, d // dsub, dsub)).astype(np.float32)
    cb[1, 3] = cb[1, 1]  # duplicate centroid: index 1 must win, flagged ambiguous
    x[4, 1, 0:2] = cb[1, 1, 0]  # exactly on the duplicated centroid
    codes, d1, d2, amb = oracle.encode(x, cb)
    for t in range(N):
        for h in range(H):
            for m in range(d // dsub):
                exp = _nearest_bruteforce([x[t, h, m * dsub:(m + 1) * dsub]], cb[h, :, m, :])[0]
                assert codes[t, h, m] == exp
    assert codes[4, 1, 0] == 1 and d1[4, 1, 0] == 0.0 and d2[4, 1, 0] == 0.0 and amb[4, 1, 0]
    assert np.all(amb[:, 1, :][codes[:, 1, :] == 1])  # every pick of the duplicate is ambiguous


def _sq_norm_f64(c):
    """Squared distance of the zero vector to centroid c, summed over j in order in
    fp64 (each square of an fp32 value is exact in fp64)."""
    s = 0.0
    for v in c:
        t = 0.0 - float(v)
        s += t * t
    return s


# fp32 values whose squared norm, summed in order in fp64, is exactly fl(1e-5): a runner-up
# at distance exactly 1e-5 * max(1, 0) from a best at distance 0
_EXACT_BAND = tuple(np.float32(float.fromhex(h)) for h in
                    ("0x1.9e772p-9", "0x1.08e4p-15", "0x1.c8d6d4p-20"))


def _band_case(best, runner_up):
    """x = 0 in 4 dimensions (one subspace of d_sub 4) and a codebook whose centroid 0
    is `best`, centroid 1 `runner_up` and centroids 2, 3 far away."""
    cb = np.zeros((1, 4, 1, 4), np.float32)
    cb[0, 0, 0, :len(best)] = best
    cb[0, 1, 0, :len(runner_up)] = runner_up
    cb[0, 2, 0, :] = 100.0
    cb[0, 3, 0, :] = -100.0
    return np.zeros((1, 1, 4), np.float32), cb


def test_encode_ambiguity_band_boundaries(oracle_mod):
    """The flag is D2 - D1 < 1e-5 * max(1, D1) (strict, relative to the best distance,
    floored at 1).  Constructed pairs at half and at twice the band for D1 = 0, 0.25, 1
    and 1000, one at exactly the band, and one just past the band at D1 = 1000 whose
    runner-up is inside 1e-5 * D2: together they fail an absolute 1e-5 or 1e-4 band, a
    band without the floor, '<=' for '<', and max(1, D2) for max(1, D1)."""
    f = np.float32
    cases = [
        # (best centroid, runner-up centroid, ambiguous?)
        ((0.0,), (f(np.sqrt(5e-6)),), True),            # D1 = 0: gap 0.5 band
        ((0.0,), (f(np.sqrt(2e-5)),), False),           # D1 = 0: gap 2 bands
        ((0.5,), (0.5, f(np.sqrt(5e-6))), True),        # D1 = 0.25: band 1e-5 (floor), gap 5e-6
        ((0.5,), (0.5, f(np.sqrt(2e-5))), False),       # D1 = 0.25: gap 2e-5 (inside a 1e-4 band)
        ((1.0,), (1.0, f(np.sqrt(5e-6))), True),        # D1 = 1
        ((1.0,), (1.0, f(np.sqrt(2e-5))), False),
        ((30.0, 10.0), (30.0, 10.0, f(np.sqrt(5e-3))), True),   # D1 = 1000: band 1e-2, gap 5e-3
        ((30.0, 10.0), (30.0, 10.0, f(np.sqrt(2e-2))), False),  # D1 = 1000: gap 2e-2
        ((0.0,), _EXACT_BAND, False),                   # D1 = 0, gap exactly fl(1e-5): '<' says no
        ((30.0, 10.0), (30.0, 10.0, f(0.1)), False),    # gap 1e-2 + 3e-10: past 1e-5 * D1, inside 1e-5 * D2
    ]
    assert _sq_norm_f64(_EXACT_BAND) == 1e-5
    for best, runner, want in cases:
        x, cb = _band_case(best, runner)
        codes, d1, d2, amb = oracle.encode(x, cb)
        e1, e2 = _sq_norm_f64(cb[0, 0, 0]), _sq_norm_f64(cb[0, 1, 0])
        assert codes[0, 0, 0] == 0 and d1[0, 0, 0] == e1 and d2[0, 0, 0] == e2, (best, runner)
        assert bool(amb[0, 0, 0]) == want, (best, runner, e1, e2)
        # the same pair with the two centroids swapped: the code follows the best one
        cb2 = cb[:, [1, 0, 2, 3]].copy()
        codes2, d1b, d2b, amb2 = oracle.encode(x, cb2)
        assert codes2[0, 0, 0] == 1 and d1b[0, 0, 0] == e1 and bool(amb2[0, 0, 0]) == want
    # the band boundaries the mistaken readings would give, on the same pairs
    b0 = _sq_norm_f64(_EXACT_BAND)
    assert not (b0 - 0.0 < 1e-5 * max(1.0, 0.0)) and (b0 - 0.0 <= 1e-5 * max(1.0, 0.0))
    e1, e2 = 1000.0, _sq_norm_f64((30.0, 10.0, f(0.1)))
    assert not (e2 - e1 < 1e-5 * max(1.0, e1)) and (e2 - e1 < 1e-5 * max(1.0, e2))


def test_encode_matches_scipy_vq(oracle_mod):
    """Library pin: scipy's vector quantiser (nearest code by Euclidean distance)."""
    from scipy.cluster.vq import vq

    rng = np.random.default_rng(9)
    N, H, d, dsub, K = 500, 2, 16, 4, 64
    x = (rng.standard_normal((N, H, d)) * 3).astype(np.float32)
    cb = rng.standard_normal((H, K, d // dsub, dsub)).astype(np.float32) * 3
    codes, d1, d2, amb = oracle.encode(x, cb)
    for h in range(H):
        for m in range(d // dsub):
            ref, dist = vq(x[:, h, m * dsub:(m + 1) * dsub].astype(np.float64), cb[h, :, m, :].astype(np.float64))
            ok = ~amb[:, h, m]
            np.testing.assert_array_equal(codes[:, h, m][ok], ref[ok])
            np.testing.assert_allclose(np.sqrt(d1[:, h, m]), dist, rtol=1e-12, atol=1e-12)


def test_encode_complete_codebook_roundtrip(oracle_mod):
    """A codebook holding every distinct subvector: decode(encode(x)) == x exactly."""
    levels = (-1.5, -0.5, 0.5, 1.5)
    x = synthkv.grid_values(21, (300, 2, 8), levels)
    grid = np.array(list(itertools.product(levels, repeat=2)), dtype=np.float32)  # 16 two-vectors
    perm = np.random.default_rng(1).permutation(16)
    cb = np.broadcast_to(grid[perm][None, :, None, :], (2, 16, 4, 2)).copy()
    codes, d1, d2, amb = oracle.encode(x, cb)
    assert np.all(d1 == 0.0) and not amb.any()
    np.testing.assert_array_equal(oracle.dequantize(codes, cb), x.astype(np.float64))


def test_encode_permutation_equivariance(oracle_mod):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((400, 2, 8)).astype(np.float32)
    cb = rng.standard_normal((2, 32, 4, 2)).astype(np.float32)
    perm = rng.permutation(32)
    inv = np.argsort(perm)
    c1, _, _, amb = oracle.encode(x, cb)
    c2, _, _, _ = oracle.encode(x, cb[:, perm])
    ok = ~amb
    np.testing.assert_array_equal(inv[c1][ok], c2[ok])


def test_code_distance_consistent(oracle_mod):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 2, 8)).astype(np.float32)
    cb = rng.standard_normal((2, 8, 4, 2)).astype(np.float32)
    codes, d1, _, _ = oracle.encode(x, cb)
    np.testing.assert_array_equal(oracle.code_distance(x, cb, codes), d1)
    other = (codes.astype(int) + 1) % 8
    assert np.all(oracle.code_distance(x, cb, other.astype(np.uint8)) >= d1)


# ------------------------------------------------------------------ O2 encode, fp32 decision
def _round_f32(q: Fraction) -> float:
    """An exact rational rounded to the nearest fp32 value, ties to even (IEEE 754
    round-to-nearest), returned as a Python float (exact)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = -q if q < 0 else q
    e = a.numerator.bit_length() - a.denominator.bit_length()  # floor(log2 a) or one above
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)  # subnormals: the smallest normal exponent, fewer significant bits
    scale = Fraction(2) ** (23 - e)
    m = a * scale
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = Fraction(n) / scale
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def _sqdist_f32_exact(x, c) -> float:
    """fp32 squared distance from exact arithmetic: each difference rounded to fp32, each
    square added to the running sum with one rounding (a fused multiply-add)."""
    d = Fraction(0)
    for a, b in zip(x, c):
        e = _round_f32(Fraction(float(a)) - Fraction(float(b)))
        d = Fraction(_round_f32(Fraction(e) * Fraction(e) + d))
    return float(d)


def test_encode_f32_distance_is_exactly_rounded(oracle_mod):
    """The fp32 distance, against exact rational arithmetic rounded to fp32 at each step,
    over magnitudes from 1e-3 to 1e3 (including cancellation and exact zeros)."""
    rng = np.random.default_rng(21)
    for dsub in (2, 4):
        for _ in range(400):
            mag = 10.0 ** rng.uniform(-3, 3)
            x = (rng.standard_normal(dsub) * mag).astype(np.float32)
            c = (x + rng.standard_normal(dsub).astype(np.float32) * np.float32(10.0 ** rng.uniform(-6, 0) * mag)
                 ).astype(np.float32)
            if rng.random() < 0.1:
                c[0] = x[0]  # an exact zero difference
            got = oracle.sqdist_f32(x, c)
            assert got == _sqdist_f32_exact(x, c), (x, c)


def test_encode_f32_bruteforce_tiny(oracle_mod):
    """Codes: the first centroid with a strictly smaller fp32 distance, by brute force over
    the exact-rounding model (with duplicate centroids, so exact ties occur)."""
    rng = np.random.default_rng(22)
    for dsub, K in ((2, 16), (4, 12)):
        H, M = 2, 3
        cb = rng.integers(-3, 4, size=(H, K, M, dsub)).astype(np.float32) * np.float32(0.5)
        cb[:, K - 1] = cb[:, 2]  # a duplicate of centroid 2 at the end
        x = (rng.integers(-6, 7, size=(40, H, M * dsub)) * 0.25).astype(np.float32)
        got = oracle.encode_f32(x, cb)
        for t in range(40):
            for h in range(H):
                for m in range(M):
                    xs = x[t, h, m * dsub:(m + 1) * dsub]
                    best, bd = 0, math.inf
                    for c in range(K):
                        dc = _sqdist_f32_exact(xs, cb[h, c, m])
                        if dc < bd:
                            best, bd = c, dc
                    assert got[t, h, m] == best, (t, h, m)


def test_encode_f32_equals_f64_outside_the_band(oracle_mod):
    """Where the fp64 decision is clear (runner-up beyond the 1e-5 band), the fp32 decision
    is the same code: outlier-bearing data, d_sub 2 and 4, 256 centroids."""
    rng = np.random.default_rng(23)
    for dsub in (2, 4):
        x = rng.standard_normal((3000, 2, 32)).astype(np.float32)
        x[:, :, 5] *= 10.0  # a channel outlier
        x[rng.random(x.shape) < 0.005] *= 20.0  # point outliers
        cb = rng.standard_normal((2, 256, 32 // dsub, dsub)).astype(np.float32)
        c32 = oracle.encode_f32(x, cb)
        c64, _, _, amb = oracle.encode(x, cb)
        assert not ((c32 != c64) & ~amb).any()


def test_encode_f32_special_cases(oracle_mod):
    # a near tie that only fp32 rounding decides: |(1, 2^-13)|^2 = 1 + 2^-26 rounds to 1,
    # so centroid 0 ties centroid 1 in fp32 and the lower index wins; fp64 picks 1
    x = np.zeros((1, 1, 2), np.float32)
    cb = np.array([[[[1.0, 2.0 ** -13]], [[1.0, 0.0]]]], np.float32)
    assert oracle.encode_f32(x, cb)[0, 0, 0] == 0
    assert oracle.encode(x, cb)[0][0, 0, 0] == 1
    # exact duplicates: the lowest index
    cb = np.array([[[[3.0, 1.0]], [[1.0, 1.0]], [[1.0, 1.0]]]], np.float32)
    assert oracle.encode_f32(np.ones((1, 1, 2), np.float32), cb)[0, 0, 0] == 1
    # a NaN centroid never wins; a NaN or infinite subvector gets code 0
    cb = np.array([[[[np.nan, 0.0]], [[5.0, 5.0]], [[1.0, 1.0]]]], np.float32)
    assert oracle.encode_f32(np.ones((1, 1, 2), np.float32), cb)[0, 0, 0] == 2
    assert oracle.encode_f32(np.full((1, 1, 2), np.nan, np.float32), cb)[0, 0, 0] == 0
    assert oracle.encode_f32(np.full((1, 1, 2), np.inf, np.float32), cb)[0, 0, 0] == 0


# ------------------------------------------------------------------ O3/O4 attention
def _case(seed, B=2, Hq=4, Hkv=2, d=16, dsub=2, K=8, T=(37, 5), R=(3, 0), Tcap=64, Rcap=4):
    rng = np.random.default_rng(seed)
    M = d // dsub
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    cbk = rng.standard_normal((Hkv, K, M, dsub)).astype(np.float32)
    cbv = rng.standard_normal((Hkv, K, M, dsub)).astype(np.float32)
    ck = rng.integers(0, K, size=(B, Hkv, Tcap, M)).astype(np.uint8)
    cv = rng.integers(0, K, size=(B, Hkv, Tcap, M)).astype(np.uint8)
    rk = rng.standard_normal((B, Hkv, Rcap, d)).astype(np.float32)
    rv = rng.standard_normal((B, Hkv, Rcap, d)).astype(np.float32)
    return dict(q=q, cb_k=cbk, cb_v=cbv, codes_k=ck, codes_v=cv, hist_len=np.array(T, np.int32),
                recent_k=rk, recent_v=rv, recent_len=np.array(R, np.int32), scale=1.0 / math.sqrt(d))


def _dequant_head(codes, cb_head):
    """codes [T, M], cb_head [K, M, dsub] -> [T, M*dsub] by direct indexing."""
    T, M = codes.shape
    return cb_head[codes, np.arange(M)[None, :]].reshape(T, -1).astype(np.float64)


def test_decode_exact_matches_torch_sdpa(oracle_mod):
    """Library pin: torch's scaled_dot_product_attention (fp64, CPU) over the
    dequantised history followed by the recent tokens; lse via logsumexp."""
    c = _case(12)
    out, lse = oracle.decode_exact(**c)
    B, Hq, d = c["q"].shape
    g = Hq // c["cb_k"].shape[0]
    for b in range(B):
        T, R = int(c["hist_len"][b]), int(c["recent_len"][b])
        for hq in range(Hq):
            h = hq // g
            keys = np.concatenate([_dequant_head(c["codes_k"][b, h, :T], c["cb_k"][h]),
                                   c["recent_k"][b, h, :R].astype(np.float64)])
            vals = np.concatenate([_dequant_head(c["codes_v"][b, h, :T], c["cb_v"][h]),
                                   c["recent_v"][b, h, :R].astype(np.float64)])
            qt = torch.from_numpy(c["q"][b, hq].astype(np.float64))[None, None, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, torch.from_numpy(keys)[None, None], torch.from_numpy(vals)[None, None],
                scale=c["scale"])[0, 0, 0].numpy()
            np.testing.assert_allclose(out[b, hq], ref, rtol=1e-12, atol=1e-12)
            s = torch.from_numpy(keys) @ qt[0, 0, 0] * c["scale"]
            assert abs(lse[b, hq] - torch.logsumexp(s, 0).item()) < 1e-12


def test_decode_exact_special_cases(oracle_mod):
    c = _case(13, B=3, T=(1, 0, 0), R=(0, 3, 0))
    out, lse = oracle.decode_exact(**c)
    g = c["q"].shape[1] // c["cb_k"].shape[0]
    for hq in range(c["q"].shape[1]):
        h = hq // g
        # one history token, no recent: out is its dequantised value, lse its score
        v0 = _dequant_head(c["codes_v"][0, h, :1], c["cb_v"][h])[0]
        k0 = _dequant_head(c["codes_k"][0, h, :1], c["cb_k"][h])[0]
        np.testing.assert_array_equal(out[0, hq], v0)
        assert abs(lse[0, hq] - c["scale"] * float(k0 @ c["q"][0, hq].astype(np.float64))) < 1e-13
        # no history: plain softmax attention over the recent tokens
        s = c["scale"] * (c["recent_k"][1, h, :3].astype(np.float64) @ c["q"][1, hq].astype(np.float64))
        p = np.exp(s - s.max())
        np.testing.assert_allclose(out[1, hq], p @ c["recent_v"][1, h, :3] / p.sum(), rtol=1e-13, atol=1e-14)
        # nothing cached: zeros and -inf
        assert np.all(out[2, hq] == 0.0) and lse[2, hq] == -math.inf


def test_decode_exact_softmax_shift_invariance(oracle_mod):
    """Adding a constant to every centroid's projection on q shifts all scores
    equally: out unchanged, lse shifted by exactly that amount."""
    c = _case(14, B=1, Hq=2, Hkv=2, T=(20,), R=(0,), Rcap=1)
    out1, lse1 = oracle.decode_exact(**c)
    c2 = dict(c)
    # raise every key by a multiple of q_hat along its first subspace: not generic; instead scale q
    c2["scale"] = c["scale"] * 2.0
    out2, lse2 = oracle.decode_exact(**c2)
    c3 = dict(c)
    c3["q"] = c["q"] * 2.0
    out3, lse3 = oracle.decode_exact(**c3)
    np.testing.assert_allclose(out2, out3, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse3, rtol=1e-12, atol=1e-13)
    assert not np.allclose(out1, out2)


# ------------------------------------------------------------------ O5 method algebra
def test_lut_identity(oracle_mod):
    """ad-LUT identity (Fig. 7 paragraph): summing table entries over a token's
    codes gives the inner product of q with the dequantised key."""
    c = _case(15, B=2, Hq=4, Hkv=2, d=32, dsub=4, K=16, T=(50, 64))
    L = oracle.lut(c["q"], c["cb_k"], 2)
    assert L.shape == (2, 4, 8, 16)
    for b in range(2):
        for hq in range(4):
            h = hq // 2
            s = oracle.lut_scores(L[b, hq], c["codes_k"][b, h], c["scale"])
            keys = _dequant_head(c["codes_k"][b, h], c["cb_k"][h])
            ref = c["scale"] * (keys @ c["q"][b, hq].astype(np.float64))
            assert np.all(np.abs(s - ref) <= 1e-12 * (1 + np.abs(ref)))
    # a single entry by hand: q subvector m . centroid c
    m, cc = 3, 5
    hand = sum(float(c["q"][1, 3, m * 4 + j]) * float(c["cb_k"][1, cc, m, j]) for j in range(4))
    assert abs(L[1, 3, m, cc] - hand) < 1e-14


def test_histogram_identity(oracle_mod):
    """Per-subspace histograms of softmax weights times the value codebook equal
    the softmax-weighted sum of dequantised values."""
    rng = np.random.default_rng(16)
    T, M, dsub, K = 300, 8, 2, 16
    s = rng.standard_normal(T) * 3
    cv = rng.integers(0, K, size=(T, M)).astype(np.uint8)
    cbv = rng.standard_normal((K, M, dsub))
    mu, l, o = oracle.hist_partial(s, cv, cbv)
    p = np.exp(s - s.max())
    ref = p @ _dequant_head(cv, cbv)
    assert mu == s.max() and abs(l - p.sum()) < 1e-12 * p.sum()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_method_equals_exact_any_partition(oracle_mod):
    """LSE-merge closed form: any split of the history into contiguous parts,
    plus the recent window, merges to the exact attention result."""
    c = _case(17, B=2, Hq=8, Hkv=2, d=16, dsub=2, K=32, T=(200, 1), R=(4, 2), Tcap=256, Rcap=4)
    ref_out, ref_lse = oracle.decode_exact(**c)
    rng = np.random.default_rng(0)
    for n_split in (1, 2, 7, 64):
        def bounds(b, T, n=n_split):
            if T == 0:
                return [0]
            cuts = np.sort(rng.choice(np.arange(1, max(T, 2)), size=min(n - 1, max(T - 1, 0)), replace=False))
            return [0] + cuts.tolist()
        out, lse = oracle.decode_method(**c, split_bounds=bounds)
        np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_merge_states_closed_form(oracle_mod):
    rng = np.random.default_rng(18)
    n, d = 5, 8
    sa, sb = rng.standard_normal((n, 6)), rng.standard_normal((n, 4))
    va, vb = rng.standard_normal((n, 6, d)), rng.standard_normal((n, 4, d))

    def state(s, v):
        p = np.exp(s - s.max(1, keepdims=True))
        return np.einsum("ns,nsd->nd", p, v) / p.sum(1, keepdims=True), np.log(np.exp(s).sum(1))

    oa, la = state(sa, va)
    ob, lb = state(sb, vb)
    of, lf = state(np.concatenate([sa, sb], 1), np.concatenate([va, vb], 1))
    out, lse = oracle.merge_states(oa, la, ob, lb)
    np.testing.assert_allclose(out, of, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lf, rtol=1e-13, atol=1e-13)
    lb2 = lb.copy()
    lb2[1] = -np.inf  # an empty side has weight zero
    out, lse = oracle.merge_states(oa, la, ob, lb2)
    np.testing.assert_array_equal(out[1], oa[1])
    assert lse[1] == la[1]
    out, lse = oracle.merge_states(oa[:1], [-np.inf], ob[:1], [-np.inf])
    assert np.all(out == 0) and lse[0] == -np.inf


def test_complete_codebook_pq_attention_is_exact(oracle_mod):
    """K/V elements drawn from 4 levels give exactly 16 distinct 2-vectors per
    subspace; k-means with K=16 on that data recovers all of them, so PQ
    attention equals exact attention on the original K/V (torch SDPA, fp64)."""
    levels = (-1.5, -0.5, 0.5, 1.5)
    H, d, dsub, K, T, R = 4, 64, 2, 16, 512, 16
    M = d // dsub
    kx = synthkv.grid_values(31, (T, H, d), levels)
    vx = synthkv.grid_values(32, (T, H, d), levels)
    order = np.stack([np.stack([np.random.default_rng(100 + h * M + m).permutation(T) for m in range(M)])
                      for h in range(H)])
    cbk = oracle.fit_codebooks(kx, dsub, K, 10, order)
    cbv = oracle.fit_codebooks(vx, dsub, K, 10, order)
    ck, d1k, _, _ = oracle.encode(kx, cbk)
    cv, d1v, _, _ = oracle.encode(vx, cbv)
    assert np.all(d1k == 0) and np.all(d1v == 0)
    q = synthkv.small_normal(33, (1, H, d))
    rk = synthkv.small_normal(34, (1, H, R, d))
    rv = synthkv.small_normal(35, (1, H, R, d))
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = oracle.decode_exact(q, cbk, cbv, ck.transpose(1, 0, 2)[None], cv.transpose(1, 0, 2)[None],
                                   [T], rk, rv, [R], scale)
    for h in range(H):
        keys = np.concatenate([kx[:, h].astype(np.float64), rk[0, h].astype(np.float64)])
        vals = np.concatenate([vx[:, h].astype(np.float64), rv[0, h].astype(np.float64)])
        qt = torch.from_numpy(q[0, h].astype(np.float64))[None, None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, torch.from_numpy(keys)[None, None], torch.from_numpy(vals)[None, None], scale=scale)
        np.testing.assert_allclose(out[0, h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ O6 accounting
def test_compression_ratio_matches_page(oracle_mod):
    g = _golden("pages_figures.json")
    cr = g["kv_compression_ratio"]
    assert oracle.compression_ratio(128, cr["d_sub"], cr["code_bits"]) == cr["value"] == 4
    assert oracle.compression_ratio(128, 4) == 8
    assert oracle.compression_ratio(64, 2) == 4
    # measured on real buffers: codes of a token-head versus its fp16 vector
    w = synthkv.WORKLOADS["llama2_7b_32k"]
    x = synthkv.kv_values(w, 0, "k", "history", 64)
    codes = np.zeros((64, w.n_kv_heads, w.n_sub), np.uint8)
    assert x.dtype == np.float16 and x.nbytes / codes.nbytes == 4
    assert g["subspace_dims"]["value"] == [2, 4]


def test_kv_cache_size_matches_page(oracle_mod):
    g = _golden("pages_figures.json")["llama2_7b_kv_fp16_at_128k"]
    s = g["shape"]
    total = oracle.kv_cache_bytes_fp16(s["n_layers"], s["n_kv_heads"], s["head_dim"], s["n_tokens"])
    assert total == 2 ** 36 and total / 2 ** 30 == g["value_gb"]
    assert oracle.kv_cache_bytes_fp16(32, 32, 128, 1) == 524288
    # PQ codes at d_sub=2 take a quarter of it
    assert total / oracle.compression_ratio(128, 2) == 16 * 2 ** 30
    assert oracle.codebook_bytes(32, 256, 128) == 8 * 2 ** 20


# ------------------------------------------------------------------ code layout
@pytest.mark.parametrize("M", [16, 32, 64])
def test_code_layout_bijection_and_roundtrip(oracle_mod, M):
    t_cap = 192
    off = oracle.code_offsets(M, t_cap)
    assert sorted(off.ravel().tolist()) == list(range(t_cap * M))
    # brute force against the definition, loop by loop
    for t in range(0, t_cap, 7):
        lane = t % 64
        for p in range(M):
            m = (p + lane) % M
            assert off[t, m] == (t // 64) * 64 * M + (p // 16) * 1024 + lane * 16 + p % 16
    codes = synthkv.small_codes(40 + M, (2, 3, 150, M), 256)
    planes = oracle.tile_codes(codes, t_cap)
    np.testing.assert_array_equal(oracle.untile_codes(planes, 150, M), codes)


def test_generator_deterministic_and_shaped():
    w = synthkv.WORKLOADS["llama2_7b_32k"]
    a = synthkv.kv_values(w, 0, "k", "history", 256)
    b = synthkv.kv_values(w, 0, "k", "history", 256)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (256, 32, 128) and a.dtype == np.float16
    # outlier structure: 4 channels per head scaled x10, ~0.5% points x20
    ch = synthkv.outlier_channels(w, 0, "k")
    assert ch.shape == (32, 4) and all(len(set(r)) == 4 for r in ch.tolist())
    big = np.abs(a.astype(np.float32)).mean(axis=0)  # [H, d]
    for h in range(32):
        assert set(np.argsort(big[h])[-4:].tolist()) == set(ch[h].tolist())
    assert synthkv.WORKLOADS["full32_ragged4"].hist_len == (14698, 3634, 31436, 30564)
    v = synthkv.kv_values(w, 0, "v", "history", 256)
    assert not np.array_equal(a, v)


def test_generator_chunks_draw_alone():
    """A sample of 1024-token chunks, drawn alone, equals the same tokens of the whole
    draw (ragged last chunk included); the sample is seeded and 1/8 of the chunks."""
    w = synthkv.WORKLOADS["full32_ragged4"]
    n = 5000
    full = synthkv.kv_values(w, 3, "v", "history", n, 1)
    part = synthkv.kv_values(w, 3, "v", "history", n, 1, chunks=[1, 4])
    np.testing.assert_array_equal(part, full[synthkv.chunk_tokens([1, 4], n)])
    assert part.shape[0] == 1024 + (n - 4096)
    ch = synthkv.sample_chunks(11, 31436)
    assert ch == synthkv.sample_chunks(11, 31436) and len(ch) == 4 and ch == sorted(set(ch))
    assert len(synthkv.sample_chunks(11, 1000)) == 1


def test_numpy_mini_oracle_rederives_tiny(oracle_mod):
    """The Tiny workload computed twice, by the C oracle and by the NumPy mini-oracle
    (oracle/mini.py, written apart from it): the same fp32 codebooks bit for bit (same
    operations in the same order), the same codes and best distances, and the same
    attention within 1e-12."""
    from oracle import mini

    w = synthkv.WORKLOADS["tiny"]
    cbs, codes = {}, {}
    for tensor in ("k", "v"):
        values = synthkv.calibration_kv(w, 0, tensor)
        order = synthkv.init_order(w, 0, tensor, values.shape[0])
        cb_c = oracle.fit_codebooks(values, w.d_sub, w.n_centroids, w.kmeans_iters, order)
        cb_n = mini.fit_codebooks(values, w.d_sub, w.n_centroids, w.kmeans_iters, order)
        np.testing.assert_array_equal(cb_c.view(np.uint32), cb_n.view(np.uint32))
        x = synthkv.history_kv(w, 0, tensor, 0)
        c_c, d1, _, _ = oracle.encode(x, cb_c)
        c_n, d_n = mini.encode(x, cb_n)
        np.testing.assert_array_equal(c_c, c_n)
        np.testing.assert_array_equal(d1, d_n)
        cbs[tensor], codes[tensor] = cb_c, c_c.transpose(1, 0, 2)  # [H, T, M]
    q = synthkv.queries(w)
    rk, rv = synthkv.recent_kv(w, 0, "k"), synthkv.recent_kv(w, 0, "v")
    scale = float(np.float32(1.0 / np.sqrt(w.head_dim)))
    ref_out, ref_lse = oracle.decode_exact(q, cbs["k"], cbs["v"], codes["k"][None], codes["v"][None], w.hist_len,
                                           rk, rv, [w.recent_len], scale)
    out, lse = mini.decode(q[0], cbs["k"], cbs["v"], codes["k"], codes["v"], rk[0], rv[0], scale)
    np.testing.assert_allclose(out, ref_out[0], rtol=0, atol=1e-12 * np.abs(ref_out).max())
    np.testing.assert_allclose(lse, ref_lse[0], rtol=1e-12, atol=0)


# ------------------------------------------------------------------ O7 live-cache step
@pytest.mark.parametrize("r_cap,n_roll", [(5, 3), (4, 4), (3, 1)])
def test_append_step_equals_bulk_quantisation(oracle_mod, r_cap, n_roll):
    """Batched, delayed quantisation moves tokens, it does not change them: after
    any number of steps the history is the starting codes followed by the
    pure-Python nearest codes of the oldest appended tokens, in order, and the
    window holds the newest ones.  How many tokens have rolled follows from the
    window arithmetic alone (an integer simulation of the lengths)."""
    B, H, d, dsub, K, steps = 2, 2, 8, 2, 8, 23
    M = d // dsub
    cbk = synthkv.small_normal(41, (H, K, M, dsub))
    cbv = synthkv.small_normal(42, (H, K, M, dsub))
    start_codes = [np.zeros((0, H, M), np.uint8), synthkv.small_codes(43, (4, H, M), K)]
    start_rk = [synthkv.small_normal(44, (0, H, d)), synthkv.small_normal(45, (r_cap, H, d))]
    start_rv = [synthkv.small_normal(46, (0, H, d)), synthkv.small_normal(47, (r_cap, H, d))]
    state = {"codes_k": list(start_codes), "codes_v": list(start_codes),
             "amb_k": [np.zeros(c.shape, bool) for c in start_codes],
             "amb_v": [np.zeros(c.shape, bool) for c in start_codes],
             "recent_k": list(start_rk), "recent_v": list(start_rv)}
    new_k = synthkv.small_normal(48, (steps, B, H, d))
    new_v = synthkv.small_normal(49, (steps, B, H, d))
    for s in range(steps):
        state = oracle.append_kv_step(state, new_k[s], new_v[s], cbk, cbv, r_cap, n_roll)
    for b in range(B):
        R, rolled = start_rk[b].shape[0], 0
        for _ in range(steps):
            if R == r_cap:
                R, rolled = R - n_roll, rolled + n_roll
            R += 1
            assert R <= r_cap
        for t_name, cb, start_r, new in (("k", cbk, start_rk, new_k), ("v", cbv, start_rv, new_v)):
            tokens = np.concatenate([start_r[b], new[:, b]], axis=0)  # every row that entered the window
            assert state["recent_" + t_name][b].shape[0] == R
            np.testing.assert_array_equal(state["recent_" + t_name][b], tokens[rolled:])
            codes = state["codes_" + t_name][b]
            assert codes.shape[0] == start_codes[b].shape[0] + rolled
            np.testing.assert_array_equal(codes[:start_codes[b].shape[0]], start_codes[b])
            for h in range(H):
                for m in range(M):
                    want = _nearest_bruteforce(tokens[:rolled, h, m * dsub:(m + 1) * dsub], cb[h, :, m])
                    np.testing.assert_array_equal(codes[start_codes[b].shape[0]:, h, m], want)
