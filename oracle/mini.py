"""NumPy mini-oracle: the Tiny workload re-derived with NumPy alone, independent of
the C oracle (oracle.c), as a cross-check of it.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the tests import it.

It follows the same definitions, written again with array operations:
  * Lloyd k-means per subspace (the Fig. 5 paragraph's clustering; the paragraph
    after it: one codebook per subspace of dimension d_sub; the Fig. 6 paragraph:
    offline training): distinct-point initialisation along a given order, then
    assignment to the nearest centroid (lowest index on ties) and update to the
    member mean (an empty cluster keeps its centroid), in fp64, rounded to fp32;
  * brute-force encode (the Fig. 6 paragraph: the prefill is quantised with the
    trained codebooks): squared distances in fp64, code = first index of the minimum;
  * exact attention over the dequantised history and the recent window (the Fig. 7
    paragraph: the two parts of one softmax attention), in fp64.
"""
from __future__ import annotations

import numpy as np


def kmeans(X, K: int, iters: int, order):
    """X [n, dsub] (fp64); order: a permutation of the points.  Returns fp64 [K, dsub]."""
    X = np.asarray(X, np.float64)
    kept = []
    for i in order:
        p = X[i]
        if not any(np.array_equal(p, c) for c in kept):
            kept.append(p.copy())
            if len(kept) == K:
                break
    C = np.array(kept + [kept[0]] * (K - len(kept)), np.float64)
    for _ in range(iters):
        d = ((X[:, None, :] - C[None, :, :]) ** 2).sum(axis=-1)  # [n, K], summed over j in order
        a = np.argmin(d, axis=1)  # the first index of the minimum
        cnt = np.bincount(a, minlength=K)
        for j in range(X.shape[1]):
            s = np.bincount(a, weights=X[:, j], minlength=K)  # member sums in point order
            C[:, j] = np.where(cnt > 0, s / np.maximum(cnt, 1), C[:, j])
    return C


def fit_codebooks(values, d_sub: int, K: int, iters: int, order):
    """values [N, H, d]; order [H, M, N].  Returns fp32 [H, K, M, d_sub]."""
    X = np.asarray(values, np.float32).astype(np.float64)
    N, H, d = X.shape
    M = d // d_sub
    cb = np.empty((H, K, M, d_sub), np.float32)
    for h in range(H):
        for m in range(M):
            cb[h, :, m, :] = kmeans(X[:, h, m * d_sub:(m + 1) * d_sub], K, iters, order[h, m]).astype(np.float32)
    return cb


def encode(x, cb):
    """x [N, H, d]; cb [H, K, M, d_sub].  Returns (codes [N, H, M] uint8, best distance [N, H, M])."""
    X = np.asarray(x, np.float32).astype(np.float64)
    N, H, d = X.shape
    _, K, M, d_sub = cb.shape
    xs = X.reshape(N, H, M, 1, d_sub)
    c = np.asarray(cb, np.float64).transpose(0, 2, 1, 3)[None]  # [1, H, M, K, d_sub]
    dist = ((xs - c) ** 2).sum(axis=-1)  # [N, H, M, K]
    codes = np.argmin(dist, axis=-1)
    return codes.astype(np.uint8), np.take_along_axis(dist, codes[..., None], -1)[..., 0]


def decode(q, cb_k, cb_v, codes_k, codes_v, recent_k, recent_v, scale):
    """One sequence: q [Hq, d]; codes [Hkv, T, M]; recent [Hkv, R, d].  Returns (out [Hq, d], lse [Hq])."""
    Hkv, K, M, d_sub = cb_k.shape
    Hq, d = q.shape
    g = Hq // Hkv
    out = np.empty((Hq, d))
    lse = np.empty(Hq)
    for hq in range(Hq):
        h = hq // g
        m = np.arange(M)
        kh = np.asarray(cb_k, np.float64)[h][codes_k[h], m].reshape(-1, d)  # [T, d]
        vh = np.asarray(cb_v, np.float64)[h][codes_v[h], m].reshape(-1, d)
        keys = np.concatenate([kh, np.asarray(recent_k[h], np.float64)])
        vals = np.concatenate([vh, np.asarray(recent_v[h], np.float64)])
        s = scale * (keys @ np.asarray(q[hq], np.float64))
        mu = s.max()
        p = np.exp(s - mu)
        out[hq] = (p @ vals) / p.sum()
        lse[hq] = mu + np.log(p.sum())
    return out, lse
