"""CPU oracle for the product-quantised KV-cache path (MILLION, DAC 2025).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it shares no code with that path: the only thing both sides share is the
seeded input generator ``synthkv``.

Precision: float64 throughout, from exact widenings of the fp16/fp32 inputs,
except ``encode_f32`` (see O2).

What it computes, and where the page (the MILLION write-up, DAC 2025)
states it:

* O1  ``kmeans`` / ``fit_codebooks`` -- Lloyd k-means per subspace (Fig. 5
  paragraph: clustering fused channels; the paragraph after it: PQ splits the
  vector into subspaces of dimension 2 or 4; Fig. 6 paragraph: codebooks are
  trained offline).
* O2  ``encode`` -- brute-force nearest centroid (Fig. 6 paragraph: the online
  prefill stage quantises the KV cache with the trained codebooks).
  ``encode_f32`` takes the same decision in fp32, the precision of the GPU path,
  so that codes can be compared byte for byte, near ties included.
* O3/O4 ``decode_exact`` -- dequantise, then plain softmax attention over
  history + recent tokens (Fig. 7 paragraph: history attention and
  generated-token attention are computed separately and combined; their union
  is ordinary attention).
* O5  ``lut``, ``lut_scores``, ``hist_partial``, ``recent_partial``,
  ``merge_partials``, ``decode_method`` -- the method's own algebra in the
  page's order: an asymmetric-distance lookup table of query x codebook
  (Fig. 7 paragraph), history scores as sums of table entries, split-wise
  softmax partials (flash decoding, Fig. 8 paragraph) and a log-sum-exp merge.
* O6  ``compression_ratio`` and friends -- byte accounting (4x at d_sub=2 with
  8-bit codes versus fp16, stated in the LongBench and TPOT paragraphs).
* O7  ``append_kv_step`` -- one step of the live cache (Fig. 7 paragraph:
  generated tokens are kept in full precision, apart from the quantised
  history, and quantised later in batches): a full recent window first moves
  its oldest tokens, encoded by O2, to the end of the history; the new token
  then joins the window.
* ``code_offsets`` / ``tile_codes`` / ``untile_codes`` -- the code-cache byte
  layout the C interface defines (a format, implemented here on its own from
  its definition).

Parity pins for each function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

AMBIGUITY_REL = 1e-5


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (always recompiles)."""
    # no contraction: every fp32 step of encode_f32 rounds exactly as written
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o",
           _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib_handle = None


def lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_kmeans.argtypes = [p, i64, i32, i32, i32, p, p, p, p]
        L.orc_kmeans.restype = i64
        L.orc_lloyd.argtypes = [p, i64, i32, i32, i32, p, p, p]
        L.orc_fit_codebooks.argtypes = [p, i64, i32, i32, i32, i32, i32, p, p, p]
        L.orc_encode.argtypes = [p, i64, i32, i32, i32, i32, p, p, p, p]
        L.orc_code_distance.argtypes = [p, i64, i32, i32, i32, i32, p, p, p]
        L.orc_encode_f32.argtypes = [p, i64, i32, i32, i32, i32, p, p]
        L.orc_sqdist_f32.argtypes = [p, p, i32]
        L.orc_sqdist_f32.restype = ctypes.c_float
        L.orc_decode_exact.argtypes = [i32, i32, i32, i32, i32, i32, p, p, p, p, p, i64, p, p, p, i64, p,
                                       f64, p, p]
        L.orc_dequantize.argtypes = [p, i64, i32, i32, i32, i32, p, p]
        L.orc_set_threads.argtypes = [i32]
        _lib_handle = L
    return _lib_handle


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float32)


# ---------------------------------------------------------------- O1 k-means
def kmeans(X, K: int, iters: int, order=None):
    """Lloyd k-means of points X [n, dsub] (fp64).

    Returns (centroids fp64 [K, dsub], assignment of the last update [n],
    SSE trace [2*iters] (after each assignment and each update), distinct kept)."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    n, dsub = X.shape
    order = np.arange(n, dtype=np.int64) if order is None else np.ascontiguousarray(order, dtype=np.int64)
    C = np.empty((K, dsub), np.float64)
    assign = np.empty(n, np.int32)
    trace = np.empty(max(1, 2 * iters), np.float64)
    kept = lib().orc_kmeans(_ptr(X), n, dsub, K, iters, _ptr(order), _ptr(C), _ptr(assign), _ptr(trace))
    if kept < 0:
        raise ValueError("bad k-means arguments")
    return C, assign, trace[: 2 * iters], int(kept)


def lloyd(X, C0, iters: int):
    """Lloyd iterations from given centroids C0 [K, dsub].  Same returns as kmeans (no kept)."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    n, dsub = X.shape
    C = np.array(C0, dtype=np.float64, order="C", copy=True)
    K = C.shape[0]
    assign = np.empty(n, np.int32)
    trace = np.empty(max(1, 2 * iters), np.float64)
    if lib().orc_lloyd(_ptr(X), n, dsub, K, iters, _ptr(C), _ptr(assign), _ptr(trace)) != 0:
        raise ValueError("bad Lloyd arguments")
    return C, assign, trace[: 2 * iters]


def fit_codebooks(values, d_sub: int, K: int, iters: int, order, return_kept: bool = False):
    """Fit every (head, subspace) codebook of one tensor.

    values: [N, H, d] fp16/fp32 token-major; order: [H, M, N] permutations.
    Returns the fp32 codebook [H, K, M, d_sub] (the fp64 fit rounded to fp32,
    which is the canonical codebook both sides consume), and with return_kept
    also the distinct points the initialisation kept, [H, M]."""
    X = _f32(values)
    N, H, d = X.shape
    M = d // d_sub
    order = np.ascontiguousarray(order, dtype=np.int64)
    assert order.shape == (H, M, N)
    cb = np.empty((H, K, M, d_sub), np.float64)
    kept = np.empty((H, M), np.int64)
    rc = lib().orc_fit_codebooks(_ptr(X), N, H, d, d_sub, K, iters, _ptr(order), _ptr(cb), _ptr(kept))
    if rc != 0:
        raise ValueError("bad fit arguments")
    return (cb.astype(np.float32), kept) if return_kept else cb.astype(np.float32)


# ---------------------------------------------------------------- O2 encode
def encode(x, codebook):
    """Brute-force nearest-centroid codes.

    x: [N, H, d] fp16/fp32; codebook: [H, K, M, d_sub] fp32.
    Returns (codes uint8 [N, H, M], d1, d2 fp64 [N, H, M], ambiguous bool [N, H, M]).
    A pair is ambiguous when the runner-up distance is within
    1e-5 * max(1, best) of the best one."""
    X = _f32(x)
    cb = _f32(codebook)
    N, H, d = X.shape
    Hc, K, M, d_sub = cb.shape
    assert Hc == H and M * d_sub == d
    codes = np.empty((N, H, M), np.uint8)
    d1 = np.empty((N, H, M), np.float64)
    d2 = np.empty((N, H, M), np.float64)
    rc = lib().orc_encode(_ptr(X), N, H, d, d_sub, K, _ptr(cb), _ptr(codes), _ptr(d1), _ptr(d2))
    if rc != 0:
        raise ValueError("bad encode arguments")
    return codes, d1, d2, ambiguous(d1, d2)


def encode_f32(x, codebook):
    """The same nearest-centroid rule, decided in fp32 (O2 in the precision the GPU
    computes in: a code is an integer that floating point decides, and the page
    fixes no precision).  The squared distance is evaluated in subspace order:
    e = x_j - c_j rounded to fp32, then d = fma(e, e, d) from d = 0.  The first
    centroid with a strictly smaller d wins (lowest index on ties); a NaN distance
    never wins; no distance below +inf gives code 0.

    x: [N, H, d] fp16/fp32; codebook: [H, K, M, d_sub] fp32.  Returns uint8 [N, H, M]."""
    X = _f32(x)
    cb = _f32(codebook)
    N, H, d = X.shape
    Hc, K, M, d_sub = cb.shape
    assert Hc == H and M * d_sub == d
    codes = np.empty((N, H, M), np.uint8)
    if lib().orc_encode_f32(_ptr(X), N, H, d, d_sub, K, _ptr(cb), _ptr(codes)) != 0:
        raise ValueError("bad encode arguments")
    return codes


def sqdist_f32(x, c) -> float:
    """encode_f32's distance of one subvector x to one centroid c (fp32)."""
    x = _f32(x).ravel()
    c = _f32(c).ravel()
    assert x.size == c.size
    return float(lib().orc_sqdist_f32(_ptr(x), _ptr(c), int(x.size)))


def ambiguous(d1, d2):
    """The tie tolerance of the encode comparison: the runner-up distance d2 lies less
    than 1e-5 * max(1, d1) above the best one d1.  The page fixes no tolerance; the
    reading is a relative band floored at 1, because an absolute 1e-5 is below fp32
    resolution for outlier subvectors (d1 of 1e2 to 1e5).  Pinned at its boundaries
    by constructed pairs in the tests."""
    return (d2 - d1) < AMBIGUITY_REL * np.maximum(1.0, d1)


def code_distance(x, codebook, codes):
    """fp64 squared distance of each (token, head, subspace) to the given code."""
    X = _f32(x)
    cb = _f32(codebook)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    N, H, d = X.shape
    _, K, M, d_sub = cb.shape
    dist = np.empty((N, H, M), np.float64)
    lib().orc_code_distance(_ptr(X), N, H, d, d_sub, K, _ptr(cb), _ptr(codes), _ptr(dist))
    return dist


def dequantize(codes, codebook):
    """codes [N, H, M] -> fp64 vectors [N, H, d]."""
    cb = _f32(codebook)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    N, H, M = codes.shape
    _, K, M2, d_sub = cb.shape
    assert M2 == M
    out = np.empty((N, H, M * d_sub), np.float64)
    lib().orc_dequantize(_ptr(codes), N, H, M * d_sub, d_sub, K, _ptr(cb), _ptr(out))
    return out


# ---------------------------------------------------------------- O3/O4 exact attention
def decode_exact(q, cb_k, cb_v, codes_k, codes_v, hist_len, recent_k, recent_v, recent_len, scale):
    """Dequantise-then-exact decode attention.

    q [B, Hq, d]; cb_k/cb_v [Hkv, K, M, d_sub]; codes_k/codes_v logical
    [B, Hkv, Tcap, M]; hist_len [B]; recent_k/recent_v [B, Hkv, Rcap, d];
    recent_len [B]; scale: the softmax scale as the GPU receives it.
    Returns (out fp64 [B, Hq, d], lse fp64 [B, Hq], natural log)."""
    qf = _f32(q)
    B, Hq, d = qf.shape
    cbk, cbv = _f32(cb_k), _f32(cb_v)
    Hkv, K, M, d_sub = cbk.shape
    ck = np.ascontiguousarray(codes_k, dtype=np.uint8)
    cv = np.ascontiguousarray(codes_v, dtype=np.uint8)
    Tcap = ck.shape[2]
    rk, rv = _f32(recent_k), _f32(recent_v)
    Rcap = rk.shape[2]
    hl = np.ascontiguousarray(hist_len, dtype=np.int32)
    rl = np.ascontiguousarray(recent_len, dtype=np.int32)
    out = np.empty((B, Hq, d), np.float64)
    lse = np.empty((B, Hq), np.float64)
    rc = lib().orc_decode_exact(B, Hq, Hkv, d, d_sub, K, _ptr(qf), _ptr(cbk), _ptr(cbv), _ptr(ck), _ptr(cv),
                                Tcap, _ptr(hl), _ptr(rk), _ptr(rv), Rcap, _ptr(rl), float(scale),
                                _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("bad decode arguments")
    return out, lse


# ---------------------------------------------------------------- O5 method algebra (fp64)
def lut(q, cb_k, group: int):
    """Asymmetric-distance lookup table LUT[b, hq, m, c] = q[b,hq,m-th subvector] . C_K[h, c, m]
    (unscaled), h = hq // group.  q [B, Hq, d]; cb_k [Hkv, K, M, d_sub]."""
    q = np.asarray(q, dtype=np.float64)
    cb = np.asarray(cb_k, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, K, M, d_sub = cb.shape
    qs = q.reshape(B, Hq, M, d_sub)
    cbq = cb[np.arange(Hq) // group]  # [Hq, K, M, d_sub]
    return np.einsum("bhmj,hcmj->bhmc", qs, cbq)


def lut_scores(lut_row, codes, scale):
    """History scores s_t = scale * sum_m LUT[m, code[t, m]].  lut_row [M, K]; codes [T, M]."""
    codes = np.asarray(codes, dtype=np.int64)
    M = lut_row.shape[0]
    vals = lut_row[np.arange(M)[None, :], codes]  # [T, M]
    return scale * vals.sum(axis=1)


def hist_partial(scores, codes_v, cb_v_head):
    """Softmax partial over one split of history tokens via per-subspace histograms.

    scores [T]; codes_v [T, M]; cb_v_head [K, M, d_sub].
    Returns (mu, l, o) with o unnormalised: o = sum_t exp(s_t - mu) vhat_t,
    computed as H[m, c] = sum_t p_t [code_v[t, m] == c], o[m, j] = sum_c H[m, c] C_V[c, m, j]."""
    cbv = np.asarray(cb_v_head, dtype=np.float64)
    K, M, d_sub = cbv.shape
    if len(scores) == 0:
        return -math.inf, 0.0, np.zeros(M * d_sub)
    mu = float(np.max(scores))
    p = np.exp(np.asarray(scores, np.float64) - mu)
    H = np.zeros((M, K))
    cv = np.asarray(codes_v, dtype=np.int64)
    for m in range(M):
        np.add.at(H[m], cv[:, m], p)
    o = np.einsum("mc,cmj->mj", H, cbv).reshape(M * d_sub)
    return mu, float(p.sum()), o


def recent_partial(q_row, rk, rv, scale):
    """Softmax partial over full-precision recent tokens. q_row [d]; rk/rv [R, d]."""
    rk = np.asarray(rk, np.float64)
    rv = np.asarray(rv, np.float64)
    if rk.shape[0] == 0:
        return -math.inf, 0.0, np.zeros(rk.shape[1])
    s = scale * (rk @ np.asarray(q_row, np.float64))
    mu = float(s.max())
    p = np.exp(s - mu)
    return mu, float(p.sum()), p @ rv


def merge_partials(parts):
    """Log-sum-exp merge of partials (mu_i, l_i, o_i) -> (out, lse)."""
    mus = [pm for pm, _, _ in parts if pm != -math.inf]
    d = len(parts[0][2])
    if not mus:
        return np.zeros(d), -math.inf
    mu = max(mus)
    num = np.zeros(d)
    den = 0.0
    for pm, pl, po in parts:
        if pm == -math.inf:
            continue
        w = math.exp(pm - mu)
        num += w * np.asarray(po, np.float64)
        den += w * pl
    return num / den, mu + math.log(den)


def merge_states(out_a, lse_a, out_b, lse_b):
    """Merge two normalised attention states row-wise (out [n, d], lse [n])."""
    out_a = np.asarray(out_a, np.float64)
    out_b = np.asarray(out_b, np.float64)
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    out = np.zeros_like(out_a)
    lse = np.full_like(lse_a, -np.inf)
    for i in range(len(lse_a)):
        parts = []
        for o, l_ in ((out_a[i], lse_a[i]), (out_b[i], lse_b[i])):
            parts.append((l_, 1.0, o) if l_ != -math.inf else (-math.inf, 0.0, o))
        out[i], lse[i] = merge_partials(parts)
    return out, lse


def decode_method(q, cb_k, cb_v, codes_k, codes_v, hist_len, recent_k, recent_v, recent_len, scale,
                  split_bounds=None):
    """The method's path in the page's order: LUT -> LUT-sum scores -> split-wise softmax
    partials with histogram value side -> recent-window partial -> log-sum-exp merge.

    split_bounds(b, T) -> list of split start offsets (default: one split).
    Same arguments and return as decode_exact."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    cbk = np.asarray(cb_k, np.float64)
    cbv = np.asarray(cb_v, np.float64)
    Hkv = cbk.shape[0]
    g = Hq // Hkv
    L = lut(q, cbk, g)
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        T = int(hist_len[b])
        R = int(recent_len[b])
        starts = [0] if split_bounds is None else list(split_bounds(b, T))
        for hq in range(Hq):
            h = hq // g
            s = lut_scores(L[b, hq], codes_k[b, h, :T], scale)
            parts = []
            for i, st in enumerate(starts):
                en = starts[i + 1] if i + 1 < len(starts) else T
                parts.append(hist_partial(s[st:en], codes_v[b, h, st:en], cbv[h]))
            parts.append(recent_partial(q[b, hq], recent_k[b, h, :R], recent_v[b, h, :R], scale))
            out[b, hq], lse[b, hq] = merge_partials(parts)
    return out, lse


# ---------------------------------------------------------------- code-cache layout
TILE_TOKENS = 64
CHUNK_BYTES = 16


def append_kv_step(state, new_k, new_v, cb_k, cb_v, r_cap: int, n_roll: int):
    """One decode step of the live cache, per sequence b (Fig. 7 paragraph).

    state: dict of per-sequence lists --
      'codes_k', 'codes_v': uint8 [T_b, H, M] history codes;
      'amb_k', 'amb_v':     bool  [T_b, H, M], True where the code's runner-up is within the
                            encode ambiguity band (always False for codes given at the start);
      'recent_k', 'recent_v': [R_b, H, d] full-precision recent rows, oldest first.
    new_k, new_v: [B, H, d].  If R_b == r_cap, rows [0, n_roll) are encoded (O2) and appended to
    the history and the window keeps rows [n_roll, R_b); then the new row is appended to the
    window.  Returns a new state dict (inputs are not modified)."""
    out = {k: list(v) for k, v in state.items()}
    for b in range(len(out["recent_k"])):
        for t_name, cb, new in (("k", cb_k, new_k), ("v", cb_v, new_v)):
            rec = out["recent_" + t_name][b]
            if rec.shape[0] == r_cap:
                codes, _, _, amb = encode(rec[:n_roll], cb)
                out["codes_" + t_name][b] = np.concatenate([out["codes_" + t_name][b], codes], axis=0)
                out["amb_" + t_name][b] = np.concatenate([out["amb_" + t_name][b], amb], axis=0)
                rec = rec[n_roll:]
            out["recent_" + t_name][b] = np.concatenate([rec, np.asarray(new[b])[None]], axis=0)
    return out


def code_offsets(n_sub: int, t_cap: int) -> np.ndarray:
    """Byte offset of (token t, subspace m) inside one (sequence, kv-head) code plane.

    Tiles of 64 tokens occupy 64*M contiguous bytes.  Inside a tile the bytes
    of token slot l (t mod 64) form M/16 chunks of 16 bytes; chunk i of every
    slot sits at i*1024 + l*16.  Byte p of slot l holds subspace (p + l) mod M.
    Returns int64 [t_cap, M]."""
    M = n_sub
    t = np.arange(t_cap, dtype=np.int64)[:, None]
    m = np.arange(M, dtype=np.int64)[None, :]
    lane = t % TILE_TOKENS
    p = (m - lane) % M
    return (t // TILE_TOKENS) * (TILE_TOKENS * M) + (p // CHUNK_BYTES) * (TILE_TOKENS * CHUNK_BYTES) \
        + lane * CHUNK_BYTES + p % CHUNK_BYTES


def tile_codes(codes, t_cap: int) -> np.ndarray:
    """Logical codes [..., T, M] (T <= t_cap) -> planes [..., t_cap*M] in the cache layout.
    Slots past T are zero."""
    codes = np.asarray(codes, np.uint8)
    *lead, T, M = codes.shape
    off = code_offsets(M, t_cap)[:T]
    planes = np.zeros((*lead, t_cap * M), np.uint8)
    flat_p = planes.reshape(-1, t_cap * M)
    flat_c = codes.reshape(-1, T, M)
    for i in range(flat_c.shape[0]):
        flat_p[i][off] = flat_c[i]
    return planes


def untile_codes(planes, T: int, n_sub: int) -> np.ndarray:
    """Cache-layout planes [..., t_cap*M] -> logical codes [..., T, M]."""
    planes = np.asarray(planes, np.uint8)
    *lead, n = planes.shape
    t_cap = n // n_sub
    off = code_offsets(n_sub, t_cap)[:T]
    flat = planes.reshape(-1, n)
    return np.stack([flat[i][off] for i in range(flat.shape[0])]).reshape(*lead, T, n_sub)


# ---------------------------------------------------------------- O6 byte accounting
def fp16_bytes_per_token(head_dim: int) -> int:
    return 2 * head_dim


def pq_bytes_per_token(head_dim: int, d_sub: int, code_bits: int = 8) -> float:
    return (head_dim // d_sub) * code_bits / 8


def compression_ratio(head_dim: int, d_sub: int, code_bits: int = 8) -> float:
    """fp16 bytes over PQ code bytes per (token, head, tensor): 16*d_sub/code_bits."""
    return fp16_bytes_per_token(head_dim) / pq_bytes_per_token(head_dim, d_sub, code_bits)


def kv_cache_bytes_fp16(n_layers: int, n_kv_heads: int, head_dim: int, n_tokens: int) -> int:
    """K and V for every layer and head at fp16."""
    return n_layers * 2 * n_kv_heads * head_dim * 2 * n_tokens


def codebook_bytes(n_kv_heads: int, n_centroids: int, head_dim: int) -> int:
    """fp32 K and V codebooks of one layer."""
    return 2 * n_kv_heads * n_centroids * head_dim * 4


def fit_workload_codebooks(w, layer: int, tensor: str, synth) -> np.ndarray:
    """Fit the codebook of (layer, tensor) of a workload on its calibration draw."""
    values = synth.calibration_kv(w, layer, tensor)
    order = synth.init_order(w, layer, tensor, values.shape[0])
    return fit_codebooks(values, w.d_sub, w.n_centroids, w.kmeans_iters, order)
