"""Seeded synthetic inputs for the product-quantised KV-cache path.

This module only draws random numbers: it holds none of the method's
arithmetic (no distances, no codebook fitting, no attention).  Both the CPU
oracle's tests and the GPU path's tests and benchmark take their inputs from
here, so the two sides see the same bytes.

Shapes follow the decode workloads the MILLION page (DAC 2025 write-up,
"KV cache" motivation paragraph and the TPOT figure, Fig. 12) talks about:
LLaMA-2-7B-shaped heads (32 x 128), a LLaMA-3-8B-shaped GQA layout
(32 query heads over 8 kv heads) and context lengths up to 128K.

Value distribution: the page's outlier analysis (Fig. 3 paragraph) says KV
outliers are mostly channel-wise, with point-like ones as well.  We model
that as N(0,1) values, 4 channels per (layer, kv-head, tensor) scaled x10 for
every token, plus independent point outliers (probability 0.005) scaled x20,
then rounded to fp16.  The clustered outliers of the same figure are not
modelled.

Random streams: every array comes from its own
``SeedSequence([seed, layer, tensor, purpose, b])`` -- K/V values from one per
1024-token chunk, ``SeedSequence([seed, layer, tensor, purpose, b, chunk])`` --:
normals from torch's CPU generator seeded by it (same values for any thread
count), everything else from ``np.random.default_rng`` on it, so arrays are
independent of generation order, and a sample of chunks can be drawn alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# stream keys
TENSOR = {"k": 0, "v": 1, "q": 2}
PURPOSE = {
    "channels": 0,
    "calib": 1,
    "history": 2,
    "recent": 3,
    "prefill": 4,
    "query": 5,
    "lengths": 6,
    "codebook": 7,
    "perm": 8,
}

N_OUTLIER_CHANNELS = 4
CHANNEL_SCALE = 10.0
POINT_PROB = 0.005
POINT_SCALE = 20.0


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, lengths and value recipe."""

    name: str
    seed: int
    batch: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_sub: int
    n_centroids: int
    hist_len: tuple  # PQ history tokens per sequence
    recent_len: int  # full-precision recent tokens per sequence
    dtype: str  # "f16" or "f32" for K/V/q
    outliers: bool
    prefill_len: int = 0  # tokens per sequence of a separately timed prefill encode
    kmeans_iters: int = 10
    n_calib: int = 4096  # calibration tokens per (layer, kv-head, tensor); 0 = fit on history
    description: str = ""

    @property
    def n_sub(self) -> int:
        return self.head_dim // self.d_sub

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_hist(self) -> int:
        return max(self.hist_len) if self.hist_len else 0

    @property
    def t_cap(self) -> int:
        """Code-cache capacity per (sequence, kv head): history rounded up to 64."""
        return max(64, -(-self.max_hist // 64) * 64)

    @property
    def np_dtype(self):
        return np.float16 if self.dtype == "f16" else np.float32


def _lengths_ragged(seed: int, n: int, lo: int, hi: int) -> tuple:
    return tuple(int(v) for v in np.random.default_rng(seed).integers(lo, hi, size=n, endpoint=True))


WORKLOADS = {
    "tiny": Workload(
        name="tiny", seed=1001, batch=1, n_layers=1, n_q_heads=4, n_kv_heads=4, head_dim=64,
        d_sub=2, n_centroids=16, hist_len=(512,), recent_len=16, dtype="f32", outliers=False,
        n_calib=0,
        description="1 seq, 1 layer, 4 heads x 64, d_sub=2, K=16 fit by 10 Lloyd iterations on its "
        "own 512 history tokens, 16 fp32 recent tokens"),
    "llama2_7b_32k": Workload(
        name="llama2_7b_32k", seed=1002, batch=1, n_layers=1, n_q_heads=32, n_kv_heads=32,
        head_dim=128, d_sub=2, n_centroids=256, hist_len=(32768,), recent_len=128, dtype="f16",
        outliers=True,
        description="LLaMA-2-7B-shaped layer, batch 1, 32 heads x 128, d_sub=2, K=256, "
        "32768 PQ history + 128 fp16 recent tokens"),
    "batched_16x8k": Workload(
        name="batched_16x8k", seed=1003, batch=16, n_layers=1, n_q_heads=32, n_kv_heads=32,
        head_dim=128, d_sub=2, n_centroids=256, hist_len=(8192,) * 16, recent_len=64, dtype="f16",
        outliers=True, prefill_len=8192,
        description="batch 16, 32 heads x 128, d_sub=2, K=256, 8192 PQ history + 64 recent per "
        "sequence; pq_encode of the 16x8192 prefill"),
    "gqa_llama3_8b_128k": Workload(
        name="gqa_llama3_8b_128k", seed=1004, batch=1, n_layers=1, n_q_heads=32, n_kv_heads=8,
        head_dim=128, d_sub=4, n_centroids=256, hist_len=(131072,), recent_len=256, dtype="f16",
        outliers=True,
        description="LLaMA-3-8B-shaped GQA, 32 q heads over 8 kv heads, d_sub=4 (8x), K=256, "
        "131072 PQ history + 256 recent"),
    "full32_ragged4": Workload(
        name="full32_ragged4", seed=1005, batch=4, n_layers=32, n_q_heads=32, n_kv_heads=32,
        head_dim=128, d_sub=2, n_centroids=256, hist_len=_lengths_ragged(1005, 4, 1024, 32768),
        recent_len=128, dtype="f16", outliers=True, prefill_len=32768,
        description="32 layers, ragged batch 4 (history lengths uniform in [1024, 32768]), "
        "32 heads x 128, d_sub=2, K=256, 128 recent; 32768-token prefill encode per layer"),
}
WORKLOAD_ORDER = ["tiny", "llama2_7b_32k", "batched_16x8k", "gqa_llama3_8b_128k", "full32_ragged4"]


def stream(seed: int, layer: int, tensor: str, purpose: str, b: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, layer, TENSOR[tensor], PURPOSE[purpose], b]))


def outlier_channels(w: Workload, layer: int, tensor: str) -> np.ndarray:
    """[n_kv_heads, 4] distinct channel indices per head, fixed per (layer, tensor)."""
    g = stream(w.seed, layer, tensor, "channels")
    return np.stack([g.choice(w.head_dim, N_OUTLIER_CHANNELS, replace=False) for _ in range(w.n_kv_heads)])


def _to_dtype(x: np.ndarray, dtype) -> np.ndarray:
    """Round float32 to the workload dtype (IEEE round-to-nearest-even)."""
    if dtype == np.float32:
        return x
    import torch

    return torch.from_numpy(x).to(torch.float16).numpy()


def _normal(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    """N(0,1) float32 from torch's seeded CPU generator (fast, and the same
    values whatever the number of threads)."""
    import torch

    g = torch.Generator().manual_seed(int(seed_seq.generate_state(1, np.uint64)[0] >> np.uint64(1)))
    return torch.randn(shape, generator=g, dtype=torch.float32).numpy()


def bernoulli_positions(g: np.random.Generator, n: int, p: float) -> np.ndarray:
    """Indices of successes of n i.i.d. Bernoulli(p) trials, drawn as geometric gaps."""
    out, pos = [], -1
    while True:
        k = max(1024, int((n - pos) * p * 1.1) + 64)
        c = pos + np.cumsum(g.geometric(p, size=k))
        out.append(c[c < n])
        if c[-1] >= n:
            break
        pos = int(c[-1])
    return np.concatenate(out)


# Values are drawn in chunks of this many tokens, each from a stream of its own, so a
# sample of chunks can be drawn without the rest (same values either way).
CHUNK_TOKENS = 1024


def n_chunks(n_tokens: int) -> int:
    return -(-n_tokens // CHUNK_TOKENS)


def kv_values(w: Workload, layer: int, tensor: str, purpose: str, n_tokens: int, b: int = 0,
              chunks=None) -> np.ndarray:
    """Token-major K or V values [n_tokens, n_kv_heads, head_dim] in the workload dtype.

    Chunk c (tokens [1024c, 1024c + 1024)) comes from
    SeedSequence([seed, layer, tensor, purpose, b, c]).  With `chunks` (a sorted list of
    chunk indices) only those chunks are drawn and concatenated, in order."""
    ids = list(range(n_chunks(n_tokens))) if chunks is None else [int(c) for c in chunks]
    sizes = [min(CHUNK_TOKENS, n_tokens - c * CHUNK_TOKENS) for c in ids]
    assert all(n > 0 for n in sizes), "chunk index past the end"
    out = np.empty((sum(sizes), w.n_kv_heads, w.head_dim), dtype=w.np_dtype)
    ch = outlier_channels(w, layer, tensor) if w.outliers else None
    pos = 0
    for c, n in zip(ids, sizes):
        ss = np.random.SeedSequence([w.seed, layer, TENSOR[tensor], PURPOSE[purpose], b, c])
        x = _normal(ss, (n, w.n_kv_heads, w.head_dim))
        if w.outliers:
            x[:, np.arange(w.n_kv_heads)[:, None], ch] *= CHANNEL_SCALE
            g = np.random.default_rng(ss.spawn(1)[0])
            flat = x.reshape(-1)
            flat[bernoulli_positions(g, flat.size, POINT_PROB)] *= POINT_SCALE
        out[pos:pos + n] = _to_dtype(x, w.np_dtype)
        pos += n
    return out


def sample_chunks(seed: int, n_tokens: int, fraction: float = 0.125) -> list:
    """A seeded sorted sample of ceil(fraction * chunks) chunk indices (at least one)."""
    n = n_chunks(n_tokens)
    k = max(1, -(-int(round(fraction * 1e6)) * n // 1000000))
    return sorted(int(c) for c in np.random.default_rng(seed).choice(n, size=min(k, n), replace=False))


def chunk_tokens(chunks, n_tokens: int) -> np.ndarray:
    """The token positions the given chunks cover, in order."""
    return np.concatenate([np.arange(c * CHUNK_TOKENS, min((c + 1) * CHUNK_TOKENS, n_tokens)) for c in chunks])


def queries(w: Workload, layer: int = 0) -> np.ndarray:
    """Decode queries [batch, n_q_heads, head_dim], N(0,1), no outliers."""
    ss = np.random.SeedSequence([w.seed, layer, TENSOR["q"], PURPOSE["query"], 0])
    return _to_dtype(_normal(ss, (w.batch, w.n_q_heads, w.head_dim)), w.np_dtype)


def recent_kv(w: Workload, layer: int, tensor: str) -> np.ndarray:
    """Recent full-precision window [batch, n_kv_heads, recent_len, head_dim]."""
    out = np.empty((w.batch, w.n_kv_heads, w.recent_len, w.head_dim), dtype=w.np_dtype)
    for b in range(w.batch):
        out[b] = kv_values(w, layer, tensor, "recent", w.recent_len, b).transpose(1, 0, 2)
    return out


def history_kv(w: Workload, layer: int, tensor: str, b: int, chunks=None) -> np.ndarray:
    """PQ-history values of sequence b, token-major [hist_len[b], n_kv_heads, head_dim]
    (only the given 1024-token chunks, concatenated, with `chunks`)."""
    return kv_values(w, layer, tensor, "history", w.hist_len[b], b, chunks)


def calibration_kv(w: Workload, layer: int, tensor: str) -> np.ndarray:
    """Calibration draw for codebook fitting [n_calib, n_kv_heads, head_dim].

    With n_calib == 0 the workload fits on its own history (sequence 0)."""
    if w.n_calib == 0:
        return history_kv(w, layer, tensor, 0)
    return kv_values(w, layer, tensor, "calib", w.n_calib)


def init_order(w: Workload, layer: int, tensor: str, n_points: int) -> np.ndarray:
    """Seeded permutations for k-means initialisation, [n_kv_heads, n_sub, n_points] int64.

    The random numbers the fitting draws are inputs, drawn here."""
    g = stream(w.seed, layer, tensor, "perm")
    return np.stack([np.stack([g.permutation(n_points) for _ in range(w.n_sub)])
                     for _ in range(w.n_kv_heads)]).astype(np.int64)


def drawn_codebook(w: Workload, layer: int, tensor: str) -> np.ndarray:
    """A codebook drawn at random from the value distribution, [n_kv_heads, K, n_sub, d_sub] fp32.

    Each centroid is an independent draw of the same outlier-bearing
    distribution as the data (channel outliers included).  It is a valid
    codebook of the right shape and magnitude, used where fitted codebooks
    are not needed (throughput runs); it is not a k-means fit."""
    x = kv_values(w, layer, tensor, "codebook", w.n_centroids).astype(np.float32)  # [K, H, d]
    cb = x.reshape(w.n_centroids, w.n_kv_heads, w.n_sub, w.d_sub).transpose(1, 0, 2, 3)
    return np.ascontiguousarray(cb)


def small_normal(seed: int, shape, dtype=np.float32) -> np.ndarray:
    """Plain seeded N(0,1) draws for small ad-hoc test inputs."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32).astype(dtype)


def small_codes(seed: int, shape, n_centroids: int) -> np.ndarray:
    """Uniform random codes in [0, n_centroids) as uint8."""
    return np.random.default_rng(seed).integers(0, n_centroids, size=shape, dtype=np.uint8)


def grid_values(seed: int, shape, levels=(-1.5, -0.5, 0.5, 1.5), dtype=np.float32) -> np.ndarray:
    """Values drawn uniformly from a small set of levels."""
    idx = np.random.default_rng(seed).integers(0, len(levels), size=shape)
    return np.asarray(levels, dtype=np.float64)[idx].astype(dtype)
