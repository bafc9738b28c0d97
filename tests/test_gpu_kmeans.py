"""GPU parity of pqkv_fit_codebooks (offline Lloyd k-means) against the oracle.

Both sides evaluate the same definition in fp64 with every product, sum and
quotient rounded on its own, members summed in point order and the same
initialisation walk, so the fp32 codebooks must be byte-identical.  Cases: the
tiny workload's own-history fit, slices of the 32K and GQA calibration draws at
full size (4096 points, K = 256, d_sub 2 and 4, fp16), fewer distinct points than
centroids, fewer points than centroids, no iterations, and strided fp32 input.
"""
import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import dims_for, to_dev

pytestmark = pytest.mark.gpu


def _gpu_fit(values, d_sub, K, iters, order, head_stride_pad=0):
    import torch

    import decode_attention_pq_amd as P

    N, H, d = values.shape
    M = d // d_sub
    dims = dims_for(d, d_sub, K, H, H)
    if head_stride_pad:  # heads spaced out inside a wider row: a strided view
        wide = np.zeros((N, H, d + head_stride_pad), values.dtype)
        wide[:, :, :d] = values
        x = to_dev(wide)[:, :, :d]
    else:
        x = to_dev(values)
    cb = torch.full((H, K, M, d_sub), float("nan"), dtype=torch.float32, device="cuda")
    kept = torch.full((H, M), -1, dtype=torch.int32, device="cuda")
    P.fit_codebooks(dims, x, to_dev(np.ascontiguousarray(order, np.int32)), iters, cb, kept)
    torch.cuda.synchronize()
    return cb.cpu().numpy(), kept.cpu().numpy()


def _check(values, d_sub, K, iters, order, **kw):
    got, kept = _gpu_fit(values, d_sub, K, iters, order, **kw)
    ref, ref_kept = oracle.fit_codebooks(values, d_sub, K, iters, order, return_kept=True)
    np.testing.assert_array_equal(kept, ref_kept)
    diff = got.view(np.uint32) != ref.view(np.uint32)
    assert not diff.any(), f"{int(diff.sum())} of {diff.size} centroid values differ, first at {np.argwhere(diff)[:3].tolist()}"
    return kept


def test_fit_tiny_workload_own_history():
    w = synthkv.WORKLOADS["tiny"]
    values = synthkv.calibration_kv(w, 0, "k")
    order = synthkv.init_order(w, 0, "k", values.shape[0])
    _check(values, w.d_sub, w.n_centroids, w.kmeans_iters, order)


@pytest.mark.parametrize("wname,tensor,heads", [("llama2_7b_32k", "k", 2), ("gqa_llama3_8b_128k", "v", 1)])
def test_fit_calibration_draw_full_size(wname, tensor, heads):
    w = synthkv.WORKLOADS[wname]
    values = synthkv.calibration_kv(w, 0, tensor)[:, :heads]
    order = synthkv.init_order(w, 0, tensor, values.shape[0])[:heads]
    kept = _check(values, w.d_sub, w.n_centroids, w.kmeans_iters, np.ascontiguousarray(order))
    assert (kept == w.n_centroids).all()


def test_fit_fewer_distinct_points_than_centroids():
    values = synthkv.grid_values(61, (300, 2, 64), levels=(-1.5, -0.5, 0.5, 1.5))  # 16 distinct 2-vectors
    order = np.stack([np.stack([np.random.default_rng(62 + 32 * h + m).permutation(300) for m in range(32)])
                      for h in range(2)])
    kept = _check(values, 2, 32, 5, order)
    assert (kept == 16).all()


def test_fit_fewer_points_than_centroids_and_no_iterations():
    values = synthkv.small_normal(63, (20, 1, 64)).astype(np.float16)
    order = np.stack([np.stack([np.random.default_rng(64 + m).permutation(20) for m in range(16)])])
    kept = _check(values, 4, 64, 3, order)
    assert (kept == 20).all()
    _check(values, 4, 64, 0, order)


def test_fit_strided_fp32_input():
    values = synthkv.small_normal(65, (700, 3, 64)) * 3.0
    order = np.stack([np.stack([np.random.default_rng(66 + 32 * h + m).permutation(700) for m in range(32)])
                      for h in range(3)])
    _check(values.astype(np.float32), 2, 100, 7, order, head_stride_pad=32)


@pytest.mark.parametrize("d_sub,K", [(2, 64), (4, 100)])
def test_fit_ragged_point_count(d_sub, K):
    # neither a multiple of 4 (the word-wise assignment scan) nor of 32 (one bit of a
    # centroid's block mask); K 100 takes the plain (not 16-blocked) nearest-centroid scan
    values = synthkv.small_normal(67, (203, 2, 64)).astype(np.float16)
    M = 64 // d_sub
    order = np.stack([np.stack([np.random.default_rng(68 + 32 * h + m).permutation(203) for m in range(M)])
                      for h in range(2)])
    _check(values, d_sub, K, 4, order)


def test_fit_maximum_point_count():
    n = 8192  # the largest fit, whose points, assignments and masks fill most of LDS
    values = synthkv.small_normal(69, (n, 1, 128)).astype(np.float16)
    order = np.stack([np.stack([np.random.default_rng(70 + m).permutation(n) for m in range(32)])])
    _check(values, 4, 256, 2, order)
