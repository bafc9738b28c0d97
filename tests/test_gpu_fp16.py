"""GPU parity of the dense fp16 decode baseline (pqkv_fp16_decode_attention)
against the oracle's exact attention, with the whole context as its
full-precision window: small shapes (ragged, empty, GQA groups, both head
sizes, one and many splits) and the full 32K and 128K decode shapes."""
import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, dims_for, softmax_scale, to_dev

pytestmark = pytest.mark.gpu


def _run(dims, q, k, v, lens, max_len=None):
    import torch

    import decode_attention_pq_amd as P

    B, Hq, d = q.shape
    t_cap = k.shape[2]
    max_len = int(max(lens)) if max_len is None else max_len
    out = torch.full((B, Hq, d), np.nan, dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), np.nan, dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(256, P.fp16_decode_workspace_bytes(dims, B, max_len)), dtype=torch.uint8, device="cuda")
    P.fp16_decode_attention(dims, to_dev(q), to_dev(k), to_dev(v), t_cap, to_dev(np.asarray(lens, np.int32)), max_len,
                            softmax_scale(d), out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _oracle(q, k, v, lens):
    B, Hkv = k.shape[:2]
    d = q.shape[2]
    empty = np.zeros((B, Hkv, 1, 1), np.uint8)
    cb = np.zeros((Hkv, 1, 1, d), np.float32)  # no history: one subspace of dimension d, never read
    return oracle.decode_exact(q, cb, cb, empty, empty, [0] * B, k, v, lens, softmax_scale(d))


CASES = [
    # d, Hq, Hkv, lengths, t_cap
    (128, 4, 4, (700, 0), 768),
    (128, 8, 2, (5000, 1, 129, 4096), 5120),      # GQA 4, ragged, several splits
    (64, 16, 2, (3000, 2048), 3072),               # GQA 8, d 64
    (64, 2, 2, (64, 63, 65), 128),                 # one wave step and its edges
    (128, 2, 1, (0,), 64),                         # nothing cached
    (128, 32, 32, (33000,), 33024),                # many heads, 16 splits
    (128, 4, 4, (100000,), 100096),                # 64 splits of a long context
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_fp16_decode_matches_oracle(case):
    d, Hq, Hkv, lens, t_cap = case
    B = len(lens)
    s = sum(lens) + d + Hq
    q = synthkv.small_normal(s, (B, Hq, d), np.float16)
    k = synthkv.small_normal(s + 1, (B, Hkv, t_cap, d), np.float16)
    v = synthkv.small_normal(s + 2, (B, Hkv, t_cap, d), np.float16)
    ref_out, ref_lse = _oracle(q, k, v, lens)
    out, lse = _run(dims_for(d, 2, 256, Hq, Hkv), q, k, v, lens)
    check_attention(out, lse, ref_out, ref_lse)
    # a looser bound on the lengths gives the same result
    out2, lse2 = _run(dims_for(d, 2, 256, Hq, Hkv), q, k, v, lens, max_len=t_cap)
    check_attention(out2, lse2, ref_out, ref_lse)


@pytest.mark.parametrize("name", ["llama2_7b_32k", "gqa_llama3_8b_128k"])
def test_fp16_decode_full_workload_shapes(name):
    """The 32K (32 heads) and 128K (32 query heads over 8 kv heads) decode shapes with
    their synthetic outlier-bearing K/V: the history and the recent window together
    as one fp16 cache."""
    w = synthkv.WORKLOADS[name]
    T = w.hist_len[0] + w.recent_len
    t_cap = -(-T // 64) * 64
    k = np.zeros((1, w.n_kv_heads, t_cap, w.head_dim), np.float16)
    v = np.zeros_like(k)
    for arr, tensor in ((k, "k"), (v, "v")):
        arr[0, :, :w.hist_len[0]] = synthkv.history_kv(w, 0, tensor, 0).transpose(1, 0, 2)
        arr[0, :, w.hist_len[0]:T] = synthkv.recent_kv(w, 0, tensor)[0]
    q = synthkv.queries(w)
    ref_out, ref_lse = _oracle(q, k, v, [T])
    out, lse = _run(dims_for(w.head_dim, w.d_sub, w.n_centroids, w.n_q_heads, w.n_kv_heads), q, k, v, [T])
    err, lerr = check_attention(out, lse, ref_out, ref_lse)
    print(f"[fp16] {name}: {T} tokens, max row error {err:.2e}, lse error {lerr:.2e}", flush=True)
