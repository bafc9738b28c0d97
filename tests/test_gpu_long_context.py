"""Decode parity at the longest histories the split plan accepts: 512 splits per
(sequence, kv head, query-head group), each split 16 rounds of 512 tokens (one or two
query heads per work-group) or 8 rounds (four).  The merge then folds 512 partial
states; one token more is refused on the host (tests/test_abi.py).

Codes are seeded random bytes: attention parity does not depend on how valid codes
were obtained.  The oracle (exact fp64 attention over the dequantised history and the
recent window) streams the history token by token, so it finishes in seconds."""
import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, dims_for, run_gpu_decode, softmax_scale

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.mark.parametrize("d,dsub,K,Hq,Hkv,T,R,lut", [
    (64, 4, 256, 1, 1, 512 * 8192 - 37, 7, "none"),   # one query head: 512 splits of 16 rounds, ragged tail
    (64, 4, 256, 4, 1, 512 * 4096, 3, "none"),        # four query heads per work-group: 512 splits of 8 rounds
    (64, 4, 256, 4, 1, 512 * 4096, 3, "gpu"),         # the same through a materialised table
])
def test_decode_at_the_split_limit(d, dsub, K, Hq, Hkv, T, R, lut):
    M = d // dsub
    t_cap = -(-T // 64) * 64
    seed = 7000 + T % 1000 + Hq
    print(f"[long] T={T} Hq={Hq} Hkv={Hkv} lut={lut}", flush=True)
    q = synthkv.small_normal(seed, (1, Hq, d), np.float16)
    cbk = synthkv.small_normal(seed + 1, (Hkv, K, M, dsub))
    cbv = synthkv.small_normal(seed + 2, (Hkv, K, M, dsub))
    ck = synthkv.small_codes(seed + 3, (1, Hkv, t_cap, M), K)
    cv = synthkv.small_codes(seed + 4, (1, Hkv, t_cap, M), K)
    rk = synthkv.small_normal(seed + 5, (1, Hkv, 8, d), np.float16)
    rv = synthkv.small_normal(seed + 6, (1, Hkv, 8, d), np.float16)
    scale = softmax_scale(d)
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, [T], rk, rv, [R], scale)
    pk, pv = oracle.tile_codes(ck, t_cap), oracle.tile_codes(cv, t_cap)
    del ck, cv
    out, lse = run_gpu_decode(dims_for(d, dsub, K, Hq, Hkv), q, cbk, cbv, pk, pv, t_cap, [T], rk, rv, [R], scale,
                              lut=lut)
    err, lerr = check_attention(out, lse, ref_out, ref_lse)
    print(f"[long] T={T}: max row error {err:.2e}, lse error {lerr:.2e}", flush=True)
