"""GPU parity at the full sizes of the five decode workloads, in the launch
configuration the benchmark uses (one pqkv_encode call per tensor over the
whole history or prefill, one pqkv_decode_attention call per layer with the
workload's own batch, lengths and max_hist_len).

Where the oracle cannot afford every output at full size it checks a seeded
sample of them, printed with the result:
  * the batched workload: every sequence of the 16 x 8192 prefill, every 8th
    token from an offset that rotates with the sequence (so every token position
    is checked in two sequences);
  * the 32-layer workload: every layer's 32768-token prefill, encoded in one
    launch, checked on every 8th token from an offset that rotates with the layer
    (every position in four layers); and a seeded eighth of the 1024-token chunks
    of every (layer, sequence) history, all of their tokens checked.
Each encode check reports how many codes fall in the ambiguity band under the
relative reading the comparison uses (D2 - D1 < 1e-5 * max(1, D1)) and under an
absolute 1e-5.  Decode inputs are codes
the oracle itself produced, or seeded random codes where encoding the whole
history on the CPU would take minutes -- attention parity does not depend on
how valid codes were obtained, and encode parity is checked separately.
"""
import functools
import math
import time

import numpy as np
import pytest

import oracle
import synthkv
from pqkv_testlib import check_attention, check_codes, dims_for, run_gpu_decode, softmax_scale, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _log(msg):
    print(f"[workload] {msg}", flush=True)


@functools.lru_cache(maxsize=16)
def _fitted(name, layer, tensor):
    w = synthkv.WORKLOADS[name]
    t0 = time.time()
    cb = oracle.fit_workload_codebooks(w, layer, tensor, synthkv)
    _log(f"{name} layer {layer} {tensor}: codebook fit {time.time() - t0:.1f}s")
    return cb


def _dims(w):
    return dims_for(w.head_dim, w.d_sub, w.n_centroids, w.n_q_heads, w.n_kv_heads)


def _gpu_encode_seq(w, x, cb, t_cap, t_start=0):
    """x [N, H, d] numpy -> code planes [H, t_cap*M] numpy (one launch over all tokens)."""
    import torch

    import decode_attention_pq_amd as P

    planes = torch.zeros((1, w.n_kv_heads, t_cap * w.n_sub), dtype=torch.uint8, device="cuda")
    P.encode(_dims(w), to_dev(x)[None], to_dev(cb), planes, t_cap, t_start)
    torch.cuda.synchronize()
    return planes[0].cpu().numpy()


def _check_sampled_codes(w, x, cb, planes, t_cap, stride, t_start=0, offset=0, positions=None, what=""):
    """Oracle-encode every `stride`-th token of x (from `offset`) and compare with the
    GPU planes; x's token i sits at plane position t_start + i, or positions[i].
    Returns (oracle codes, codes in the relative band, in an absolute 1e-5 band, codes)."""
    idx = np.arange(offset, x.shape[0], stride)
    ref, d1, d2, _ = oracle.encode(x[idx], cb)
    pos = (t_start + idx) if positions is None else np.asarray(positions)[idx]
    off = oracle.code_offsets(w.n_sub, t_cap)[pos]  # [n, M]
    got = planes[:, off].transpose(1, 0, 2)  # [n, H, M]
    n_amb, n_tot = check_codes(got, x[idx], cb, ref, d1, d2)
    n_abs = int(np.sum((d2 - d1) < 1e-5))
    _log(f"{what} encode parity on {len(idx)} tokens (stride {stride}, offset {offset}): {n_amb} of {n_tot} "
         f"codes in the relative band, {n_abs} in an absolute 1e-5 band")
    return ref, n_amb, n_abs, n_tot


def _decode_and_check(w, layer, q, cbk, cbv, codes_k, codes_v, hist, rk, rv, rec):
    scale = softmax_scale(w.head_dim)
    t_cap = codes_k.shape[2]
    t0 = time.time()
    ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, codes_k, codes_v, hist, rk, rv, rec, scale)
    t1 = time.time()
    out, lse = run_gpu_decode(_dims(w), q, cbk, cbv, oracle.tile_codes(codes_k, t_cap),
                              oracle.tile_codes(codes_v, t_cap), t_cap, hist, rk, rv, rec, scale,
                              max_hist=w.max_hist)
    err, lerr = check_attention(out, lse, ref_out, ref_lse)
    _log(f"{w.name} layer {layer}: decode parity max row error {err:.2e}, lse error {lerr:.2e} "
         f"(oracle {t1 - t0:.1f}s)")


def test_llama2_7b_32k_full():
    """32768-token history, 32 heads: every code of K and V and every output row."""
    w = synthkv.WORKLOADS["llama2_7b_32k"]
    codes = {}
    for tensor in ("k", "v"):
        cb = _fitted(w.name, 0, tensor)
        x = synthkv.history_kv(w, 0, tensor, 0)
        planes = _gpu_encode_seq(w, x, cb, w.t_cap)
        codes[tensor] = _check_sampled_codes(w, x, cb, planes, w.t_cap, stride=1, what=tensor)[0]
    ck = codes["k"].transpose(1, 0, 2)[None]
    cv = codes["v"].transpose(1, 0, 2)[None]
    _decode_and_check(w, 0, synthkv.queries(w), _fitted(w.name, 0, "k"), _fitted(w.name, 0, "v"), ck, cv,
                      w.hist_len, synthkv.recent_kv(w, 0, "k"), synthkv.recent_kv(w, 0, "v"), [w.recent_len] * w.batch)


def test_batched_16x8k_full():
    """Batch 16 x 8192: the 16x8192 prefill encoded in one launch, every sequence
    checked on every 8th token (offset rotating with the sequence), and decode of all
    16 sequences in one call."""
    import torch

    import decode_attention_pq_amd as P

    w = synthkv.WORKLOADS["batched_16x8k"]
    T, H, M = w.max_hist, w.n_kv_heads, w.n_sub
    cbk, cbv = _fitted(w.name, 0, "k"), _fitted(w.name, 0, "v")
    for tensor, cb in (("k", cbk), ("v", cbv)):
        x = np.stack([synthkv.history_kv(w, 0, tensor, b) for b in range(w.batch)])  # [B, T, H, d]
        planes = torch.zeros((w.batch, H, w.t_cap * M), dtype=torch.uint8, device="cuda")
        P.encode(_dims(w), to_dev(x), to_dev(cb), planes, w.t_cap)
        torch.cuda.synchronize()
        planes = planes.cpu().numpy()
        tot = np.zeros(3, np.int64)
        for b in range(w.batch):
            _, n_amb, n_abs, n_tot = _check_sampled_codes(w, x[b], cb, planes[b], w.t_cap, stride=8, offset=b % 8,
                                                          what=f"{tensor} seq {b}")
            tot += (n_amb, n_abs, n_tot)
        _log(f"{w.name} {tensor}: {tot[2]} codes checked, {tot[0]} in the relative band, {tot[1]} in an "
             f"absolute 1e-5 band")
        del x
    ck = synthkv.small_codes(31, (w.batch, H, w.t_cap, M), w.n_centroids)
    cv = synthkv.small_codes(32, (w.batch, H, w.t_cap, M), w.n_centroids)
    _decode_and_check(w, 0, synthkv.queries(w), cbk, cbv, ck, cv, w.hist_len, synthkv.recent_kv(w, 0, "k"),
                      synthkv.recent_kv(w, 0, "v"), [w.recent_len] * w.batch)


def test_gqa_llama3_8b_128k_full():
    """131072-token history, 32 query heads over 8 kv heads, d_sub=4: every code and output."""
    w = synthkv.WORKLOADS["gqa_llama3_8b_128k"]
    codes = {}
    for tensor in ("k", "v"):
        cb = _fitted(w.name, 0, tensor)
        x = synthkv.history_kv(w, 0, tensor, 0)
        planes = _gpu_encode_seq(w, x, cb, w.t_cap)
        codes[tensor] = _check_sampled_codes(w, x, cb, planes, w.t_cap, stride=1, what=tensor)[0]
        del x
    _decode_and_check(w, 0, synthkv.queries(w), _fitted(w.name, 0, "k"), _fitted(w.name, 0, "v"),
                      codes["k"].transpose(1, 0, 2)[None], codes["v"].transpose(1, 0, 2)[None], w.hist_len,
                      synthkv.recent_kv(w, 0, "k"), synthkv.recent_kv(w, 0, "v"), [w.recent_len] * w.batch)


def _full32_codebook(w, layer, tensor):
    """Oracle-fitted codebooks for layers 0 and 31, codebooks drawn from the data
    distribution for the others (fitting all 64 tensors on the CPU would take an hour)."""
    if layer in (0, w.n_layers - 1):
        return _fitted(w.name, layer, tensor)
    return synthkv.drawn_codebook(w, layer, tensor)


LAYER_GROUPS = [list(range(g * 8, g * 8 + 8)) for g in range(4)]


@pytest.mark.parametrize("group", range(4))
def test_full32_ragged4_prefill_encode(group):
    """The 32768-token prefill of every layer, encoded in one launch per tensor as the
    benchmark times it; every 8th token checked, from an offset that rotates with the
    layer."""
    w = synthkv.WORKLOADS["full32_ragged4"]
    tot = np.zeros(3, np.int64)
    for layer in LAYER_GROUPS[group]:
        for tensor in ("k", "v"):
            cb = _full32_codebook(w, layer, tensor)
            x = synthkv.kv_values(w, layer, tensor, "prefill", w.prefill_len)
            planes = _gpu_encode_seq(w, x, cb, w.prefill_len)
            _, n_amb, n_abs, n_tot = _check_sampled_codes(w, x, cb, planes, w.prefill_len, stride=8,
                                                          offset=layer % 8, what=f"layer {layer} {tensor} prefill")
            tot += (n_amb, n_abs, n_tot)
            del x
    _log(f"layers {LAYER_GROUPS[group][0]}-{LAYER_GROUPS[group][-1]} prefill: {tot[2]} codes checked, {tot[0]} in "
         f"the relative band, {tot[1]} in an absolute 1e-5 band")


@pytest.mark.parametrize("group", range(4))
def test_full32_ragged4_history_encode(group):
    """Every (layer, sequence) history: a seeded eighth of its 1024-token chunks drawn,
    each encoded into its place in the sequence's cache plane, every token of them
    checked (an eighth of all history tokens)."""
    import torch

    import decode_attention_pq_amd as P

    w = synthkv.WORKLOADS["full32_ragged4"]
    H, M, t_cap = w.n_kv_heads, w.n_sub, w.t_cap
    tot = np.zeros(3, np.int64)
    for layer in LAYER_GROUPS[group]:
        for tensor in ("k", "v"):
            cb = _full32_codebook(w, layer, tensor)
            cbd = to_dev(cb)
            for b in range(w.batch):
                T = w.hist_len[b]
                chunks = synthkv.sample_chunks(10000 * layer + 100 * b + (tensor == "v"), T)
                x = synthkv.history_kv(w, layer, tensor, b, chunks)
                pos = synthkv.chunk_tokens(chunks, T)
                plane = torch.zeros((1, H, t_cap * M), dtype=torch.uint8, device="cuda")
                xd = to_dev(x)
                i = 0
                for c in chunks:
                    n = min(synthkv.CHUNK_TOKENS, T - c * synthkv.CHUNK_TOKENS)
                    P.encode(_dims(w), xd[i:i + n][None], cbd, plane, t_cap, c * synthkv.CHUNK_TOKENS)
                    i += n
                torch.cuda.synchronize()
                _, n_amb, n_abs, n_tot = _check_sampled_codes(
                    w, x, cb, plane[0].cpu().numpy(), t_cap, stride=1, positions=pos,
                    what=f"layer {layer} {tensor} seq {b} chunks {chunks}")
                tot += (n_amb, n_abs, n_tot)
                del x, xd, plane
    _log(f"layers {LAYER_GROUPS[group][0]}-{LAYER_GROUPS[group][-1]} histories: {tot[2]} codes checked, {tot[0]} "
         f"in the relative band, {tot[1]} in an absolute 1e-5 band")


@pytest.mark.parametrize("layer", [0, 31])
def test_full32_ragged4_layer(layer):
    """One layer of the ragged 4-sequence workload at full size with its fitted
    codebooks, decoded with the ragged lengths (its codes' encode parity is covered
    above)."""
    w = synthkv.WORKLOADS["full32_ragged4"]
    H, M, t_cap = w.n_kv_heads, w.n_sub, w.t_cap
    cbs = {t: _fitted(w.name, layer, t) for t in ("k", "v")}
    ck = synthkv.small_codes(100 + layer, (w.batch, H, t_cap, M), w.n_centroids)
    cv = synthkv.small_codes(200 + layer, (w.batch, H, t_cap, M), w.n_centroids)
    _decode_and_check(w, layer, synthkv.queries(w, layer), cbs["k"], cbs["v"], ck, cv, w.hist_len,
                      synthkv.recent_kv(w, layer, "k"), synthkv.recent_kv(w, layer, "v"), [w.recent_len] * w.batch)


def test_full32_ragged4_step_all_layers():
    """The full 32-layer decode step as the benchmark runs it: 32 back-to-back
    pqkv_decode_attention calls on one stream, one per layer (own query, codebooks
    and recent window; one shared set of code planes), each layer's output checked."""
    import torch

    import decode_attention_pq_amd as P

    w = synthkv.WORKLOADS["full32_ragged4"]
    H, M, t_cap, d = w.n_kv_heads, w.n_sub, w.t_cap, w.head_dim
    dims = _dims(w)
    scale = softmax_scale(d)
    ck = synthkv.small_codes(300, (w.batch, H, t_cap, M), w.n_centroids)
    cv = synthkv.small_codes(301, (w.batch, H, t_cap, M), w.n_centroids)
    pk, pv = to_dev(oracle.tile_codes(ck, t_cap)), to_dev(oracle.tile_codes(cv, t_cap))
    hl = torch.tensor(w.hist_len, dtype=torch.int32, device="cuda")
    rl = torch.full((w.batch,), w.recent_len, dtype=torch.int32, device="cuda")
    ws = torch.zeros(P.decode_workspace_bytes(dims, w.batch, w.max_hist), dtype=torch.uint8, device="cuda")
    layers = []
    for layer in range(w.n_layers):
        inp = dict(q=synthkv.queries(w, layer), cbk=synthkv.drawn_codebook(w, layer, "k"),
                   cbv=synthkv.drawn_codebook(w, layer, "v"), rk=synthkv.recent_kv(w, layer, "k"),
                   rv=synthkv.recent_kv(w, layer, "v"))
        dev = {k: to_dev(v) for k, v in inp.items()}
        dev["out"] = torch.full((w.batch, w.n_q_heads, d), float("nan"), device="cuda")
        dev["lse"] = torch.full((w.batch, w.n_q_heads), float("nan"), device="cuda")
        layers.append((inp, dev))
    for inp, dev in layers:  # back to back on one stream, one shared workspace
        P.decode_attention(dims, dev["q"], dev["cbk"], dev["cbv"], pk, pv, t_cap, hl, w.max_hist, dev["rk"],
                           dev["rv"], rl, scale, dev["out"], dev["lse"], ws)
    torch.cuda.synchronize()
    worst = 0.0
    for layer, (inp, dev) in enumerate(layers):
        ref_out, ref_lse = oracle.decode_exact(inp["q"], inp["cbk"], inp["cbv"], ck, cv, w.hist_len, inp["rk"],
                                               inp["rv"], [w.recent_len] * w.batch, scale)
        err, _ = check_attention(dev["out"].cpu().numpy(), dev["lse"].cpu().numpy(), ref_out, ref_lse)
        worst = max(worst, err)
    _log(f"32-layer step: all layers within tolerance, worst row error {worst:.2e}")


def test_workspace_reuse_across_calls():
    """Back-to-back calls with different inputs on one workspace: each result is
    that call's own (the completion counters reset and partials are not stale)."""
    import torch

    import decode_attention_pq_amd as P

    w = synthkv.WORKLOADS["llama2_7b_32k"]
    H, M, d = 8, w.n_sub, w.head_dim
    T, t_cap = 20000, 20032
    dims = dims_for(d, w.d_sub, w.n_centroids, H, H)
    scale = softmax_scale(d)
    ws = torch.zeros(P.decode_workspace_bytes(dims, 1, T), dtype=torch.uint8, device="cuda")
    results = []
    for it in range(3):
        q = synthkv.small_normal(500 + it, (1, H, d), np.float16)
        cbk = synthkv.small_normal(510 + it, (H, w.n_centroids, M, w.d_sub))
        cbv = synthkv.small_normal(520 + it, (H, w.n_centroids, M, w.d_sub))
        ck = synthkv.small_codes(530 + it, (1, H, t_cap, M), w.n_centroids)
        cv = synthkv.small_codes(540 + it, (1, H, t_cap, M), w.n_centroids)
        out = torch.empty((1, H, d), device="cuda")
        lse = torch.empty((1, H), device="cuda")
        P.decode_attention(dims, to_dev(q), to_dev(cbk), to_dev(cbv), to_dev(oracle.tile_codes(ck, t_cap)),
                           to_dev(oracle.tile_codes(cv, t_cap)), t_cap,
                           torch.tensor([T - 1000 * it], dtype=torch.int32, device="cuda"), T, None, None, None,
                           scale, out, lse, ws)
        results.append((q, cbk, cbv, ck, cv, T - 1000 * it, out, lse))
    torch.cuda.synchronize()
    for q, cbk, cbv, ck, cv, t, out, lse in results:
        ref_out, ref_lse = oracle.decode_exact(q, cbk, cbv, ck, cv, [t], np.zeros((1, H, 0, d), np.float16),
                                               np.zeros((1, H, 0, d), np.float16), [0], scale)
        check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse)
