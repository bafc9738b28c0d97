"""Python binding of libpqkv: product-quantised KV cache (MILLION) on MI355X.

Thin ctypes marshalling over the C interface declared in ``include/pqkv.h``:
every call checks tensor shapes, dtypes and devices, passes raw device
pointers and torch's current HIP stream, and turns a non-zero status into a
``PQKVError``.  All computation runs in the HIP kernels of ``libpqkv.so``;
there is no fallback path.  PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime libpqkv.so binds to (same soname)

__all__ = [
    "PQKVError", "Dims", "lib", "LIB_PATH", "encode", "build_lut", "decode_workspace_bytes", "decode_plan", "DecodePlanInfo",
    "decode_attention", "fp16_decode_workspace_bytes", "fp16_decode_attention", "append_kv", "NOALLOC_SCRATCH_BYTES", "NOALLOC_MAX_ROWS", "fit_codebooks", "merge", "code_plane_bytes", "MAX_FIT_POINTS", "F16", "F32", "MAX_RECENT", "TILE_TOKENS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpqkv.so")
F16, F32 = 0, 1
MAX_RECENT = 1024
MAX_FIT_POINTS = 8192
TILE_TOKENS = 64
NOALLOC_SCRATCH_BYTES = 8 << 20
NOALLOC_MAX_ROWS = 16384

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace missing or too small",
           4: "HIP launch failed"}


class PQKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("d_sub", ctypes.c_int32), ("n_centroids", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32)]

    @property
    def n_sub(self) -> int:
        return self.head_dim // self.d_sub

    def __repr__(self):
        return (f"Dims(head_dim={self.head_dim}, d_sub={self.d_sub}, n_centroids={self.n_centroids}, "
                f"n_q_heads={self.n_q_heads}, n_kv_heads={self.n_kv_heads})")


class DecodePlanInfo(ctypes.Structure):
    """pqkv_decode_plan_info: the preset a decode call of given sizes runs."""
    _fields_ = [("q_heads_per_group", ctypes.c_int32), ("splits", ctypes.c_int32), ("split_tokens", ctypes.c_int64),
                ("rounds", ctypes.c_int32), ("build_rounds", ctypes.c_int32), ("work_groups", ctypes.c_int64),
                ("device_plan", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libpqkv.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libpqkv.so not built at {LIB_PATH}; run decode_attention_pq_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        dp = ctypes.POINTER(Dims)
        L.pqkv_encode.argtypes = [dp, vp, i32, i32, i64, i64, i64, i64, vp, vp, i64, i64, vp]
        L.pqkv_encode.restype = i32
        L.pqkv_build_lut.argtypes = [dp, i32, vp, i32, vp, vp, vp]
        L.pqkv_build_lut.restype = i32
        L.pqkv_decode_workspace_bytes.argtypes = [dp, i32, i64]
        L.pqkv_decode_workspace_bytes.restype = sz
        L.pqkv_decode_plan.argtypes = [dp, i32, i64, ctypes.POINTER(DecodePlanInfo)]
        L.pqkv_decode_plan.restype = i32
        L.pqkv_decode_attention.argtypes = [dp, i32, vp, i32, vp, vp, vp, vp, vp, i64, vp, i64, vp, vp, i32,
                                            i64, vp, f32, vp, vp, vp, sz, vp]
        L.pqkv_decode_attention.restype = i32
        L.pqkv_decode_attention_noalloc.argtypes = [dp, i32, vp, i32, vp, vp, vp, vp, vp, i64, vp, i64, vp, vp,
                                                    i32, i64, vp, f32, vp, vp, vp]
        L.pqkv_decode_attention_noalloc.restype = i32
        L.pqkv_fp16_decode_workspace_bytes.argtypes = [dp, i32, i64]
        L.pqkv_fp16_decode_workspace_bytes.restype = sz
        L.pqkv_fp16_decode_attention.argtypes = [dp, i32, vp, vp, vp, i64, vp, i64, f32, vp, vp, vp, sz, vp]
        L.pqkv_fp16_decode_attention.restype = i32
        L.pqkv_append_kv.argtypes = [dp, i32, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                     i64, i64, vp]
        L.pqkv_append_kv.restype = i32
        L.pqkv_fit_codebooks.argtypes = [dp, vp, i32, i64, i64, i64, vp, i32, vp, vp, vp]
        L.pqkv_fit_codebooks.restype = i32
        L.pqkv_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp]
        L.pqkv_merge.restype = i32
        L.pqkv_status_str.argtypes = [i32]
        L.pqkv_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PQKVError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"expected float16 or float32, got {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libpqkv takes device tensors")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def code_plane_bytes(dims: Dims, t_cap: int) -> int:
    return t_cap * dims.n_sub


def encode(dims: Dims, x: torch.Tensor, codebook: torch.Tensor, codes: torch.Tensor, t_cap: int,
           t_start: int = 0) -> None:
    """pqkv_encode.  x: [n_seqs, n_tokens, Hkv, d] or [n_tokens, Hkv, d] (last dim contiguous);
    codebook: fp32 [Hkv, K, M, d_sub]; codes: uint8 [n_seqs, Hkv, t_cap*M] (or [Hkv, t_cap*M])."""
    _dev(x, codebook, codes)
    if x.dim() == 3:
        x = x.unsqueeze(0)
    n_seqs, n_tok, H, d = x.shape
    if x.stride(3) != 1:
        raise ValueError("x rows must be contiguous")
    if codebook.dtype != torch.float32 or not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous fp32")
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous uint8")
    if codes.numel() < n_seqs * dims.n_kv_heads * t_cap * dims.n_sub:
        raise ValueError("codes buffer too small")
    _check("pqkv_encode", lib().pqkv_encode(
        ctypes.byref(dims), _ptr(x), _dtype_code(x), n_seqs, n_tok, x.stride(0), x.stride(1), x.stride(2),
        _ptr(codebook), _ptr(codes), t_cap, t_start, _stream()))


def build_lut(dims: Dims, q: torch.Tensor, codebook_k: torch.Tensor, lut: torch.Tensor) -> None:
    """pqkv_build_lut.  q: [B, Hq, d] contiguous; lut: fp32 [B, Hq, M, K]."""
    _dev(q, codebook_k, lut)
    if not q.is_contiguous() or not lut.is_contiguous() or lut.dtype != torch.float32:
        raise ValueError("q and lut must be contiguous; lut fp32")
    B = q.shape[0]
    if lut.numel() < B * dims.n_q_heads * dims.n_sub * dims.n_centroids:
        raise ValueError("lut buffer too small")
    _check("pqkv_build_lut", lib().pqkv_build_lut(ctypes.byref(dims), B, _ptr(q), _dtype_code(q),
                                                  _ptr(codebook_k), _ptr(lut), _stream()))


def decode_workspace_bytes(dims: Dims, batch: int, max_hist_len: int) -> int:
    return int(lib().pqkv_decode_workspace_bytes(ctypes.byref(dims), batch, max_hist_len))


def decode_plan(dims: Dims, batch: int, max_hist_len: int) -> dict:
    """The preset pqkv_decode_attention runs for these sizes (pqkv_decode_plan), as a dict."""
    info = DecodePlanInfo()
    _check("pqkv_decode_plan", lib().pqkv_decode_plan(ctypes.byref(dims), batch, max_hist_len, ctypes.byref(info)))
    return {name: int(getattr(info, name)) for name, _ in DecodePlanInfo._fields_}


def _check_numel(name, t, n):
    if t.numel() < n:
        raise ValueError(f"{name} has {t.numel()} elements, needs {n}")


def decode_attention(dims: Dims, q, codebook_k, codebook_v, codes_k, codes_v, t_cap: int, hist_len,
                     max_hist_len: int, recent_k, recent_v, recent_len, softmax_scale: float, out, lse,
                     workspace, lut=None, noalloc=False) -> None:
    """pqkv_decode_attention.  q: [B, Hq, d]; codes_k/v: uint8 [B, Hkv, t_cap*M];
    hist_len/recent_len: int32 [B] (device); recent_k/v: [B, Hkv, r_cap, d] or None;
    out: fp32 [B, Hq, d]; lse: fp32 [B, Hq]; workspace: a device tensor (uint8) or None;
    lut: None (the kernel builds the ad-LUT) or fp32 [B, Hq, M, K] from build_lut
    (codebook_k may then be None).  noalloc=True calls pqkv_decode_attention_noalloc
    (the library's static device array instead of `workspace`, which must be None)."""
    _dev(q, lut, codebook_k, codebook_v, codes_k, codes_v, hist_len, recent_k, recent_v, recent_len, out, lse,
         workspace)
    B = q.shape[0]
    d, M, K, Hq, Hkv = dims.head_dim, dims.n_sub, dims.n_centroids, dims.n_q_heads, dims.n_kv_heads
    for t in (q, lut, codebook_k, codebook_v, codes_k, codes_v, out, lse, hist_len):
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if hist_len is not None and hist_len.dtype != torch.int32:
        raise ValueError("hist_len must be int32")
    _check_numel("q", q, B * Hq * d)
    _check_numel("out", out, B * Hq * d)
    _check_numel("lse", lse, B * Hq)
    if out.dtype != torch.float32 or lse.dtype != torch.float32:
        raise ValueError("out and lse must be fp32")
    if max_hist_len > 0:
        if hist_len is None or codes_k is None or codes_v is None or codebook_v is None:
            raise ValueError("a history needs hist_len, codes_k/v and codebook_v")
        _check_numel("hist_len", hist_len, B)
        _check_numel("codes_k", codes_k, B * Hkv * t_cap * M)
        _check_numel("codes_v", codes_v, B * Hkv * t_cap * M)
        for name, cb in (("codebook_k", codebook_k), ("codebook_v", codebook_v)):
            if cb is None:
                continue
            if cb.dtype != torch.float32:
                raise ValueError(f"{name} must be fp32")
            _check_numel(name, cb, Hkv * K * d)
        if lut is not None:
            if lut.dtype != torch.float32:
                raise ValueError("lut must be fp32")
            _check_numel("lut", lut, B * Hq * M * K)
    r_cap = 0 if recent_k is None else recent_k.shape[2]
    rdt = F16 if recent_k is None else _dtype_code(recent_k)
    if recent_k is not None:
        if not (recent_k.is_contiguous() and recent_v.is_contiguous()) or recent_len.dtype != torch.int32:
            raise ValueError("recent_k/v must be contiguous and recent_len int32")
        if recent_k.shape != recent_v.shape or recent_k.dtype != recent_v.dtype:
            raise ValueError("recent_k and recent_v differ")
        if tuple(recent_k.shape) != (B, Hkv, r_cap, d):
            raise ValueError(f"recent_k has shape {tuple(recent_k.shape)}, expected ({B}, {Hkv}, r_cap, {d})")
        _check_numel("recent_len", recent_len, B)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        _check("pqkv_decode_attention_noalloc", lib().pqkv_decode_attention_noalloc(
            ctypes.byref(dims), B, _ptr(q), _dtype_code(q), _ptr(lut), _ptr(codebook_k), _ptr(codebook_v),
            _ptr(codes_k), _ptr(codes_v), t_cap, _ptr(hist_len), max_hist_len, _ptr(recent_k), _ptr(recent_v),
            rdt, r_cap, _ptr(recent_len), float(softmax_scale), _ptr(out), _ptr(lse), _stream()))
        return
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pqkv_decode_attention", lib().pqkv_decode_attention(
        ctypes.byref(dims), B, _ptr(q), _dtype_code(q), _ptr(lut), _ptr(codebook_k), _ptr(codebook_v),
        _ptr(codes_k), _ptr(codes_v), t_cap, _ptr(hist_len), max_hist_len, _ptr(recent_k), _ptr(recent_v), rdt,
        r_cap, _ptr(recent_len), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream()))


def fp16_decode_workspace_bytes(dims: Dims, batch: int, max_len: int) -> int:
    return int(lib().pqkv_fp16_decode_workspace_bytes(ctypes.byref(dims), batch, max_len))


def fp16_decode_attention(dims: Dims, q, k_cache, v_cache, t_cap: int, seq_len, max_len: int, softmax_scale: float,
                          out, lse, workspace) -> None:
    """pqkv_fp16_decode_attention (the dense fp16 baseline).  q: fp16 [B, Hq, d];
    k_cache/v_cache: fp16 [B, Hkv, t_cap, d]; seq_len: int32 [B] (device);
    out: fp32 [B, Hq, d]; lse: fp32 [B, Hq]; workspace: a device tensor (uint8)."""
    _dev(q, k_cache, v_cache, seq_len, out, lse, workspace)
    B = q.shape[0]
    d, Hq, Hkv = dims.head_dim, dims.n_q_heads, dims.n_kv_heads
    for t in (q, k_cache, v_cache, seq_len, out, lse):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if q.dtype != torch.float16 or k_cache.dtype != torch.float16 or v_cache.dtype != torch.float16:
        raise ValueError("q and the caches must be fp16")
    if seq_len.dtype != torch.int32 or out.dtype != torch.float32 or lse.dtype != torch.float32:
        raise ValueError("seq_len must be int32, out and lse fp32")
    _check_numel("q", q, B * Hq * d)
    _check_numel("k_cache", k_cache, B * Hkv * t_cap * d)
    _check_numel("v_cache", v_cache, B * Hkv * t_cap * d)
    _check_numel("seq_len", seq_len, B)
    _check_numel("out", out, B * Hq * d)
    _check_numel("lse", lse, B * Hq)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pqkv_fp16_decode_attention", lib().pqkv_fp16_decode_attention(
        ctypes.byref(dims), B, _ptr(q), _ptr(k_cache), _ptr(v_cache), t_cap, _ptr(seq_len), max_len,
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream()))


def append_kv(dims: Dims, new_k, new_v, recent_k, recent_v, hist_len_in, recent_len_in, hist_len_out,
              recent_len_out, n_roll: int, codebook_k, codebook_v, codes_k, codes_v, t_cap: int,
              max_hist_len: int) -> None:
    """pqkv_append_kv.  new_k/v: [B, Hkv, d]; recent_k/v: [B, Hkv, r_cap, d] (same dtype, updated in
    place); *_len_in / *_len_out: int32 [B] (device, out distinct from in); codes_k/v: uint8
    [B, Hkv, t_cap*M] (updated in place)."""
    _dev(new_k, new_v, recent_k, recent_v, hist_len_in, recent_len_in, hist_len_out, recent_len_out,
         codebook_k, codebook_v, codes_k, codes_v)
    B = new_k.shape[0]
    for t in (new_k, new_v, recent_k, recent_v, codebook_k, codebook_v, codes_k, codes_v):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    for t in (hist_len_in, recent_len_in, hist_len_out, recent_len_out):
        if t.dtype != torch.int32:
            raise ValueError("lengths must be int32")
    if not (new_k.dtype == new_v.dtype == recent_k.dtype == recent_v.dtype):
        raise ValueError("new and recent rows must share one dtype")
    _check("pqkv_append_kv", lib().pqkv_append_kv(
        ctypes.byref(dims), B, _ptr(new_k), _ptr(new_v), _ptr(recent_k), _ptr(recent_v), _dtype_code(recent_k),
        recent_k.shape[2], _ptr(hist_len_in), _ptr(recent_len_in), _ptr(hist_len_out), _ptr(recent_len_out),
        n_roll, _ptr(codebook_k), _ptr(codebook_v), _ptr(codes_k), _ptr(codes_v), t_cap, max_hist_len,
        _stream()))


def fit_codebooks(dims: Dims, x, order, iters: int, codebook, kept=None) -> None:
    """pqkv_fit_codebooks.  x: [N, Hkv, d] (rows contiguous); order: int32 [Hkv, M, N];
    codebook: fp32 out [Hkv, K, M, d_sub]; kept: int32 out [Hkv, M] or None."""
    _dev(x, order, codebook, kept)
    if x.stride(2) != 1:
        raise ValueError("x rows must be contiguous")
    if order.dtype != torch.int32 or not order.is_contiguous():
        raise ValueError("order must be contiguous int32")
    if codebook.dtype != torch.float32 or not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous fp32")
    if kept is not None and (kept.dtype != torch.int32 or not kept.is_contiguous()):
        raise ValueError("kept must be contiguous int32")
    n = x.shape[0]
    if order.numel() < dims.n_kv_heads * dims.n_sub * n:
        raise ValueError("order too small")
    _check("pqkv_fit_codebooks", lib().pqkv_fit_codebooks(
        ctypes.byref(dims), _ptr(x), _dtype_code(x), n, x.stride(0), x.stride(1), _ptr(order), iters,
        _ptr(codebook), _ptr(kept), _stream()))


def merge(out_a, lse_a, out_b, lse_b, out, lse) -> None:
    """pqkv_merge over rows: out_*: fp32 [n, d]; lse_*: fp32 [n]."""
    _dev(out_a, lse_a, out_b, lse_b, out, lse)
    n, d = out_a.shape[0], out_a.shape[-1]
    for t in (out_a, lse_a, out_b, lse_b, out, lse):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("merge takes contiguous fp32 tensors")
    _check("pqkv_merge", lib().pqkv_merge(n, d, _ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out),
                                          _ptr(lse), _stream()))
