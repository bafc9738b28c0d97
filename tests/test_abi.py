"""The C ABI without a GPU: the library loads, exports what include/pqkv.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def P():
    import decode_attention_pq_amd as P

    P.lib()
    return P


def _declared():
    src = open(os.path.join(ROOT, "include", "pqkv.h")).read()
    return sorted(set(re.findall(r"\b(pqkv_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(P):
    names = _declared()
    assert {"pqkv_encode", "pqkv_build_lut", "pqkv_decode_attention", "pqkv_merge", "pqkv_append_kv",
            "pqkv_fit_codebooks",
            "pqkv_decode_workspace_bytes", "pqkv_status_str"} <= set(names)
    for n in names:
        assert hasattr(P.lib(), n), n


def test_status_strings(P):
    L = P.lib()
    assert L.pqkv_status_str(0) == b"ok"
    assert L.pqkv_status_str(3).startswith(b"workspace")
    assert L.pqkv_status_str(99) == b"unknown status"


def _d(P, *a):
    return ctypes.byref(P.Dims(*a))


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def test_encode_validation(P):
    L = P.lib()
    ok = (128, 2, 256, 32, 32)
    args = lambda dims, n=10, t_cap=64, t_start=0, x=FAKE, dt=0: (
        _d(P, *dims), x, dt, 1, n, 0, 4096, 128, FAKE, FAKE, t_cap, t_start, None)
    assert L.pqkv_encode(*args((96, 2, 256, 32, 32))) == 2      # head_dim unsupported
    assert L.pqkv_encode(*args((128, 3, 256, 32, 32))) == 1     # d_sub does not divide d... 128 % 3 != 0
    assert L.pqkv_encode(*args((128, 8, 256, 32, 32))) == 2     # d_sub 8 unsupported
    assert L.pqkv_encode(*args((128, 2, 257, 32, 32))) == 2     # K > 256
    assert L.pqkv_encode(*args((128, 2, 256, 32, 5))) == 1      # Hq % Hkv
    assert L.pqkv_encode(*args(ok, t_cap=100)) == 1             # t_cap not a multiple of 64
    assert L.pqkv_encode(*args(ok, n=60, t_start=10)) == 1      # past capacity
    assert L.pqkv_encode(*args(ok, x=None)) == 1                # null input
    assert L.pqkv_encode(*args(ok, dt=7)) == 1                  # bad dtype
    assert L.pqkv_encode(*args(ok, n=0, x=None)) == 0           # nothing to do
    assert L.pqkv_encode(*args(ok, x=ctypes.c_void_p(0x10002))) == 1  # misaligned rows
    assert L.pqkv_encode(None, FAKE, 0, 1, 10, 0, 4096, 128, FAKE, FAKE, 64, 0, None) == 1


def test_decode_validation(P):
    L = P.lib()
    dims = (128, 2, 256, 32, 32)
    ws_need = L.pqkv_decode_workspace_bytes(_d(P, *dims), 1, 32768)
    assert ws_need > 0

    def call(dims=dims, batch=1, t_cap=32768, maxh=32768, r_cap=128, ws=FAKE, wsb=None, codes=FAKE, qdt=0,
             scale=0.088, q=FAKE, lut=None, cbk=FAKE, cbv=FAKE, hist=FAKE, rk=FAKE):
        return L.pqkv_decode_attention(
            _d(P, *dims), batch, q, qdt, lut, cbk, cbv, codes, codes, t_cap, hist, maxh, rk, FAKE, 0, r_cap,
            FAKE, scale, FAKE, FAKE, ws, ws_need if wsb is None else wsb, None)

    assert call(ws=None) == 3
    assert call(wsb=ws_need - 1) == 3
    assert call(ws=ctypes.c_void_p(0x10010)) == 3        # workspace not 256-byte aligned
    assert call(maxh=40000) == 1                          # longer than the capacity
    assert call(t_cap=1000, maxh=900) == 1                # capacity not a multiple of 64
    assert call(r_cap=2000) == 2                          # recent window too large
    assert call(codes=ctypes.c_void_p(0x10004)) == 1      # misaligned code planes
    assert call(qdt=5) == 1
    assert call(batch=-1) == 1
    assert call(batch=0) == 0
    assert call(scale=float("nan")) == 1
    assert call(dims=(128, 2, 1, 32, 32)) == 2            # K < 2
    assert call(dims=(128, 2, 256, 0, 32)) == 1
    assert call(hist=None) == 1                           # lengths needed when there is a history
    assert call(q=ctypes.c_void_p(0x10008)) == 1          # q not 16-byte aligned
    assert call(cbv=ctypes.c_void_p(0x10008)) == 1        # value codebook not 16-byte aligned
    assert call(rk=ctypes.c_void_p(0x10004)) == 1         # recent rows not 16-byte aligned
    assert call(cbk=None) == 1                            # no key codebook and no table
    assert call(cbk=None, lut=FAKE, wsb=ws_need - 1) == 3  # the table stands in for the key codebook
    assert call(lut=ctypes.c_void_p(0x10004)) == 1        # table not 16-byte aligned
    assert call(dims=(128, 2, 250, 32, 32), lut=FAKE) == 2  # the table is read 4 centroids at a time


def test_workspace_formula(P):
    L = P.lib()
    # one u32 completion counter per (sequence, query head) padded to 256 bytes, then
    # the partials (132 floats per query head and split), padded
    # LLaMA-2-7B shape at 32K context: 32 kv heads, one query head each, 8 splits of 4096 tokens
    assert L.pqkv_decode_workspace_bytes(_d(P, 128, 2, 256, 32, 32), 1, 32768) == 32 * 8 * 132 * 4 + 256
    # no history: one split per unit for the recent window
    assert L.pqkv_decode_workspace_bytes(_d(P, 128, 2, 256, 32, 32), 1, 0) == 32 * 1 * 132 * 4 + 256
    assert L.pqkv_decode_workspace_bytes(_d(P, 96, 2, 256, 32, 32), 1, 100) == 0
    assert L.pqkv_decode_workspace_bytes(_d(P, 128, 2, 256, 32, 32), 0, 100) == 0
    # GQA 32/8 at d_sub=4: two query heads per work-group, 16 splits of 8192 tokens
    assert L.pqkv_decode_workspace_bytes(_d(P, 128, 4, 256, 32, 8), 1, 131072) == 32 * 16 * 132 * 4 + 256


def test_split_plan_choices(P):
    """The split plan, read back through the workspace size (one u32 counter per
    sequence and query head, padded to 256 bytes, then the partials of 132 floats per
    query head and split, padded)."""
    L = P.lib()
    ws = lambda dims, batch, maxh: L.pqkv_decode_workspace_bytes(_d(P, *dims), batch, maxh)
    pad = lambda n: -(-n // 256) * 256
    full = (128, 2, 256, 32, 32)
    # batch 16 x 8192: one 16-round split per (sequence, head), 512 work-groups
    assert ws(full, 16, 8192) == pad(16 * 32 * 1 * 528) + pad(16 * 32 * 4)
    # four ragged sequences bounded by 31436 tokens: 4 splits of 8192 per sequence
    assert ws(full, 4, 31436) == pad(4 * 32 * 4 * 528) + pad(4 * 32 * 4)
    # batch 16 x 5021: one 10-round split each (12-round build), not two of 5 rounds
    assert ws(full, 16, 5021) == pad(16 * 32 * 1 * 528) + pad(16 * 32 * 4)
    # batch 4 x 20083: 4 splits of 10 rounds (512 work-groups), not 3 of 14 (384)
    assert ws(full, 4, 20083) == pad(4 * 32 * 4 * 528) + pad(4 * 32 * 4)
    # one head of 300000 tokens: 196 splits of 3 rounds, within the merge's 512-split limit
    assert ws((128, 2, 256, 1, 1), 1, 300000) == pad(196 * 528) + 256
    # 5,000,000 tokens need more than 512 splits even at 16 rounds: refused
    need = ws((128, 2, 256, 1, 1), 1, 5000000)
    assert need == pad(611 * 528) + 256
    assert L.pqkv_decode_attention(_d(P, 128, 2, 256, 1, 1), 1, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, 5000000, FAKE,
                                   5000000, FAKE, FAKE, 0, 0, FAKE, 0.088, FAKE, FAKE, FAKE, need, None) == 2
    # the limit itself: 512 splits of 16 rounds (8192 tokens) with one or two query heads
    # per work-group, of 8 rounds with four; one token more is refused
    for dims, limit in (((128, 2, 256, 1, 1), 512 * 8192), ((64, 4, 256, 4, 1), 512 * 4096)):
        assert ws(dims, 1, limit) == pad(512 * (dims[0] + 4) * 4 * dims[3]) + 256
        for maxh, status in ((limit + 1, 2), (limit + 64, 2)):
            w_need = ws(dims, 1, maxh)
            assert L.pqkv_decode_attention(_d(P, *dims), 1, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, limit + 64, FAKE,
                                           maxh, FAKE, FAKE, 0, 0, FAKE, 0.088, FAKE, FAKE, FAKE, w_need,
                                           None) == status


def test_decode_plan_presets(P):
    """pqkv_decode_plan: the preset a call runs, per context length (splits, split length,
    kernel build, query heads per work-group), consistent with the workspace size and with
    itself; the table over context lengths is printed."""
    L = P.lib()
    shapes = {"MHA d_sub 2 (32 heads x 128)": P.Dims(128, 2, 256, 32, 32),
              "GQA d_sub 4 (32 over 8 heads)": P.Dims(128, 4, 256, 32, 8),
              "GQA d_sub 4, head_dim 64 (16 over 4)": P.Dims(64, 4, 256, 16, 4)}
    for name, dims in shapes.items():
        M = dims.head_dim // dims.d_sub
        g = dims.n_q_heads // dims.n_kv_heads
        print(f"{name}: context -> splits x tokens, rounds / build, q heads per group, work-groups")
        for batch in (1, 4, 16):
            for T in (0, 64, 512, 4096, 8192, 32768, 131072, 1 << 20):
                p = P.decode_plan(dims, batch, T)
                if batch == 1:
                    print(f"  batch {batch} T {T:8d}: {p['splits']:4d} x {p['split_tokens']:5d}, "
                          f"{p['rounds']:2d} / {p['build_rounds']:2d}, {p['q_heads_per_group']}, {p['work_groups']}")
                assert p["workspace_bytes"] == L.pqkv_decode_workspace_bytes(ctypes.byref(dims), batch, T)
                qh = p["q_heads_per_group"]
                assert qh in (1, 2, 4) and g % qh == 0 and qh * M <= 64
                assert p["work_groups"] == batch * dims.n_kv_heads * (g // qh) * p["splits"]
                assert p["device_plan"] == (1 if 2 <= batch <= 16 and T > 0 else 0)
                if T == 0:
                    assert p["splits"] == 1 and p["split_tokens"] == 0 and p["rounds"] == 0
                    continue
                assert p["split_tokens"] == 512 * p["rounds"]
                # the splits cover the history, none of them empty
                assert p["splits"] * p["split_tokens"] >= T > (p["splits"] - 1) * p["split_tokens"]
                assert p["rounds"] <= p["build_rounds"] <= (8 if qh == 4 else 16)
                assert p["build_rounds"] in ((2, 4, 8, 12, 16) if M == 64 else (4, 8, 16))
    # the presets the workloads run
    mha, gqa = shapes["MHA d_sub 2 (32 heads x 128)"], shapes["GQA d_sub 4 (32 over 8 heads)"]
    assert {k: P.decode_plan(mha, 1, 32768)[k] for k in ("splits", "split_tokens", "work_groups")} == \
        {"splits": 8, "split_tokens": 4096, "work_groups": 256}
    assert {k: P.decode_plan(gqa, 1, 131072)[k] for k in ("q_heads_per_group", "splits", "split_tokens")} == \
        {"q_heads_per_group": 2, "splits": 16, "split_tokens": 8192}
    assert P.decode_plan(mha, 16, 8192)["splits"] == 1
    # errors
    info = P.DecodePlanInfo()
    assert L.pqkv_decode_plan(ctypes.byref(mha), 1, 100, None) == 1
    assert L.pqkv_decode_plan(ctypes.byref(mha), 0, 100, ctypes.byref(info)) == 1
    assert L.pqkv_decode_plan(ctypes.byref(mha), 1, -1, ctypes.byref(info)) == 1
    assert L.pqkv_decode_plan(_d(P, 96, 2, 256, 32, 32), 1, 100, ctypes.byref(info)) == 2
    assert L.pqkv_decode_plan(_d(P, 128, 2, 256, 1, 1), 1, 5000000, ctypes.byref(info)) == 2  # > 512 splits


def test_noalloc_refuses_sizes_beyond_its_array(P):
    """pqkv_decode_attention_noalloc checks on the host that the call fits its static
    array (rows of counters, then partials) before it touches a device."""
    L = P.lib()

    def call(batch, hq, maxh, t_cap):
        return L.pqkv_decode_attention_noalloc(_d(P, 128, 2, 256, hq, hq), batch, FAKE, 0, None, FAKE, FAKE, FAKE,
                                               FAKE, t_cap, FAKE, maxh, None, None, 0, 0, None, 0.088, FAKE, FAKE,
                                               None)

    assert P.NOALLOC_MAX_ROWS == 16384 and P.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert call(600, 32, 64, 64) == 3              # 19200 (sequence, query head) rows
    assert call(128, 32, 32768, 32768) == 3        # 4 splits each: 8.65 MB of partials
    assert call(1, 32, 40000, 32768) == 1          # ordinary validation comes first
    assert call(0, 32, 64, 64) == 0                # nothing to do


def test_merge_validation(P):
    L = P.lib()
    assert L.pqkv_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.pqkv_merge(4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.pqkv_merge(4, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.pqkv_merge(0, 128, None, None, None, None, None, None, None) == 0
    assert L.pqkv_merge(4, 128, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1


def test_append_validation(P):
    L = P.lib()
    F2, F3, F4, F5 = (ctypes.c_void_p(0x20000 + 0x1000 * i) for i in range(4))  # distinct length arrays

    def call(dims=(128, 2, 256, 32, 32), batch=2, r_cap=128, n_roll=64, t_cap=4096, max_hist=1000,
             hin=F2, rin=F3, hout=F4, rout=F5, dt=0, new_k=FAKE, rk=FAKE, cb=FAKE):
        return L.pqkv_append_kv(_d(P, *dims), batch, new_k, FAKE, rk, FAKE, dt, r_cap, hin, rin, hout, rout,
                                n_roll, cb, FAKE, FAKE, FAKE, t_cap, max_hist, None)

    assert call(batch=0, new_k=None) == 0                  # nothing to do
    assert call(dims=(96, 2, 256, 32, 32)) == 2            # head_dim unsupported
    assert call(n_roll=0) == 1 and call(n_roll=129) == 1   # n_roll outside 1..r_cap
    assert call(r_cap=2048, n_roll=600) == 2               # window and roll beyond the supported sizes
    assert call(r_cap=0) == 1
    assert call(t_cap=100) == 1                            # not a multiple of 64
    assert call(max_hist=4090) == 1                        # a roll could pass the capacity
    assert call(dt=5) == 1
    assert call(new_k=None) == 1
    assert call(rk=ctypes.c_void_p(0x10008)) == 1          # rows not 16-byte aligned
    assert call(hout=F2) == 1 and call(rout=F3) == 1       # out lengths alias the in lengths
    assert call(hout=ctypes.c_void_p(0x20004)) == 1        # out overlaps in by one element
    assert call(rout=F4) == 1                              # the two out arrays overlap


def test_fit_codebooks_validation(P):
    L = P.lib()

    def call(dims=(128, 2, 256, 32, 32), n=4096, iters=10, x=FAKE, order=FAKE, cb=FAKE, dt=0, ts=4096, hs=128):
        return L.pqkv_fit_codebooks(_d(P, *dims), x, dt, n, ts, hs, order, iters, cb, None, None)

    assert call(dims=(96, 2, 256, 32, 32)) == 2
    assert call(n=0) == 1 and call(iters=-1) == 1 and call(ts=-1) == 1 and call(dt=9) == 1
    assert call(n=8193) == 2                       # more points than one work-group stages
    assert call(x=None) == 1 and call(order=None) == 1 and call(cb=None) == 1


def test_plain_c_program_against_the_abi(P, tmp_path):
    """tests/abi_check.c includes only include/pqkv.h, links libpqkv.so with gcc as
    C11 and checks the host-side contract without a GPU."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    libdir = os.path.dirname(P.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "abi_check.c"), "-L", libdir, "-lpqkv",
                    f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "decode_attention_pq_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", src), f"{f} mentions the oracle"
